// Online acceptance estimator for gfx950: the refit step.  (The scoring
// pass - feature, score, survival prune - runs on the verification's
// statistics kernel, in stream.hip.)
//
// Method: [AV] "Adaptive Verification ohne Confidence Head" (spke.com; Arabic
// mirror "التحقق التكيفي بدون رأس ثقة"):
//   "Solution" / "Scoring the distribution": score_i = sigmoid(omega * x +
//   beta_i) with x = logit(q_max) of the draft distribution, one shared slope
//   and one intercept per draft position;
//   "Other features considered": survival = running product of the scores;
//   "Fitting the coefficients": IRLS on the accept/reject labels up to the
//   first rejection, H and g accumulated over a round and the Newton system
//   solved on its last step, each step damped by n / (n + constant).
#include "sv_device.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// refit step: one workgroup of 256 threads.  Thread t takes requests
// b = t, t + 256, ..., loading all of a request's labels and features at
// once; per position the six sums are formed in fp64, reduced per wave
// (butterfly) into LDS and then over the waves in order, a fixed order that
// makes the result deterministic.  On the round's last step thread 0 solves the arrowhead
// Newton system H * delta = -g by eliminating the intercepts (Schur
// complement on the slope), damps, bounds the step, updates the parameters
// and clears the accumulator.
// ---------------------------------------------------------------------------

constexpr int kFitT = 256;  // threads of the refit (1024 measured slower: binary64-bound)
constexpr int kFitW = kFitT / 64;

__device__ __forceinline__ double sigmoid_d(double t) {
  if (t >= 0.0) return 1.0 / (1.0 + exp(-t));
  const double e = exp(t);
  return e / (1.0 + e);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(kFitT) void av_fit_kernel(int B, int max_k, const float* feature,
                                                       const int8_t* labels, float* params, double* accum,
                                                       float damping_c, float ridge, float max_step, int do_update) {
  __shared__ double red[kFitW][SV_MAX_K][6];  // per wave and position, summed over the chunks in order
  __shared__ double acc[SV_MAX_K][6];          // accumulator after this step
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // parameters and the incoming accumulator with the first chunk's items:
  // one round trip to memory instead of one per position
  const double omega = params[0];
  double beta[SV_MAX_K];
#pragma unroll
  for (int i = 0; i < SV_MAX_K; ++i) beta[i] = i < max_k ? double(params[1 + i]) : 0.0;
  const double acc_in = tid < 6 * max_k ? accum[tid] : 0.0;
  for (int e = tid; e < kFitW * SV_MAX_K * 6; e += kFitT) (&red[0][0][0])[e] = 0.0;
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += kFitT) {
    const int b = b0 + tid;
    int y[SV_MAX_K];
    float x[SV_MAX_K];
#pragma unroll
    for (int i = 0; i < SV_MAX_K; ++i) {
      const bool in = b < B && i < max_k;
      y[i] = in ? labels[size_t(b) * max_k + i] : -1;
      x[i] = in ? feature[size_t(b) * max_k + i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < SV_MAX_K; ++i) {
      if (i >= max_k) continue;  // uniform
      double v[6] = {0, 0, 0, 0, 0, 0};
      if (y[i] == 0 || y[i] == 1) {
        const double xd = x[i];
        const double pi = sigmoid_d(omega * xd + beta[i]);
        const double w = pi * (1.0 - pi);
        const double r = pi - double(y[i]);
        v[0] = 1.0;
        v[1] = w;
        v[2] = w * xd;
        v[3] = w * xd * xd;
        v[4] = r;
        v[5] = r * xd;
      }
#pragma unroll
      for (int k = 0; k < 6; ++k) v[k] = wave_sum_d(v[k]);
      if (lane == 0)
#pragma unroll
        for (int k = 0; k < 6; ++k) red[wave][i][k] += v[k];
    }
  }
  __syncthreads();
  if (tid < 6 * max_k) {
    const int i = tid / 6, k = tid % 6;
    double t = red[0][i][k];
    for (int w = 1; w < kFitW; ++w) t += red[w][i][k];
    t += acc_in;
    acc[i][k] = t;
    if (!do_update) accum[tid] = t;
  }
  __syncthreads();
  if (!do_update) return;
  if (tid == 0) {
    double N = 0.0, h = ridge, gw = 0.0;
    for (int i = 0; i < max_k; ++i) {
      N += acc[i][0];
      h += acc[i][3];
      gw += acc[i][5];
    }
    if (N > 0.0) {
      // eliminate the intercepts of positions with labels
      double schur = h, rhs = -gw;
      for (int i = 0; i < max_k; ++i) {
        const double n = acc[i][0];
        if (n <= 0.0) continue;
        const double D = acc[i][1] + ridge, Bi = acc[i][2], gb = acc[i][4];
        schur -= Bi * Bi / D;
        rhs += Bi * gb / D;
      }
      const double dw = (schur > 0.0) ? rhs / schur : 0.0;
      // damped steps, then the whole step scaled so that no parameter moves
      // by more than max_step (far from the optimum, or for a position whose
      // labels all agree, the Newton step on the logistic loss overshoots)
      double step[SV_MAX_K + 1];
      step[0] = dw * (N / (N + double(damping_c)));
      double largest = fabs(step[0]);
      for (int i = 0; i < max_k; ++i) {
        const double n = acc[i][0];
        step[1 + i] = 0.0;
        if (n <= 0.0) continue;
        const double D = acc[i][1] + ridge, Bi = acc[i][2], gb = acc[i][4];
        step[1 + i] = ((-gb - Bi * dw) / D) * (n / (n + double(damping_c)));
        largest = fmax(largest, fabs(step[1 + i]));
      }
      const double shrink = largest > double(max_step) ? double(max_step) / largest : 1.0;
      params[0] = float(omega + step[0] * shrink);
      for (int i = 0; i < max_k; ++i)
        if (acc[i][0] > 0.0) params[1 + i] = float(double(params[1 + i]) + step[1 + i] * shrink);
    }
  }
  __syncthreads();
  for (int k = tid; k < 6 * max_k; k += kFitT) accum[k] = 0.0;
}

hipError_t launch_av_fit(int B, int max_k, const float* feature, const int8_t* labels, float* params,
                         double* accum, float damping_c, float ridge, float max_step, int do_update,
                         hipStream_t stream) {
  hipLaunchKernelGGL(av_fit_kernel, dim3(1), dim3(kFitT), 0, stream, B, max_k, feature, labels, params, accum,
                     damping_c, ridge, max_step, do_update);
  return hipGetLastError();
}

}  // namespace sv
