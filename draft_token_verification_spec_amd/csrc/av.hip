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
      double v[6];
      fit_item(omega, beta[i], x[i], y[i], v);
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
  if (tid == 0) fit_update_params(acc, max_k, params, damping_c, ridge, max_step);
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
