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
// refit step: one workgroup of 256 threads.  The batch's labelled drafts are
// items b * max_k + i; the first T = max_k * floor(256 / max_k) threads take
// items t, t + T, ... (coalesced loads), so that every item a thread takes
// belongs to the same position i = t mod max_k, and the thread keeps that
// position's six sums, formed in fp64, in registers.  The threads' sums then
// go to LDS and are added per position and sum in thread order (chunks of
// threads, then the chunk sums), a fixed order that makes the result
// deterministic.  On the round's last step the
// first max_k threads solve the arrowhead Newton system H * delta = -g by
// eliminating the intercepts (Schur complement on the slope), damp, bound
// the step, update the parameters and clear the accumulator.
// ---------------------------------------------------------------------------

constexpr int kFitT = 256;

__global__ __launch_bounds__(kFitT) void av_fit_kernel(int B, int max_k, const float* feature,
                                                       const int8_t* labels, float* params, double* accum,
                                                       float damping_c, float ridge, float max_step, int do_update) {
  __shared__ double part[6][kFitT];          // per thread, by sum
  __shared__ double mid[kFitT];              // chunk sums
  __shared__ double acc[SV_MAX_K][6];        // accumulator after this step
  __shared__ FitShared fsh;
  const int tid = threadIdx.x;
  const int T = (kFitT / max_k) * max_k;  // threads taking items (max_k >= 1)
  const int pos = tid % max_k;
  // parameters and the incoming accumulator with the first items: one round
  // trip to memory instead of one per item
  const double omega = params[0];
  const double beta = params[1 + pos];
  const double acc_in = tid < 6 * max_k ? accum[tid] : 0.0;
  double sum[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (tid < T) {
    const int n = B * max_k;
    // kChunk items per thread in flight: their loads are issued together
    constexpr int kChunk = 8;
    for (int it0 = tid; it0 < n; it0 += kChunk * T) {
      float x[kChunk];
      int y[kChunk];
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        // every load unconditional (past the end: the last item, masked), so
        // that the compiler does not order them one after another
        const int it = it0 + c * T, itc = min(it, n - 1);
        const float xv = feature[itc];
        const int yv = labels[itc];
        x[c] = it < n ? xv : 0.f;
        y[c] = it < n ? yv : -1;
      }
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        double v[6];
        fit_item(omega, beta, x[c], y[c], v);
#pragma unroll
        for (int k = 0; k < 6; ++k) sum[k] += v[k];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 6; ++k) part[k][tid] = sum[k];
  __syncthreads();
  // each of the 6 * max_k sums adds the M = T / max_k threads of its
  // position in two levels: C chunks of L threads, then the C chunk sums
  const int M = T / max_k, C = kFitT / (6 * max_k), L = (M + C - 1) / C;
  if (tid < 6 * max_k * C) {
    const int o = tid / C, c = tid % C;
    const int i = o / 6, k = o % 6;
    double t = 0.0;
    for (int u = c * L; u < min(M, (c + 1) * L); ++u) t += part[k][i + u * max_k];
    mid[tid] = t;
  }
  __syncthreads();
  if (tid < 6 * max_k) {
    const int i = tid / 6, k = tid % 6;
    double t = 0.0;
    for (int c = 0; c < C; ++c) t += mid[(i * 6 + k) * C + c];
    t += acc_in;
    acc[i][k] = t;
    if (!do_update) accum[tid] = t;
  }
  __syncthreads();
  if (!do_update) return;
  fit_update_params(acc, max_k, params, damping_c, ridge, max_step, fsh, tid);
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
