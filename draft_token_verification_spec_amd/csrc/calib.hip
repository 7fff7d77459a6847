// Calibration metrics of the online acceptance estimator over its labelled
// stream: AUC, log-loss and ECE.
//
// [AV] "Adaptive Verification ohne Confidence Head" (Arabic mirror), section
// "Other features considered": AUC is the probability that an accepted draft
// scores above a rejected one (ties count half); log-loss the mean negative
// log-probability of the observed outcome; ECE the occupancy-weighted gap
// between mean prediction and observed frequency over probability bins.
// The labels are those of the refit ([AV] "Fitting the coefficients").
//
// The stream is kept in a caller-owned binary64 accumulator (SV_CALIB_WORDS
// words): labelled count, accepted count, the log-loss sum, per ECE bin
// (10 equal-width bins) the count, the sum of scores and the sum of labels,
// and per class a histogram of the score over SV_CALIB_AUC_BINS equal-width
// bins.  Each kernel is one workgroup with a fixed reduction order, so the
// same calls give bit-identical accumulators and metrics.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kCT = 1024;
constexpr int kCW = kCT / 64;
constexpr int kEceBins = 10;
constexpr int kAucBins = SV_CALIB_AUC_BINS;
// accumulator words
constexpr int kAN = 0, kAPos = 1, kALoss = 2, kAEceN = 3, kAEceP = kAEceN + kEceBins, kAEceY = kAEceP + kEceBins,
              kAPosHist = kAEceY + kEceBins, kANegHist = kAPosHist + kAucBins;
static_assert(kANegHist + kAucBins == SV_CALIB_WORDS, "accumulator layout");
constexpr double kEps = 1e-7;

// Sum over the workgroup in a fixed order; the result in every thread.
__device__ __forceinline__ double block_sum(double v, double* part, int tid) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((tid & 63) == 0) part[tid >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kCW; ++w) s += part[w];
  __syncthreads();
  return s;
}

__device__ __forceinline__ int score_bin(float p, int bins) {
  return min(max(int(floorf(p * float(bins))), 0), bins - 1);
}

struct CalibShared {
  uint32_t hist[2][kAucBins];  // accepted, rejected
  uint32_t ece_n[kEceBins], ece_y[kEceBins];
  double part[kCW];
  double psum[kEceBins][kCW];  // per bin and wave: sums of the scores
};

__global__ __launch_bounds__(kCT) void calib_accumulate_kernel(int items, const float* score, const int8_t* labels,
                                                               double* acc) {
  __shared__ CalibShared sh;
  const int tid = threadIdx.x;
  for (int b = tid; b < 2 * kAucBins; b += kCT) (&sh.hist[0][0])[b] = 0u;
  if (tid < kEceBins) sh.ece_n[tid] = sh.ece_y[tid] = 0u;
  __syncthreads();
  double loss = 0.0, ps[kEceBins];
#pragma unroll
  for (int k = 0; k < kEceBins; ++k) ps[k] = 0.0;
  for (int e = tid; e < items; e += kCT) {
    const int y = labels[e];
    if (y != 0 && y != 1) continue;
    const float p = score[e];
    const double pc = fmin(fmax(double(p), kEps), 1.0 - kEps);
    loss -= y ? log(pc) : log(1.0 - pc);
    const int eb = score_bin(p, kEceBins);
#pragma unroll
    for (int k = 0; k < kEceBins; ++k) ps[k] += (k == eb) ? double(p) : 0.0;
    atomicAdd(&sh.ece_n[eb], 1u);
    atomicAdd(&sh.ece_y[eb], uint32_t(y));
    atomicAdd(&sh.hist[y ? 0 : 1][score_bin(p, kAucBins)], 1u);
  }
  // per bin: each wave's sum (butterfly), then the waves in order
#pragma unroll
  for (int k = 0; k < kEceBins; ++k) {
    double v = ps[k];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((tid & 63) == 0) sh.psum[k][tid >> 6] = v;
  }
  loss = block_sum(loss, sh.part, tid);  // its barriers also order the LDS counts and sums
  // this workgroup is the only writer of the accumulator
  for (int b = tid; b < kAucBins; b += kCT) {
    acc[kAPosHist + b] += double(sh.hist[0][b]);
    acc[kANegHist + b] += double(sh.hist[1][b]);
  }
  if (tid < kEceBins) {
    acc[kAEceN + tid] += double(sh.ece_n[tid]);
    acc[kAEceY + tid] += double(sh.ece_y[tid]);
    double sp = 0.0;
    for (int w = 0; w < kCW; ++w) sp += sh.psum[tid][w];
    acc[kAEceP + tid] += sp;
  }
  if (tid == 0) {
    double n = 0.0, pos = 0.0;
    for (int k = 0; k < kEceBins; ++k) {
      n += double(sh.ece_n[k]);
      pos += double(sh.ece_y[k]);
    }
    acc[kAN] += n;
    acc[kAPos] += pos;
    acc[kALoss] += loss;
  }
}

__global__ __launch_bounds__(kCT) void calib_metrics_kernel(double* acc, double* out, int reset) {
  __shared__ double part[kCW];
  __shared__ double carry[kCW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const double n = acc[kAN], npos = acc[kAPos], nneg = n - npos;
  // AUC: for each bin, accepted drafts there times rejected drafts in lower
  // bins, plus half the pairs within the bin; bins in contiguous runs per thread
  constexpr int per = kAucBins / kCT;
  static_assert(kAucBins % kCT == 0, "AUC bins per thread");
  double negrun = 0.0;
  for (int q = 0; q < per; ++q) negrun += acc[kANegHist + tid * per + q];
  // exclusive prefix of the rejected counts over the threads, in order
  double incl = negrun;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) carry[wave] = incl;
  __syncthreads();
  double below = incl - negrun;
  for (int w = 0; w < wave; ++w) below += carry[w];
  double wins = 0.0;
  for (int q = 0; q < per; ++q) {
    const double pos = acc[kAPosHist + tid * per + q], neg = acc[kANegHist + tid * per + q];
    wins += pos * below + 0.5 * pos * neg;
    below += neg;
  }
  wins = block_sum(wins, part, tid);
  if (tid == 0) {
    double ece = 0.0;
    for (int k = 0; k < kEceBins; ++k) ece += fabs(acc[kAEceP + k] - acc[kAEceY + k]);
    out[0] = (npos > 0.0 && nneg > 0.0) ? wins / (npos * nneg) : NAN;
    out[1] = n > 0.0 ? acc[kALoss] / n : NAN;
    out[2] = n > 0.0 ? ece / n : NAN;
  }
  if (reset) {
    __syncthreads();  // every read of the accumulator is done
    for (int w = tid; w < SV_CALIB_WORDS; w += kCT) acc[w] = 0.0;
  }
}

}  // namespace

hipError_t launch_calib_accumulate(int items, const float* score, const int8_t* labels, double* accum,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(calib_accumulate_kernel, dim3(1), dim3(kCT), 0, stream, items, score, labels, accum);
  return hipGetLastError();
}

hipError_t launch_calib_metrics(double* accum, double* metrics, int reset, hipStream_t stream) {
  hipLaunchKernelGGL(calib_metrics_kernel, dim3(1), dim3(kCT), 0, stream, accum, metrics, reset);
  return hipGetLastError();
}

}  // namespace sv
