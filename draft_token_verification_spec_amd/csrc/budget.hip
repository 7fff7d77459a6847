// The estimator's global draft budget, on one workgroup.
//
// [AV] "Adaptive Verification ohne Confidence Head" (Arabic mirror), section
// "Other features considered": survivals are running products of the scores
// along each request's draft positions; the batch's survivals are ranked and
// the highest j are kept; the budget j maximises (sampling requests + sum of
// the j kept survivals) / (draft cost + verify cost of a step with j draft
// tokens).
//
// A batch holds at most SV_BUDGET_MAX_ITEMS positions (a serving batch times
// its drafts), so the whole decision fits one workgroup and its LDS: the
// survivals are formed in place, sorted (bitonic, descending), summed in
// binary64 and scanned for the best ratio; the kept drafts are then every
// survival above the cut plus, of those equal to it, the first ones in flat
// order (request-major), which keeps each request's kept drafts a prefix.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kBT = 1024;      // threads of the workgroup
constexpr int kBW = kBT / 64;  // waves
static_assert((SV_BUDGET_MAX_ITEMS & (SV_BUDGET_MAX_ITEMS - 1)) == 0, "the sort size is a power of two");

struct BudgetShared {
  float vals[SV_BUDGET_MAX_ITEMS];  // survivals (-1 where no draft), then ranked
  double dpart[kBW];
  int ipart[kBW];
  double best_r[kBW];
  int best_j[kBW];
  int word;
};

// Exclusive prefix over the workgroup of one value per thread, in thread
// order; `total` gets the sum.  T is int or double.
template <typename T>
__device__ __forceinline__ T block_exclusive(T v, T* part, T& total, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  T incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  T before = T(0), all = T(0);
  for (int w = 0; w < kBW; ++w) {
    if (w < wave) before += part[w];
    all += part[w];
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// Draft positions of request b that take part.
__device__ __forceinline__ int row_drafts(const int32_t* num_draft, int b, int max_k) {
  return min(max(num_draft[b], 0), max_k);
}

__global__ __launch_bounds__(kBT) void av_budget_kernel(int B, int max_k, const float* score,
                                                        const int32_t* num_draft, const float* draft_cost,
                                                        const float* verify_cost, int32_t* num_kept,
                                                        int32_t* budget_out) {
  __shared__ BudgetShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int items = B * max_k;
  int P = 1;  // sort size: a power of two >= items
  while (P < items) P <<= 1;

  // survivals (running products of the scores in binary32, left to right)
  // in flat order; -1, below every survival, marks positions past K_b
  int mine = 0;
  for (int b = tid; b < B; b += kBT) {
    const int K = row_drafts(num_draft, b, max_k);
    float run = 1.f;
    for (int i = 0; i < max_k; ++i) {
      if (i < K) run *= score[size_t(b) * max_k + i];
      sh.vals[b * max_k + i] = i < K ? run : -1.f;
    }
    mine += K;
  }
  for (int e = items + tid; e < P; e += kBT) sh.vals[e] = -1.f;
  int N = 0;
  (void)block_exclusive<int>(mine, sh.ipart, N, tid);  // also orders the stores above

  // rank: bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kBT) {
        const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
        const float x = sh.vals[lo], y = sh.vals[hi];
        if ((x < y) == ((lo & size) == 0)) {
          sh.vals[lo] = y;
          sh.vals[hi] = x;
        }
      }
      __syncthreads();
    }
  }

  // estimated tokens per cost for j = 0..N kept drafts (binary64 sums over
  // the ranked survivals, in rank order within each thread's run)
  const int c = (N + kBT - 1) / kBT;
  const int j0 = min(N, tid * c), j1 = min(N, j0 + c);
  double local = 0.0;
  for (int j = j0; j < j1; ++j) local += double(sh.vals[j]);
  double total = 0.0;
  double run = block_exclusive<double>(local, sh.dpart, total, tid);
  double best = -1.0;
  int bj = 0x7fffffff;
  if (tid == 0) {
    best = double(B) / (double(draft_cost[0]) + double(verify_cost[0]));
    bj = 0;
  }
  for (int j = j0; j < j1; ++j) {
    run += double(sh.vals[j]);
    const double r = (double(B) + run) / (double(draft_cost[j + 1]) + double(verify_cost[j + 1]));
    if (r > best) {
      best = r;
      bj = j + 1;
    }
  }
  // the largest ratio; the smallest j among equal ones
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double r2 = __shfl_xor(best, o, 64);
    const int j2 = __shfl_xor(bj, o, 64);
    if (r2 > best || (r2 == best && j2 < bj)) {
      best = r2;
      bj = j2;
    }
  }
  if (lane == 0) {
    sh.best_r[wave] = best;
    sh.best_j[wave] = bj;
  }
  __syncthreads();
  if (tid == 0) {
    double r = sh.best_r[0];
    int j = sh.best_j[0];
    for (int w = 1; w < kBW; ++w)
      if (sh.best_r[w] > r || (sh.best_r[w] == r && sh.best_j[w] < j)) {
        r = sh.best_r[w];
        j = sh.best_j[w];
      }
    sh.word = j;
    *budget_out = j;
  }
  __syncthreads();
  const int budget = sh.word;

  // kept drafts: survivals above the cut, then those equal to it in flat order
  const float cut = budget > 0 ? sh.vals[budget - 1] : 2.f;
  const int rb = (B + kBT - 1) / kBT;  // requests per thread, contiguous
  const int b0 = min(B, tid * rb), b1 = min(B, b0 + rb);
  int gt = 0, eq = 0;
  for (int b = b0; b < b1; ++b) {
    const int K = row_drafts(num_draft, b, max_k);
    float s = 1.f;
    for (int i = 0; i < K; ++i) {
      s *= score[size_t(b) * max_k + i];
      gt += s > cut;
      eq += s == cut;
    }
  }
  int gt_all = 0, eq_all = 0;
  (void)block_exclusive<int>(gt, sh.ipart, gt_all, tid);
  int eq_before = block_exclusive<int>(eq, sh.ipart, eq_all, tid);
  const int ties = budget - gt_all;  // equal survivals to keep, in flat order
  for (int b = b0; b < b1; ++b) {
    const int K = row_drafts(num_draft, b, max_k);
    float s = 1.f;
    int g = 0, e = 0;
    for (int i = 0; i < K; ++i) {
      s *= score[size_t(b) * max_k + i];
      g += s > cut;
      e += s == cut;
    }
    num_kept[b] = g + min(e, max(0, ties - eq_before));
    eq_before += e;
  }
}

}  // namespace

hipError_t launch_av_budget(int B, int max_k, const float* score, const int32_t* num_draft, const float* draft_cost,
                            const float* verify_cost, int32_t* num_kept, int32_t* budget, hipStream_t stream) {
  hipLaunchKernelGGL(av_budget_kernel, dim3(1), dim3(kBT), 0, stream, B, max_k, score, num_draft, draft_cost,
                     verify_cost, num_kept, budget);
  return hipGetLastError();
}

}  // namespace sv
