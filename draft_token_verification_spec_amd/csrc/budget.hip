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
// survivals are formed in place, sorted (descending: each wave sorts a
// sixteenth in registers, then four rounds of merges by rank), summed in
// binary64 and scanned for the best ratio; the kept drafts are then every
// survival above the cut plus, of those equal to it, the first ones in flat
// order (request-major), which keeps each request's kept drafts a prefix.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kBT = 1024;      // threads of the workgroup
constexpr int kBW = kBT / 64;  // waves
static_assert((SV_BUDGET_MAX_ITEMS & (SV_BUDGET_MAX_ITEMS - 1)) == 0, "the sort size is a power of two");

constexpr int kPer = SV_BUDGET_MAX_ITEMS / kBT;  // sorted elements per thread at most
static_assert(kPer == 1 || kPer == 2 || kPer == 4, "the wave sort is instantiated for 1, 2 and 4");

struct BudgetShared {
  float surv[SV_BUDGET_MAX_ITEMS];  // survivals in flat order (b * max_k + i)
  float vals[SV_BUDGET_MAX_ITEMS];  // the survivals being sorted, then the ranked survivals
  float tmp[SV_BUDGET_MAX_ITEMS];   // the other buffer of the merge rounds
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

// Request b's survivals (running products of its scores in binary32, left to
// right) at positions 0..max_k-1; -1, below every survival, past K_b.  The
// scores are loaded together, without waiting for K_b.
__device__ __forceinline__ void row_survivals(const float* score, int b, int K, int max_k,
                                              float (&out)[SV_MAX_K]) {
  float sc[SV_MAX_K];
#pragma unroll
  for (int i = 0; i < SV_MAX_K; ++i) sc[i] = i < max_k ? score[size_t(b) * max_k + i] : 0.f;
  float run = 1.f;
#pragma unroll
  for (int i = 0; i < SV_MAX_K; ++i) {
    if (i < K) run *= sc[i];
    out[i] = i < K ? run : -1.f;
  }
}

// Descending bitonic sort of one wave's chunk of 64 * PER values, value
// k * 64 + lane of the chunk in v[k] of that lane: pairs closer than 64 are
// exchanged between lanes, the others inside a thread.  No LDS, no barrier;
// every stride is a compile-time constant.
template <int PER, int SIZE, int STRIDE>
__device__ __forceinline__ void sort_stage(float (&v)[kPer], int lane) {
  if constexpr (STRIDE >= 64) {
    constexpr int ks = STRIDE / 64;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if ((k & ks) == 0) {
        const float x = v[k], y = v[k | ks];
        const bool desc = ((k * 64 + lane) & SIZE) == 0;
        v[k] = desc ? fmaxf(x, y) : fminf(x, y);
        v[k | ks] = desc ? fminf(x, y) : fmaxf(x, y);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = k * 64 + lane;
      const float y = __shfl_xor(v[k], STRIDE, 64);
      const bool lower = (e & STRIDE) == 0;
      const bool desc = (e & SIZE) == 0;
      v[k] = (lower == desc) ? fmaxf(v[k], y) : fminf(v[k], y);
    }
  }
  if constexpr (STRIDE > 1) sort_stage<PER, SIZE, STRIDE / 2>(v, lane);
}

template <int PER, int SIZE>
__device__ __forceinline__ void sort_sizes(float (&v)[kPer], int lane) {
  sort_stage<PER, SIZE, SIZE / 2>(v, lane);
  if constexpr (SIZE < 64 * PER) sort_sizes<PER, SIZE * 2>(v, lane);
}

template <int PER>
__device__ __forceinline__ void wave_sort(float (&v)[kPer], int lane) {
  sort_sizes<PER, 2>(v, lane);
}

// Entries of the descending run r[0..n-1] that come before x in the merged
// order: those greater than x, and (if x is from the right run of the pair)
// those equal to it.
__device__ __forceinline__ int merge_rank(const float* r, int n, float x, bool right) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (right ? r[mid] >= x : r[mid] > x)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kBT) void av_budget_kernel(int B, int max_k, const float* score,
                                                        const int32_t* num_draft, const float* draft_cost,
                                                        const float* verify_cost, int32_t* num_kept,
                                                        int32_t* budget_out) {
  __shared__ BudgetShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int items = B * max_k;
  int P = kBT;  // sort size: a power of two >= items, at least one element per thread
  while (P < items) P <<= 1;
  const int per = P / kBT;  // elements per thread: element k * kBT + tid in v[k]

  // survivals in flat order into the exchange buffer (requests in contiguous
  // runs per thread; the same runs pick the kept prefixes at the end)
  const int rb = (B + kBT - 1) / kBT;
  const int b0 = min(B, tid * rb), b1 = min(B, b0 + rb);
  int mine = 0;
  for (int b = b0; b < b1; ++b) {
    const int K = row_drafts(num_draft, b, max_k);
    float sv[SV_MAX_K];
    row_survivals(score, b, K, max_k, sv);
#pragma unroll
    for (int i = 0; i < SV_MAX_K; ++i)
      if (i < max_k) sh.surv[b * max_k + i] = sh.vals[b * max_k + i] = sv[i];
    mine += K;
  }
  for (int e = items + tid; e < P; e += kBT) sh.vals[e] = -1.f;
  int N = 0;
  (void)block_exclusive<int>(mine, sh.ipart, N, tid);  // also orders the stores above

  // rank: wave w sorts values [w * C, (w + 1) * C) (C = P / 16) in
  // registers, then four rounds merge pairs of sorted runs: each value's
  // place in the merged run is its place in its own run plus the number of
  // values of the other run before it (found by bisection), so the rounds
  // need no compare-exchange network and one barrier each
  {
    const int C = 64 * per;
    float v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = k < per ? sh.vals[wave * C + k * 64 + lane] : 0.f;
    if (per == 1)
      wave_sort<1>(v, lane);
    else if (per == 2)
      wave_sort<2>(v, lane);
    else
      wave_sort<4>(v, lane);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (k < per) sh.vals[wave * C + k * 64 + lane] = v[k];
    float* src = sh.vals;
    float* dst = sh.tmp;
    for (int L = C; L < P; L <<= 1) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if (k < per) {
          const int g = k * kBT + tid;
          const int run = g / L, i = g - run * L;
          const float x = src[g];
          dst[(run & ~1) * L + i + merge_rank(src + (run ^ 1) * L, L, x, run & 1)] = x;
        }
      }
      float* t = src;
      src = dst;
      dst = t;
    }
    __syncthreads();
    // four rounds: the ranked survivals are back in sh.vals
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
  for (int j0b = j0; j0b < j1; j0b += kPer) {
    float dc[kPer], vc[kPer];  // the run's cost entries, loaded together
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      dc[q] = j0b + q < j1 ? draft_cost[j0b + q + 1] : 1.f;
      vc[q] = j0b + q < j1 ? verify_cost[j0b + q + 1] : 1.f;
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (j0b + q < j1) {
        run += double(sh.vals[j0b + q]);
        const double r = (double(B) + run) / (double(dc[q]) + double(vc[q]));
        if (r > best) {
          best = r;
          bj = j0b + q + 1;
        }
      }
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
  int gt = 0, eq = 0;
  for (int e = b0 * max_k; e < b1 * max_k; ++e) {  // past K_b the survival is -1: neither
    gt += sh.surv[e] > cut;
    eq += sh.surv[e] == cut;
  }
  int gt_all = 0, eq_all = 0;
  (void)block_exclusive<int>(gt, sh.ipart, gt_all, tid);
  int eq_before = block_exclusive<int>(eq, sh.ipart, eq_all, tid);
  const int ties = budget - gt_all;  // equal survivals to keep, in flat order
  for (int b = b0; b < b1; ++b) {
    int g = 0, e = 0;
    for (int i = 0; i < max_k; ++i) {
      g += sh.surv[b * max_k + i] > cut;
      e += sh.surv[b * max_k + i] == cut;
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
