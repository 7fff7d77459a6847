// Verification on top-k / top-p filtered distributions.
//
// [AV] "Adaptive Verification ohne Confidence Head", sections "Other
// features considered" and "Benchmarks": drafts are sampled and verified at
// temperature 1 with top-p 0.95, so the distributions speculative sampling
// ([CS] "One speculative step") compares are the filtered ones.  Readings:
// top-p keeps a token when the tokens with a strictly larger logit hold less
// than top_p of the row's probability; top-k keeps it when fewer than k
// tokens have a strictly larger logit; with both, a token must pass both.
// Each row of a stochastic request is filtered and renormalised; greedy
// requests are not filtered (the argmax is always kept).
//
// A row's kept set is {v : key(z_v) >= t} for a threshold key t (key = the
// order-preserving integer image of the logit), found by an exact radix
// select with deterministic histograms:
//   level 0  built by the statistics pass itself, so that one read of a
//            filtered row serves both.  fp32 rows: bins of 1/8 unit of log2
//            weight on an absolute grid, the 511 grid cells from the row
//            maximum's down (the last bin collecting everything further
//            down), each with its count and its mass; the row's total mass
//            is the sum of its bins.  bf16 rows: exact counts of the 1024
//            keys from the row maximum's down, and the row's total mass from
//            the segments' weight sums; a threshold inside that window is
//            found here, with no key level;
//   level L  8-bit digits of the key within the boundary bin's keys, until
//            one key remains (fp32: 4 levels at most); bf16 rows whose
//            threshold lies below the window take the keys below it by
//            weight cells first, then 2 levels of digits at most.
// Each level's counts come from a streaming pass (one workgroup per 32 KiB
// row segment; every count an integer added with LDS atomics, so the result
// does not depend on the order of the additions) and a selection (one wave
// per row: segment histograms merged in order, exclusive scans, the boundary
// bin, key or digit).  Key levels read only the segments of the rows still
// searching (fp32 rows: every filtered row at the first key level).  The
// verdict, the residual / bonus weights and the draw then run on the
// filtered rows.
#include <type_traits>

#include "sv_segment.hpp"

namespace sv {

namespace {

constexpr int kFT = 256;  // threads of the histogram and selection kernels
constexpr int kFV = 8;    // 16-byte vectors per thread and segment (32 KiB)
constexpr int kBins = 256;  // key-digit bins
constexpr float kFix = 1099511627776.f;  // 2^40
static_assert(kFT * kFV * 16 == kHalfBytes, "a histogram segment is a 32 KiB sampling segment");
static_assert(kFT == kThreads && kFV == kNV, "a histogram segment is a statistics segment");

// Order-preserving key of a logit: bf16 rows use the 16 bits of the value,
// fp32 rows all 32; -0 is keyed as +0.
template <typename ET>
struct Key;

template <>
struct Key<uint16_t> {
  static constexpr uint32_t kMin = 0x007fu;  // -inf
  [[maybe_unused]] static constexpr uint32_t kMax = 0xff80u;  // +inf
  __device__ __forceinline__ static uint32_t of(float z) {
    uint32_t u = __float_as_uint(z) >> 16;
    if (u == 0x8000u) u = 0u;
    return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
  }
  __device__ __forceinline__ static float value(uint32_t k) {
    const uint32_t u = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
    return __uint_as_float(u << 16);
  }
};

template <>
struct Key<float> {
  static constexpr uint32_t kMin = 0x007fffffu;
  static constexpr uint32_t kMax = 0xff800000u;
  __device__ __forceinline__ static uint32_t of(float z) {
    uint32_t u = __float_as_uint(z);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  __device__ __forceinline__ static float value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
  }
};

// Level-0 bins.  The grid cell of a logit z is F(z) = floor(z * 8c) (the
// product rounded once, then floored: a non-decreasing function of z alone),
// and cell F holds the weights 2^(z c) in [2^(F/8), 2^((F+1)/8)).  A row's bin
// of z is G - F(z) clamped to [0, 511], with G = ceil(max * 8c): bin 0 or 1
// holds the maximum, bin 511 everything 511 cells or more below G, whose
// weights are below 2^-63.6 of the maximum's (all of them together below
// 2^-42 of it, even at the longest rows: they are left out of the row's
// total).  The statistics pass bins a segment against its own grid point
// Gs = ceil(segment max * 8c), and a segment bin shifts into the row bin by
// the integer G - Gs, so that the segments need not know the row maximum.
// Within a cell a weight is the cell's lower edge times r = 2^((z 8c - F)/8)
// in [1, 2^(1/8)).  Each element adds one 64-bit word, 2^45 + bits(r): the
// count in the top 19 bits and, below them, the sum of the binary32 bit
// patterns of r (< 2^45 for the 2^14 elements of a segment).  For r in [1, 2)
// bits(r) - bits(1) is (r - 1) 2^23 exactly, so a bin's mass is
// edge x (count + (sum - count bits(1)) 2^-23): the sum of the weights r as
// computed, added exactly, independent of the order of the additions.  (A
// weight rounded just below 1 counts one unit of 2^-23 low.)
constexpr int kBins0 = 512;
constexpr int kBinsPerLog2 = 8;
constexpr int kCountShift0 = 45;  // level-0 word: count << 45 | sum of bits(r)
constexpr uint64_t kOne0 = 1ull << kCountShift0;
constexpr uint64_t kOneBits = 0x3f800000ull;  // bits(1.0f)
constexpr double kFrac0 = 8388608.0;            // 2^23

// bf16 rows take level 0 at key resolution instead: a bf16 logit has 2^16
// possible values, and the 1024 keys from a maximum's down cover 8 octaves
// of |z| (128 keys each), where a top-p boundary usually lies.  Each segment
// counts its elements by key in that window below its own maximum's key
// (every element of a key has the same weight, so a count is all a key
// needs), and sums the weights of all its elements for the row's total.
// The row's window is the one below the row maximum's key; a segment's
// window reaches at least as far down, since its maximum is not above the
// row's.  When the threshold lies below the row's window, the search
// continues with the key levels over the keys below it.
constexpr int kWin = 2 * kBins0;  // window keys: the level-0 histogram's words, as 32-bit counts
template <typename ET>
constexpr bool kKeyWindow = sizeof(ET) == 2;
// km - Key<uint16_t>::of(z) for a bf16 value z, from its bits: with t the
// bits sign-extended, the key is (t ^ (0x7fff if z < 0)) + 0x8000 (z + 0
// turns -0 into +0 first)
__device__ __forceinline__ uint32_t key_offset16(uint32_t km, float z) {
  const int t = __float_as_int(z + 0.f) >> 16;
  return uint32_t(int(km) - 0x8000 - (t ^ ((t >> 15) & 0x7fff)));
}
__device__ __forceinline__ float cell_of(float z, float c8) { return floorf(z * c8); }
// the bin of z against grid point g (a whole number of cells): g - F(z),
// exact where it is below 511, clamped to [0, 511]
__device__ __forceinline__ float bin0f(float z, float c8, float g) {
  return __builtin_amdgcn_fmed3f(g - cell_of(z, c8), 0.f, float(kBins0 - 1));
}
__device__ __forceinline__ int bin0(float z, float c8, float g) { return int(bin0f(z, c8, g)); }
// the grid point of a row or segment maximum m
__device__ __forceinline__ float grid_point(float m, float c8) { return ceilf(m * c8); }

// Weight of an element relative to the row maximum, in 2^-40 fixed point.
__device__ __forceinline__ uint64_t fixed_mass(float z, float c, float mc) {
  return uint64_t(__builtin_rintf(fast_exp2(fmaf(z, c, -mc)) * kFix));
}

// State of one threshold search of one row (slot 0: top-k, slot 1: top-p).
// Masses are in units of the row maximum's weight.
struct FSearch {
  uint32_t lo, hi;  // key interval holding the threshold
  uint32_t cabove;  // tokens with a key above the interval
  uint32_t state;   // 0 unused, 1 searching, 2 done, 3 searching by weight cells (below)
  double mabove;    // mass above the interval (from the window pass on)
  double mfinal;    // done: mass of the kept tokens; weight cells: the edge of the top cell
  double target;    // top-k: k; top-p: top_p x the row's mass
  uint32_t key;     // done: the threshold key
  uint32_t kept;    // done: kept tokens
};
static_assert(sizeof(FSearch) == kFilterSearchBytes, "search state layout");
static_assert(kBins == kFilterBins && kBins0 == kFilterBins0, "histogram bins");
static_assert(kFT * kFV * 8 < (1 << (64 - kCountShift0)) && kFT * kFV * 8 * double(0x3f8b95c2u) < double(kOne0),
              "level-0 counts and bit sums of a segment fit their fields");
static_assert(kFT * kFV * 8 < 65536, "a bf16 segment's key counts fit 16 bits");

struct FiltArgs {
  int B, V, max_k, R, nseg2;
  const void* draft;
  const int64_t* draft_start;
  int64_t draft_stride;
  const void* target;
  const int64_t* target_start;
  int64_t target_stride;
  const int32_t* num_draft;
  const int32_t* tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* u_accept;
  const float* u_residual;
  const float* u_bonus;
  int32_t* accept_len;
  int32_t* out_tokens;
  int8_t* labels;
  float* p_draft;
  float* p_target;
  int32_t* kept;
  Partial* partials;        // [B][R][nseg2] segment statistics
  float* zval;              // [B][R] logits at the draft tokens
  uint64_t* hmass;          // [B][R][nseg2][2][kBins]  key-level masses (digits wider than one key)
  uint32_t* hcount;         // [B][R][nseg2][2][kBins0]  level 0: per bin count << 45 | sum of bits(r) (u64);
                            //   key levels: counts
  FSearch* search;          // [B][R][2]
  uint32_t* tickets;        // [B][R]  arrivals per row (zero between passes)
  uint32_t* work;           // [2][B][R][nseg2]  segments still searching, for the next key level
  uint32_t* wcount;         // [kMaxKeyLevels]  entries of work per key level after the first
};

struct ReqFilter {
  int K;
  float T;
  bool on_k, on_p;
  int top_k;
  float top_p;
};

__device__ __forceinline__ ReqFilter req_filter(const FiltArgs& a, int b) {
  ReqFilter f;
  f.K = min(max(a.num_draft[b], 0), a.max_k);
  f.T = a.temperature[b];
  f.top_k = a.top_k[b];
  f.top_p = a.top_p[b];
  const bool stoch = f.T > 0.f;
  f.on_k = stoch && f.top_k > 0 && f.top_k < a.V;
  f.on_p = stoch && f.top_p < 1.f;
  return f;
}

// Is row slot rs (draft i at i, target j at max_k + j) of the request read
// and filtered?
__device__ __forceinline__ bool row_filtered(const FiltArgs& a, const ReqFilter& f, int rs) {
  if (!(f.on_k || f.on_p)) return false;
  return rs < a.max_k ? rs < f.K : rs - a.max_k <= f.K;
}

template <typename ET>
__device__ __forceinline__ const ET* row_ptr(const FiltArgs& a, int b, int rs) {
  if (rs < a.max_k) return static_cast<const ET*>(a.draft) + (a.draft_start[b] + rs) * a.draft_stride;
  return static_cast<const ET*>(a.target) + (a.target_start[b] + (rs - a.max_k)) * a.target_stride;
}

// Maximum logit of a row from its segment statistics (exact: a maximum).
__device__ __forceinline__ float wave_row_max(const Partial* p, int n, int lane) {
  float m = -INFINITY;
  for (int q = lane; q < n; q += 64) m = fmaxf(m, p[q].m);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Vector of a row holding elements first..first+N-1; positions >= limit
// hold a NaN (never a logit: rows have no NaN).
template <typename ET>
__device__ __forceinline__ uint4 load_nan_tail(const ET* row, int first, int limit, bool aligned) {
  constexpr int N = Elem<ET>::N;
  if (aligned && first + N <= limit) return *reinterpret_cast<const uint4*>(row + first);
  constexpr uint32_t nan = N == 8 ? 0x7fc0u : 0x7fc00000u;
  uint4 w;
#pragma unroll
  for (int j = 0; j < N; ++j) Elem<ET>::put(w, j, (first + j < limit) ? Elem<ET>::raw(row + first + j) : nan);
  return w;
}

// ---------------------------------------------------------------------------
// selection
// ---------------------------------------------------------------------------
//
// Level 0 and an fp32 row's first key level are selected by kernels of their
// own (one wave per row).  The other key levels, where few rows still
// search, run on the listed segments only, and a row's selection is made
// there by the workgroup that delivers the row's last segment histogram
// (every segment workgroup publishes its histogram with device-scope stores,
// then takes a ticket on the row's arrival counter; see arrive_last_all),
// reading the others' histograms with device-scope loads.  The counter is
// back at zero when the selection ends.

constexpr int kMaxSegs = int(int64_t(SV_MAX_V) * 4 / (kFT * kFV * 16));  // 32 KiB segments of the longest row
constexpr int kMaxKeyLevels = 4;  // fp32 keys: 4 digits of 8 bits
// Entry of wcount counting the bf16 rows' segments listed for the first key
// level (levels 2.. count theirs in entries 0..kMaxKeyLevels - 2; a bf16
// search has 3 key levels at most, so the entry is free for it, and list 1
// of `work` is read by the first key level before the second lists the
// third level's segments there); cleared by the statistics pass.
constexpr int kFirstList = kMaxKeyLevels - 1;

__device__ __forceinline__ uint64_t load_dev64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_dev32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 2^(-k/8), k = 0..7: a level-0 bin edge is 2^(-j/8) = 2^-(j/8 rounded down)
// times the entry for j mod 8.
__constant__ const double kPow2Eighth[8] = {0x1.0000000000000p+0, 0x1.d5818dcfba487p-1, 0x1.ae89f995ad3adp-1,
                                            0x1.8ace5422aa0dbp-1, 0x1.6a09e667f3bcdp-1, 0x1.4bfdad5362a27p-1,
                                            0x1.306fe0a31b715p-1, 0x1.172b83c7d517bp-1};

// Arrival counter of a row, for histograms that every thread of the
// workgroup published: each thread waits until its own stores have
// completed, then thread 0 takes a ticket.  The workgroup taking the last
// one (want - 1) selects the row; its loads of the published data are
// issued after its ticket returned.  The verdict in all threads.
__device__ __forceinline__ bool arrive_last_all(uint32_t* ticket, uint32_t want, int* lds_flag) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0): this thread's published stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    *lds_flag = (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want - 1) ? 1 : 0;
  __syncthreads();
  return *lds_flag != 0;
}

// The smallest key whose level-0 bin is <= j and the largest whose bin is
// >= j (the bin is non-increasing in the key): the keys of bins [.., j] and
// [j, ..].  Bisections of the key space; they start from a few keys around
// the bin edge's value ((g - j)/8c, resp. (g - j + 1)/8c) when those keys
// are seen to enclose the answer, and from the whole key space otherwise.
template <typename ET>
__device__ uint32_t key_lo_of_bin(int j, float c8, float g) {
  uint64_t lo = Key<ET>::kMin, hi = Key<ET>::kMax;
  const float ze = (g - float(j)) / c8;
  if (isfinite(ze)) {
    const uint64_t k0 = Key<ET>::of(ze);
    const uint64_t l = max(k0, uint64_t(Key<ET>::kMin) + 4) - 4, h = min(k0 + 4, uint64_t(Key<ET>::kMax));
    if (bin0(Key<ET>::value(uint32_t(h)), c8, g) <= j &&
        (l == Key<ET>::kMin || bin0(Key<ET>::value(uint32_t(l - 1)), c8, g) > j)) {
      lo = l;
      hi = h;
    }
  }
  while (lo < hi) {
    const uint64_t mid = (lo + hi) >> 1;
    if (bin0(Key<ET>::value(uint32_t(mid)), c8, g) <= j) hi = mid;
    else lo = mid + 1;
  }
  return uint32_t(lo);
}

template <typename ET>
__device__ uint32_t key_hi_of_bin(int j, float c8, float g) {
  uint64_t lo = Key<ET>::kMin, hi = Key<ET>::kMax;
  const float ze = (g - float(j) + 1.f) / c8;
  if (isfinite(ze)) {
    const uint64_t k0 = Key<ET>::of(ze);
    const uint64_t l = max(k0, uint64_t(Key<ET>::kMin) + 4) - 4, h = min(k0 + 4, uint64_t(Key<ET>::kMax));
    if (bin0(Key<ET>::value(uint32_t(l)), c8, g) >= j &&
        (h == Key<ET>::kMax || bin0(Key<ET>::value(uint32_t(h + 1)), c8, g) < j)) {
      lo = l;
      hi = h;
    }
  }
  while (lo < hi) {
    const uint64_t mid = (lo + hi + 1) >> 1;
    if (bin0(Key<ET>::value(uint32_t(mid)), c8, g) >= j) lo = mid;
    else hi = mid - 1;
  }
  return uint32_t(lo);
}

// A bf16 search whose threshold lies below the key window (state
// kSearchCells) takes its first key level by weight cells instead of key
// digits: the keys below the window spread over many octaves of |z|, most of
// them near zero, where a cell of 1/8 log2 unit of weight holds thousands of
// keys but 8-bit key digits split nothing.  Digit 255 - j holds level-0 bin
// j against the cell g of the interval's top value (j = g - F(z), the cells
// g .. g - 254), digit 0 every lower cell; a digit's key range comes from
// the level-0 bisections.  Each element adds one 64-bit word as at level 0,
// 2^45 + bits(r) with r its weight relative to its cell's lower edge (1 in
// digit 0, whose mass is only needed when it narrows to one key, and is
// then its count times that key's weight).
constexpr uint32_t kSearchCells = 3u;

// Wave-wide reductions and exclusive prefix in lane order (every lane gets
// the result).
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}
template <typename T>
__device__ __forceinline__ T wave_excl_scan(T x, int lane, T* total) {
  T incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  *total = __shfl(incl, 63, 64);
  return incl - x;
}

constexpr int kSelBins = kBins0 / 64;  // level-0 bins per lane of the selection

struct Sel0Shared {
  float segm[kMaxSegs];  // segment maxima of the row
  int segn[kMaxSegs];    // bins (bf16: window counts) stored per segment
  double segt[kMaxSegs];  // bf16: the segments' weight sums relative to their maxima
  uint32_t win[kWin + kWin / 16];  // bf16: the row's window counts, one pad word per 16
  uint32_t cab[2];
  double mab[2];
  uint32_t klo[2], khi[2];
};

// Level-0 selection of a row slot by one wave, lane t holding bins 8t ..
// 8t + 7.  The row's segment histograms are shifted onto the row's grid
// point and merged in segment order; bin masses, in units of the row
// maximum's weight, are edge x (count + excess 2^-23), and the row's total mass
// is the sum of the masses of bins 0..510 (bin 511's never enters; its count
// is the row's length less the other bins').  The boundary bin of each
// search is the last non-empty bin whose count (top-k) or mass (top-p,
// against top_p x the row's total) above it is below the target; the search
// continues over that bin's keys with the count and mass above it.
template <typename ET>
__device__ void select0_row(const FiltArgs& a, const ReqFilter& f, size_t row, const Partial& p0, Sel0Shared& sh,
                            int lane) {
  static_assert(kSelBins == 8 && kBinsPerLog2 == 8, "a lane's bins are one log2 unit: edges 2^-t x 2^(-q/8)");
  const int n = a.nseg2;
  const int j0 = kSelBins * lane;
  const float c = kLog2e / f.T;
  const float c8 = c * float(kBinsPerLog2);
  // the segment maxima and the row's (segment `lane` preloaded as p0)
  float m = -INFINITY;
  for (int q = lane; q < n; q += 64) {
    const Partial x = q == lane ? p0 : a.partials[row * n + q];
    sh.segm[q] = x.m;
    sh.segn[q] = x.idx;
    m = fmaxf(m, x.m);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __syncthreads();
  const float g = grid_point(m, c8);
  uint32_t cnt[kSelBins] = {};
  int64_t frac[kSelBins] = {};  // sums of (r - 1) 2^23: up to V x 759237
  const uint64_t* h64 = reinterpret_cast<const uint64_t*>(a.hcount) + row * n * kBins0;
  // Segments are taken kGather at a time: every lane loads all its bins of
  // them (clamped into each segment's stored bins, those out of range masked
  // afterwards) before adding any, so that the loads go out together.
  constexpr int kGather = 4;
  for (int s0 = 0; s0 < n; s0 += kGather) {
    uint64_t x[kGather][kSelBins];
    bool in[kGather][kSelBins];
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int s = min(s0 + u, n - 1);
      // cells between the row's grid point and the segment's; a segment
      // stored its bins 0 .. nbs - 1 (none without a finite logit)
      const float shc = g - grid_point(sh.segm[s], c8);
      const int jl = j0 - int(fminf(shc, float(kBins0)));
      const int nbs = s0 + u < n ? sh.segn[s] : 0;
#pragma unroll
      for (int q = 0; q < kSelBins; ++q) {
        const int jj = jl + q;
        in[u][q] = j0 + q < kBins0 - 1 && jj >= 0 && jj < nbs;
        x[u][q] = h64[size_t(s) * kBins0 + min(max(jj, 0), max(nbs - 1, 0))];
      }
    }
#pragma unroll
    for (int u = 0; u < kGather; ++u)
#pragma unroll
      for (int q = 0; q < kSelBins; ++q) {
        const uint32_t k = uint32_t(x[u][q] >> kCountShift0);
        const int64_t e = int64_t(x[u][q] & (kOne0 - 1)) - int64_t(k) * int64_t(kOneBits);
        cnt[q] += in[u][q] ? k : 0u;
        frac[q] += in[u][q] ? e : 0;
      }
  }
  // the last bin (lane 63's last) holds every element not in the others
  uint32_t lc = 0;
#pragma unroll
  for (int q = 0; q < kSelBins; ++q) lc += cnt[q];
  uint32_t in_bins;
  (void)wave_excl_scan<uint32_t>(lc, lane, &in_bins);
  if (lane == 63) cnt[kSelBins - 1] = uint32_t(a.V) - in_bins;
  // edge of bin 8t + q relative to the row maximum's weight: 2^(g/8 - m c) 2^-t 2^(-q/8)
  const double e0 = ldexp(exp2(double(g) * (1.0 / kBinsPerLog2) - double(m * c)), -lane);
  double mass[kSelBins];
  uint32_t tc = 0;
  double tm = 0.0;
#pragma unroll
  for (int q = 0; q < kSelBins; ++q) {
    mass[q] = j0 + q < kBins0 - 1 && cnt[q] > 0u
                  ? e0 * kPow2Eighth[q] * (double(cnt[q]) + double(frac[q]) / kFrac0)
                  : 0.0;
    tc += cnt[q];
    tm += mass[q];
  }
  uint32_t call;
  double S;
  uint32_t fc = wave_excl_scan<uint32_t>(tc, lane, &call);
  double fm = wave_excl_scan<double>(tm, lane, &S);
  const double tk = double(f.top_k);
  const double tp = double(f.top_p) * S;
  int first = kBins0, ck = -1, cp = -1;
  uint32_t fcq[kSelBins];
  double fmq[kSelBins];
#pragma unroll
  for (int q = 0; q < kSelBins; ++q) {
    fcq[q] = fc;
    fmq[q] = fm;
    if (cnt[q] > 0u) {
      first = min(first, j0 + q);
      if (f.on_k && double(fc) < tk) ck = j0 + q;
      if (f.on_p && fm < tp) cp = j0 + q;
    }
    fc += cnt[q];
    fm += mass[q];
  }
  const int top = -wave_max_int(-first);
  const int jk = wave_max_int(ck);
  const int jp = wave_max_int(cp);
  const int jq[2] = {jk >= 0 ? jk : top, jp >= 0 ? jp : top};
#pragma unroll
  for (int qq = 0; qq < 2; ++qq)
#pragma unroll
    for (int q = 0; q < kSelBins; ++q)
      if (j0 + q == jq[qq]) {
        sh.cab[qq] = fcq[q];
        sh.mab[qq] = fmq[q];
      }
  if (lane < 4) {
    // the boundary bin's key interval: two bisections per search, one lane each
    const int q = lane >> 1, side = lane & 1;
    const bool on = q == 0 ? f.on_k : f.on_p;
    if (on) {
      if (side == 0) sh.klo[q] = key_lo_of_bin<ET>(jq[q], c8, g);
      else sh.khi[q] = key_hi_of_bin<ET>(jq[q], c8, g);
    }
  }
  __syncthreads();
  if (lane < 2) {
    const int q = lane;
    const bool on = q == 0 ? f.on_k : f.on_p;
    FSearch w{};
    if (on) {
      w.lo = sh.klo[q];
      w.hi = sh.khi[q];
      w.cabove = sh.cab[q];
      w.mabove = sh.mab[q];
      w.target = q == 0 ? tk : tp;
      w.state = 1u;
    }
    a.search[row * 2 + q] = w;
  }
}

// Level-0 selection of a bf16 row from its key windows, by one wave: lane t
// holds the row's window keys km - (16t + i), i = 0..15 (km the row
// maximum's key), so that a prefix in lane order sums the larger keys.  A
// segment's counts shift into the row's window by the keys between its
// maximum's and the row's; they are merged in segment order.  A key's mass
// is its count times its weight (the same float expression as an element's
// weight), and the row's total mass is the sum of the segments' weight sums,
// each scaled from its maximum's weight to the row maximum's.  A search whose
// threshold is in the window is done here; otherwise (the window holds less
// than the target and the row has keys below it) it continues over the keys
// below the window, with the window's count and mass above.
template <typename ET>
__device__ void select0_window(const FiltArgs& a, const ReqFilter& f, size_t row, const Partial& p0, Sel0Shared& sh,
                               int lane) {
  constexpr int kPer = kWin / 64;
  const int n = a.nseg2;
  const float c = kLog2e / f.T;
  // the segment maxima, the row's, and the segments' weight sums relative
  // to their own maxima (segment `lane` preloaded as p0)
  float m = -INFINITY;
  for (int q = lane; q < n; q += 64) {
    const Partial x = q == lane ? p0 : a.partials[row * n + q];
    sh.segm[q] = x.m;
    sh.segn[q] = x.idx;
    sh.segt[q] = double(x.s) + double(x.cnt);
    m = fmaxf(m, x.m);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __syncthreads();
  const float mc = m * c;
  const uint32_t km = Key<ET>::of(m);
  double S = 0.0;
  for (int q = lane; q < n; q += 64)
    S += sh.segm[q] != -INFINITY ? sh.segt[q] * exp2(double(sh.segm[q] * c) - double(mc)) : 0.0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(a.hcount + row * n * (2 * kBins0));
  // the merge reads offsets 64 i + lane (each load a contiguous 128 bytes),
  // then hands each lane its 16 offsets through LDS
  uint32_t cm[kPer] = {};
  // segments kGather at a time, every load of them issued before any sum
  // (offsets outside a segment's stored counts load a stored one, masked)
  constexpr int kGather = 4;
  for (int s0 = 0; s0 < n; s0 += kGather) {
    uint32_t x[kGather][kPer];
    bool in[kGather][kPer];
#pragma unroll
    for (int u = 0; u < kGather; ++u) {
      const int sg = min(s0 + u, n - 1);
      const int shift = int(km - Key<ET>::of(sh.segm[sg]));
      const int nbs = s0 + u < n ? sh.segn[sg] : 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int ds = 64 * i + lane - shift;
        in[u][i] = ds >= 0 && ds < nbs;
        x[u][i] = h16[size_t(sg) * (4 * kBins0) + min(max(ds, 0), max(nbs - 1, 0))];
      }
    }
#pragma unroll
    for (int u = 0; u < kGather; ++u)
#pragma unroll
      for (int i = 0; i < kPer; ++i) cm[i] += in[u][i] ? x[u][i] : 0u;
  }
  // offset d at word d + d / 16: the lanes' runs of 16 start 17 words apart
#pragma unroll
  for (int i = 0; i < kPer; ++i) sh.win[68 * i + lane + (lane >> 4)] = cm[i];
  __syncthreads();
  uint32_t cnt[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) cnt[i] = sh.win[17 * lane + i];
  double mass[kPer];
  uint32_t tc = 0;
  double tm = 0.0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const float w = fast_exp2(fmaf(Key<ET>::value(km - uint32_t(kPer * lane + i)), c, -mc));
    mass[i] = cnt[i] > 0u ? double(cnt[i]) * double(w) : 0.0;
    tc += cnt[i];
    tm += mass[i];
  }
  uint32_t call;
  double mall;
  const uint32_t fc0 = wave_excl_scan<uint32_t>(tc, lane, &call);
  const double fm0 = wave_excl_scan<double>(tm, lane, &mall);
  const bool below = uint32_t(a.V) > call;  // the row has keys below the window
  bool any_open = false;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const bool on = q == 0 ? f.on_k : f.on_p;
    const double target = q == 0 ? double(f.top_k) : double(f.top_p) * S;
    // the smallest qualifying key (the largest offset; the maximum's key,
    // offset 0, if none qualifies)
    uint32_t fc = fc0;
    double fm = fm0;
    int dq = -1;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (cnt[i] > 0u && (q == 0 ? double(fc) < target : fm < target)) dq = kPer * lane + i;
      fc += cnt[i];
      fm += mass[i];
    }
    dq = max(wave_max_int(dq), 0);
    const bool open = below && (q == 0 ? double(call) < target : mall < target);
    FSearch w{};
    if (on && open) {
      w.lo = Key<ET>::kMin;
      w.hi = km - uint32_t(kWin);
      w.cabove = call;
      w.mabove = mall;
      w.target = target;
      w.state = kSearchCells;
      // the edge of the interval's top cell relative to the row maximum's weight
      w.mfinal = exp2(double(cell_of(Key<ET>::value(w.hi), c * float(kBinsPerLog2))) / kBinsPerLog2 - double(mc));
    }
    fc = fc0;
    fm = fm0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (on && !open && kPer * lane + i == dq) {
        w.lo = w.hi = w.key = km - uint32_t(dq);
        w.cabove = fc;
        w.mabove = fm;
        w.kept = fc + cnt[i];
        w.mfinal = fm + mass[i];
        w.target = target;
        w.state = 2u;
      }
      fc += cnt[i];
      fm += mass[i];
    }
    // the lane holding the threshold key writes a finished search, lane 0
    // an open or unused one
    const bool mine = on && !open ? (dq / kPer == lane) : lane == 0;
    if (mine) a.search[row * 2 + q] = w;
    any_open |= on && open;
  }
  // a row still searching lists its segments for the first key level
  if (any_open) {
    uint32_t base = 0;
    if (lane == 0)
      base = __hip_atomic_fetch_add(&a.wcount[kFirstList], uint32_t(n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    base = __shfl(base, 0, 64);
    uint32_t* list = a.work + size_t(a.B) * a.R * n;
    for (int q = lane; q < n; q += 64) list[base + q] = uint32_t(row * n + q);
  }
}

constexpr int kSelDigits = kBins / 64;  // key digits per lane of the selection

// Key-level selection of a row by one wave, in a kernel of its own (an fp32
// row's first key level); lane l owns digits kBins - 1 - (4l + k), k = 0..3,
// so that a prefix in lane order (and k order within a lane) sums the digits
// of larger keys.  The segment histograms are merged in segment order.
// Returns (in every lane) whether a search of the row is still open.
template <typename ET>
__device__ bool select_row(const FiltArgs& a, float c, float mc, size_t row, int lane) {
  const int n = a.nseg2;
  FSearch* st = a.search + row * 2;
  int more = 0;
#pragma unroll 1
  for (int q = 0; q < 2; ++q) {
    const FSearch cur = st[q];
    if (cur.state != 1u) continue;
    const uint32_t w = cur.hi - cur.lo;
    const int shf = w == 0u ? 0 : max(0, 32 - __clz(w) - 8);
    const int nd = int(w >> shf);  // the interval's last digit (no others are stored)
    uint32_t cd[kSelDigits] = {};
    uint64_t mfix[kSelDigits] = {};
    // segments kGather at a time, every load of them issued before any sum
    // (digits past the interval's last and segments past the row's load a
    // stored entry instead and are masked)
    constexpr int kGather = 4;
    auto gather = [&](auto wide_t) {
      constexpr bool wide = decltype(wide_t)::value;
      for (int s0 = 0; s0 < n; s0 += kGather) {
        uint32_t xc[kGather][kSelDigits];
        uint64_t xm[kGather][kSelDigits];
#pragma unroll
        for (int u = 0; u < kGather; ++u) {
          const size_t seg = row * n + min(s0 + u, n - 1);
#pragma unroll
          for (int k = 0; k < kSelDigits; ++k) {
            const int d = min(kBins - 1 - (kSelDigits * lane + k), nd);  // within the stored digits
            xc[u][k] = a.hcount[seg * 2 * kBins0 + q * kBins0 + d];
            if constexpr (wide) xm[u][k] = a.hmass[(seg * 2 + q) * kBins + d];
          }
        }
#pragma unroll
        for (int u = 0; u < kGather; ++u)
#pragma unroll
          for (int k = 0; k < kSelDigits; ++k) {
            const int d = kBins - 1 - (kSelDigits * lane + k);
            const bool in = s0 + u < n && d <= nd;
            cd[k] += in ? xc[u][k] : 0u;
            if constexpr (wide) mfix[k] += in ? xm[u][k] : 0ull;
          }
      }
    };
    // masses are stored only for digits wider than one key
    if (shf > 0) gather(std::true_type{});
    else gather(std::false_type{});
    double md[kSelDigits];
    uint32_t tc = 0;
    double tm = 0.0;
#pragma unroll
    for (int k = 0; k < kSelDigits; ++k) {
      const int d = kBins - 1 - (kSelDigits * lane + k);
      // a one-key digit's mass: its count times the weight of that key, the
      // same float expression as an element's weight
      md[k] = shf > 0 ? double(mfix[k]) / double(kFix)
                      : (cd[k] > 0u ? double(cd[k]) * double(fast_exp2(fmaf(Key<ET>::value(cur.lo + uint32_t(d)), c,
                                                                                -mc)))
                                    : 0.0);
      tc += cd[k];
      tm += md[k];
    }
    uint32_t call;
    double mall;
    uint32_t fc = cur.cabove + wave_excl_scan<uint32_t>(tc, lane, &call);
    double fm = cur.mabove + wave_excl_scan<double>(tm, lane, &mall);
    // the smallest qualifying digit (the largest non-empty one if none is)
    int dq = kBins, dtop = -1;
    uint32_t fck[kSelDigits];
    double fmk[kSelDigits];
#pragma unroll
    for (int k = 0; k < kSelDigits; ++k) {
      const int d = kBins - 1 - (kSelDigits * lane + k);
      fck[k] = fc;
      fmk[k] = fm;
      if (cd[k] > 0u) {
        if (q == 0 ? double(fc) < cur.target : fm < cur.target) dq = min(dq, d);
        dtop = max(dtop, d);
      }
      fc += cd[k];
      fm += md[k];
    }
    dq = -wave_max_int(-dq);
    dtop = wave_max_int(dtop);
    const int ds = dq < kBins ? dq : dtop;
    // the lane holding digit ds takes its figures out of the unrolled arrays,
    // then forms the digit's key range once
    int sd = -1;
    uint32_t sc = 0, scd = 0;
    double sm = 0.0, smd = 0.0;
#pragma unroll
    for (int k = 0; k < kSelDigits; ++k) {
      const int d = kBins - 1 - (kSelDigits * lane + k);
      if (d != ds) continue;
      sd = d;
      sc = fck[k];
      scd = cd[k];
      sm = fmk[k];
      smd = md[k];
    }
    int open = 0;
    if (sd >= 0) {
      FSearch nx = cur;
      const uint64_t lo = uint64_t(cur.lo) + (uint64_t(sd) << shf);
      const uint64_t hi = min(uint64_t(cur.hi), lo + (uint64_t(1) << shf) - 1);
      nx.lo = uint32_t(lo);
      nx.hi = uint32_t(hi);
      nx.mabove = sm;
      nx.cabove = sc;
      nx.state = 1u;
      if (lo == hi) {
        nx.state = 2u;
        nx.key = uint32_t(lo);
        nx.kept = sc + scd;
        nx.mfinal = sm + smd;
      } else {
        open = 1;
      }
      st[q] = nx;
    }
    more |= wave_max_int(open);
  }
  return more != 0;
}

// ---------------------------------------------------------------------------
// statistics and level 0
// ---------------------------------------------------------------------------

struct Stats0Shared {
  union {
    uint64_t bins[kBins0];  // count << 45 | sum of bits(r), by segment bin
    uint32_t win[kWin];     // bf16 rows: counts by key below the maximum's
  };
  double tot[kFT / 64];
  float red[kFT / 64];
  int lastb[kFT / 64];
  Partial part[kWaves];
};

// Maximum of a segment held as bf16 pairs: the high half of each word is
// compared as the word itself (the low half only adds bits below the bf16's
// precision, and a word whose high half is -inf reads as a NaN, which
// fmaxf passes over), the low half shifted up; the high halves' maximum is
// cleared of the low bits at the end.  fp32 elements are compared directly.
template <typename ET>
__device__ __forceinline__ float segment_max(const uint4 (&v)[kFV]) {
  if constexpr (Elem<ET>::N == 8) {
    float hi = -INFINITY, lo = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFV; ++k) {
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
        hi = fmaxf(hi, fmaxf(__uint_as_float(w[q]), __uint_as_float(w[q + 1])));
        lo = fmaxf(lo, fmaxf(__uint_as_float(w[q] << 16), __uint_as_float(w[q + 1] << 16)));
      }
    }
    return fmaxf(__uint_as_float(__float_as_uint(hi) & 0xffff0000u), lo);
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFV; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, Elem<ET>::get(v[k], j));
    return m;
  }
}

// One workgroup per 32 KiB segment of every row slot (draft rows, then
// target rows, of each request in turn).  Segments of a filtered row: the
// segment maximum and the level-0 histogram against the segment's own grid
// point, from one read.  Other rows read:
// the verification's statistics (lowest argmax for greedy target rows).  The
// segment holding a draft token also stores the logit there.
template <typename ET>
__global__ __launch_bounds__(kFT) __attribute__((amdgpu_waves_per_eu(8))) void filt_stats0_kernel(FiltArgs a) {
  __shared__ Stats0Shared sh;
  constexpr int N = Elem<ET>::N;
  constexpr int E = kFT * kFV * N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = a.nseg2, R = a.R, max_k = a.max_k;
  const uint32_t item = blockIdx.x;
  const int s = int(item % uint32_t(n));
  const int rs = int((item / uint32_t(n)) % uint32_t(R));
  const int b = int(item / (uint32_t(n) * uint32_t(R)));
  // every scalar the workgroup needs in one round trip, before any decision
  const ReqFilter f = req_filter(a, b);
  const bool is_draft = rs < max_k;
  const int i = is_draft ? rs : rs - max_k;
  const int64_t start = is_draft ? a.draft_start[b] : a.target_start[b];
  const int d = i < max_k ? a.tokens[size_t(b) * max_k + i] : -1;
  const bool greedy = !(f.T > 0.f);
  if (kKeyWindow<ET> && item == 0u && tid == 0) a.wcount[kFirstList] = 0u;  // no list before the selection
  if (is_draft ? (greedy || i >= f.K) : (i > f.K)) return;  // not read
  const float c = uniform(kLog2e / (greedy ? 1.f : f.T));
  const ET* row = is_draft ? static_cast<const ET*>(a.draft) + (start + i) * a.draft_stride
                           : static_cast<const ET*>(a.target) + (start + i) * a.target_stride;
  const bool ztok = !greedy && i < f.K && d >= s * E && d < (s + 1) * E && d < a.V;
  if (greedy) {
    stats_segment<ET, kArgmax>(a, sh.part, b, rs, s, false, c, row, d, tid);
    return;
  }
  if (!row_filtered(a, f, rs)) {
    stats_segment<ET, kSumInclusive>(a, sh.part, b, rs, s, ztok, c, row, d, tid);
    return;
  }
  const int hb = s * E;
  float zd = 0.f;
  if (ztok && tid == 0) zd = Elem<ET>::one(row + d);  // in flight with the segment
  uint4 v[kFV];
  load_seg<ET>(row, hb, a.V, v, tid);
  for (int j = tid; j < kBins0; j += kFT) sh.bins[j] = 0u;
  float m = segment_max<ET>(v);
  if (N == 8) fence_regs(v);  // the words, not their shifted halves, live on into the binning
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) sh.red[wv] = m;
  __syncthreads();
  m = fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
  const size_t row_slot = size_t(b) * R + rs;
  if (tid == 0 && ztok) a.zval[row_slot] = zd;
  if constexpr (kKeyWindow<ET>) {
    // the segment's statistics: its maximum, the sum of its weights
    // relative to the maximum's (s + cnt, two floats), and (in idx) how many
    // of its key counts, from the maximum's key down, are stored: up to the
    // last non-empty one
    int nb = 0;
    double tot = 0.0;
    if (m != -INFINITY) {  // uniform; the selection reads no count of a segment without a finite logit
      const uint32_t km = Key<ET>::of(m);
      const float mcs = m * c;
      static_assert(N == 8, "a bf16 vector's weights are summed pairwise");
#pragma unroll
      for (int k = 0; k < kFV; ++k) {
        if (hb + (k * kFT + tid) * N >= a.V) continue;  // past the end: nothing to count or weigh
        float w[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
          const float z = Elem<ET>::get(v[k], j);
          const uint32_t dd = key_offset16(km, z);
          if (dd < uint32_t(kWin)) atomicAdd(&sh.win[dd], 1u);
          w[j] = fast_exp2(fmaf(z, c, -mcs));
        }
        tot += double(((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7])));
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
      if (lane == 0) sh.tot[wv] = tot;
      __syncthreads();
      int last = -1;
      for (int j = tid; j < kWin; j += kFT)
        if (sh.win[j] != 0u) last = j;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
      if (lane == 0) sh.lastb[wv] = last;
      __syncthreads();
      nb = max(max(sh.lastb[0], sh.lastb[1]), max(sh.lastb[2], sh.lastb[3])) + 1;
      tot = ((sh.tot[0] + sh.tot[1]) + sh.tot[2]) + sh.tot[3];
      // stored as 16-bit counts (a segment's 2^14 tokens fit), two to a word
      uint32_t* h32 = a.hcount + (row_slot * n + s) * (2 * kBins0);
      for (int j = tid; 2 * j < nb; j += kFT) h32[j] = sh.win[2 * j] | (sh.win[2 * j + 1] << 16);
    }
    const float th = float(tot);
    if (tid == 0) a.partials[row_slot * n + s] = Partial{m, th, float(tot - double(th)), nb};
    return;
  }
  // the segment's statistics: its maximum, and (in idx) how many of its
  // bins, from bin 0, are stored: up to the last non-empty one below 511
  int nb = 0;
  if (m != -INFINITY) {  // uniform; the selection reads no bin of a segment without a finite logit
    const float c8 = c * float(kBinsPerLog2);
    const float gs = grid_point(m, c8), g8 = gs * (1.f / kBinsPerLog2);
    // r = 2^(z c - gs/8 + bin/8) in [1, 2^(1/8)) for bins below 511 (the
    // last bin is never read: there r is below 1, down to 0)
    // The bin is taken as its byte offset in sh.bins, 8 (gs - F(z)) clamped
    // to [0, 8 x 511] (bin0f's value times 8, exactly), so that it converts
    // straight to an LDS address.
    const float gs8 = gs * 8.f;
    auto add0 = [&](float z) {
      const float jb = __builtin_amdgcn_fmed3f(fmaf(cell_of(z, c8), -8.f, gs8), 0.f, float(8 * (kBins0 - 1)));
      const float r = fast_exp2(fmaf(jb, 1.f / (8 * kBinsPerLog2), fmaf(z, c, -g8)));
      atomicAdd(reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(sh.bins) + int(jb)),
                static_cast<unsigned long long>(kOne0 | __float_as_uint(r)));
    };
    // past the end of the row the loads hold -inf (bin 511, never read by
    // the selection): whole vectors of them are skipped, so that they do
    // not pile onto one LDS word
#pragma unroll
    for (int k = 0; k < kFV; ++k) {
      if (hb + (k * kFT + tid) * N >= a.V) continue;
#pragma unroll
      for (int j = 0; j < N; ++j) add0(Elem<ET>::get(v[k], j));
    }
    __syncthreads();
    int last = -1;
    for (int j = tid; j < kBins0 - 1; j += kFT)
      if (sh.bins[j] != 0u) last = j;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    if (lane == 0) sh.lastb[wv] = last;
    __syncthreads();
    nb = max(max(sh.lastb[0], sh.lastb[1]), max(sh.lastb[2], sh.lastb[3])) + 1;
    uint64_t* h64 = reinterpret_cast<uint64_t*>(a.hcount) + (row_slot * n + s) * kBins0;
    for (int j = tid; j < nb; j += kFT) h64[j] = sh.bins[j];
  }
  if (tid == 0) a.partials[row_slot * n + s] = Partial{m, 0.f, 0.f, nb};
}

// Level-0 selection: one wave per row slot.  Workgroup 0 also clears the
// counters of the later key levels' lists; a bf16 row also clears its
// arrival counter, which its first key level uses.
template <typename ET>
__global__ __launch_bounds__(64) void filt_select0_kernel(FiltArgs a) {
  __shared__ Sel0Shared sh;
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < kFirstList) a.wcount[tid] = 0u;
  const int R = a.R, n = a.nseg2;
  const int rs = int(blockIdx.x % uint32_t(R));
  const int b = int(blockIdx.x / uint32_t(R));
  const size_t row = size_t(b) * R + rs;
  // the row's first 64 segment statistics and the request's scalars in one round trip
  const Partial p0 = a.partials[row * n + min(tid, n - 1)];
  const ReqFilter f = req_filter(a, b);
  pin_all(f.K, f.T, f.top_k, f.top_p, p0.m, p0.idx);
  if (kKeyWindow<ET> && tid == 0) a.tickets[row] = 0u;  // the later levels' arrival counter
  if (!row_filtered(a, f, rs)) return;
  if constexpr (kKeyWindow<ET>) select0_window<ET>(a, f, row, p0, sh, tid);
  else select0_row<ET>(a, f, row, p0, sh, tid);
}

// ---------------------------------------------------------------------------
// key levels
// ---------------------------------------------------------------------------

struct HistShared {
  uint64_t mass[2][kBins];
  uint32_t count[2][kBins];
  uint32_t base;
  int last, more;
  // the workgroup selection's per-wave figures
  uint32_t wc[kFT / 64];
  double wm[kFT / 64];
  int wq[kFT / 64], wt[kFT / 64];
};

// Key-level selection of a row by a whole workgroup, the one that delivered
// the row's last segment histogram (the histograms read with device-scope
// loads): thread t owns digit kBins - 1 - t, so that a prefix in thread
// order (lanes, then waves) sums the digits of larger keys.  The rules are
// select_row's; one digit per thread keeps the pass's register budget, and
// with it its waves.  Returns (in every thread) whether a search of the row
// is still open.
template <typename ET>
__device__ bool select_row_wg(const FiltArgs& a, float c, float mc, size_t row, HistShared& sh, int tid) {
  static_assert(kFT == kBins, "one digit per thread");
  const int n = a.nseg2, lane = tid & 63, wv = tid >> 6;
  constexpr int kW = kFT / 64;
  FSearch* st = a.search + row * 2;
  int more = 0;
#pragma unroll 1
  for (int q = 0; q < 2; ++q) {
    const FSearch cur = st[q];
    if (cur.state != 1u && cur.state != kSearchCells) continue;
    const bool cells = kKeyWindow<ET> && cur.state == kSearchCells;
    const uint32_t w = cur.hi - cur.lo;
    const int shf = w == 0u ? 0 : max(0, 32 - __clz(w) - 8);
    const int nd = cells ? kBins - 1 : int(w >> shf);
    const bool wide = cells || shf > 0;
    const int d = kBins - 1 - tid;
    uint32_t cd = 0;
    uint64_t mfix = 0;  // fixed-point mass; weight cells: sum of (r - 1) 2^23
    if (d <= nd) {
      constexpr int kGather = 4;
      for (int s0 = 0; s0 < n; s0 += kGather) {
        uint32_t xc[kGather];
        uint64_t xm[kGather];
#pragma unroll
        for (int u = 0; u < kGather; ++u) {
          const size_t seg = row * n + min(s0 + u, n - 1);
          xc[u] = load_dev32(&a.hcount[seg * 2 * kBins0 + q * kBins0 + d]);
          xm[u] = wide ? load_dev64(&a.hmass[(seg * 2 + q) * kBins + d]) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kGather; ++u) {
          const bool in = s0 + u < n;
          cd += in ? xc[u] : 0u;
          mfix += in ? (cells ? (xm[u] & (kOne0 - 1)) - uint64_t(xc[u]) * kOneBits : xm[u]) : 0ull;
        }
      }
    }
    double md = 0.0;
    if (cd > 0u) {
      if (cells) {
        const int j = kBins - 1 - d;
        const double ce = cur.mfinal;  // the top cell's edge
        md = d > 0 ? ldexp(ce * kPow2Eighth[j & 7], -(j >> 3)) * (double(cd) + double(int64_t(mfix)) / kFrac0)
                   : 0.0;
      } else if (wide) {
        md = double(mfix) / double(kFix);
      } else {
        // a one-key digit: its count times that key's weight (an element's expression)
        md = double(cd) * double(fast_exp2(fmaf(Key<ET>::value(cur.lo + uint32_t(d)), c, -mc)));
      }
    }
    // exclusive prefix in thread order: within the wave, then the waves before
    uint32_t wct;
    double wmt;
    const uint32_t pc = wave_excl_scan<uint32_t>(cd, lane, &wct);
    const double pm = wave_excl_scan<double>(md, lane, &wmt);
    if (lane == 0) {
      sh.wc[wv] = wct;
      sh.wm[wv] = wmt;
    }
    __syncthreads();
    uint32_t fc = cur.cabove;
    double fm = cur.mabove;
    for (int u = 0; u < wv; ++u) {
      fc += sh.wc[u];
      fm += sh.wm[u];
    }
    fc += pc;
    fm += pm;
    // the smallest qualifying digit (the largest non-empty one if none is)
    const bool qual = cd > 0u && (q == 0 ? double(fc) < cur.target : fm < cur.target);
    int dq = -wave_max_int(qual ? -d : -kBins);
    int dt = wave_max_int(cd > 0u ? d : -1);
    if (lane == 0) {
      sh.wq[wv] = dq;
      sh.wt[wv] = dt;
    }
    __syncthreads();
    for (int u = 0; u < kW; ++u) {
      dq = min(dq, sh.wq[u]);
      dt = max(dt, sh.wt[u]);
    }
    const int ds = dq < kBins ? dq : dt;
    if (d == ds) {
      FSearch nx = cur;
      uint64_t lo, hi;
      if (cells) {
        const float c8 = c * float(kBinsPerLog2);
        const float g = cell_of(Key<ET>::value(cur.hi), c8);
        const int j = kBins - 1 - d;  // the level-0 bin against g
        lo = j == kBins - 1 ? uint64_t(cur.lo) : max(uint64_t(cur.lo), uint64_t(key_lo_of_bin<ET>(j, c8, g)));
        hi = min(uint64_t(cur.hi), uint64_t(key_hi_of_bin<ET>(j, c8, g)));
      } else {
        lo = uint64_t(cur.lo) + (uint64_t(d) << shf);
        hi = min(uint64_t(cur.hi), lo + (uint64_t(1) << shf) - 1);
      }
      nx.lo = uint32_t(lo);
      nx.hi = uint32_t(hi);
      nx.mabove = fm;
      nx.cabove = fc;
      nx.state = 1u;
      if (lo == hi) {
        nx.state = 2u;
        nx.key = uint32_t(lo);
        nx.kept = fc + cd;
        // (a weight cell's mass by its one key's weight: digit 0 has none)
        nx.mfinal = fm + (cells ? double(cd) * double(fast_exp2(fmaf(Key<ET>::value(uint32_t(lo)), c, -mc))) : md);
      } else {
        sh.more = 1;
      }
      st[q] = nx;
    }
    __syncthreads();
  }
  more = sh.more;
  return more != 0;
}

// The segments of a row still searching after key level `level` are listed
// for the next level, if there is one.
__device__ __forceinline__ void list_row(const FiltArgs& a, size_t row, int level, int levels, uint32_t* base,
                                         int tid) {
  if (level >= levels) return;
  const int n = a.nseg2;
  const int nxt = level - 1;  // list and counter of level + 1
  if (tid == 0) *base = __hip_atomic_fetch_add(&a.wcount[nxt], uint32_t(n), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  uint32_t* list = a.work + size_t(nxt & 1) * (size_t(a.B) * a.R * n);
  for (int q = tid; q < n; q += kFT) list[*base + q] = uint32_t(row * n + q);
}

// One key-level pass over segment s of row slot rs of request b: per
// searching slot, the elements of its key interval by key digit: counts,
// and 2^-40 fixed-point masses when a digit spans several keys (a single
// key's mass is its count times its weight), or by weight cells.  At an fp32
// row's first key level they are stored for the selection kernel; otherwise
// (LATER) they are published for the row's selection, which the row's last
// arriving segment workgroup then makes, listing the row for the next level
// if it still searches.
template <typename ET, bool LATER>
__device__ void keys_segment(const FiltArgs& a, int b, int rs, int s, int level, int levels, HistShared& sh,
                             int tid) {
  constexpr int N = Elem<ET>::N;
  const int lane = tid & 63;
  const int n = a.nseg2, R = a.R;
  const size_t row = size_t(b) * R + rs;
  // every scalar the workgroup needs in one round trip, before any decision
  const ReqFilter f = req_filter(a, b);
  const bool is_draft = rs < a.max_k;
  const int64_t start = is_draft ? a.draft_start[b] : a.target_start[b];
  uint32_t st_state[2], lo[2], hi[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const FSearch& st = a.search[row * 2 + q];
    st_state[q] = st.state;
    lo[q] = st.lo;
    hi[q] = st.hi;
  }
  if (!row_filtered(a, f, rs)) return;
  bool on[2], cells[2];
  int shift[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    on[q] = st_state[q] == 1u || st_state[q] == kSearchCells;
    cells[q] = st_state[q] == kSearchCells;
    const uint32_t w = hi[q] - lo[q];
    shift[q] = w == 0u ? 0 : max(0, 32 - __clz(w) - 8);
  }
  // a listed row searches; at the first key level, the rows whose level-0
  // selection left a search open (fp32 rows: every one; bf16 rows: those
  // whose threshold is below the key window)
  if (!LATER && !(on[0] || on[1])) return;
  const ET* rp = is_draft ? static_cast<const ET*>(a.draft) + (start + rs) * a.draft_stride
                          : static_cast<const ET*>(a.target) + (start + (rs - a.max_k)) * a.target_stride;
  const bool al = is_aligned16(rp);
  const int hb = s * kFT * kFV * N;
  const bool full = hb + kFT * kFV * N <= a.V;
  uint4 v[kFV];
  if (al && full) {
#pragma unroll
    for (int k = 0; k < kFV; ++k) v[k] = load_stream16(rp + hb + (k * kFT + tid) * N);
  } else {
#pragma unroll
    for (int k = 0; k < kFV; ++k) v[k] = load_nan_tail<ET>(rp, hb + (k * kFT + tid) * N, a.V, al);
  }
  const float c = kLog2e / f.T;
  const float mc = wave_row_max(a.partials + row * n, n, lane) * c;
  const float c8 = c * float(kBinsPerLog2);
  float gc[2];  // a weight-cell search: the cell of the interval's top value
#pragma unroll
  for (int q = 0; q < 2; ++q) gc[q] = cells[q] ? cell_of(Key<ET>::value(hi[q]), c8) : 0.f;
  for (int j = tid; j < 2 * kBins; j += kFT) {
    (&sh.count[0][0])[j] = 0u;
    (&sh.mass[0][0])[j] = 0u;
  }
  // a slot's key interval as a value interval (the key order is the value
  // order, -0 and +0 one value): two compares dismiss an element; past the
  // end of the row the tail loads hold NaN, which no interval holds
  float zlo[2], zhi[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    zlo[q] = on[q] ? Key<ET>::value(lo[q]) : INFINITY;
    zhi[q] = on[q] ? Key<ET>::value(hi[q]) : INFINITY;
  }
  __syncthreads();
  // per element a test against each searching slot's value interval; the
  // common case of one search gets a loop of its own
  auto digit_add = [&](int q, float z, auto cells_t) {
    if constexpr (decltype(cells_t)::value) {
      const float j = gc[q] - cell_of(z, c8);
      const bool deep = !(j < float(kBins - 1));  // digit 0 (also -inf)
      const float r = deep ? 1.f : fast_exp2(fmaf(j, 1.f / kBinsPerLog2, fmaf(z, c, gc[q] * (-1.f / kBinsPerLog2))));
      atomicAdd(reinterpret_cast<unsigned long long*>(&sh.mass[q][deep ? 0 : kBins - 1 - int(j)]),
                static_cast<unsigned long long>(kOne0 | __float_as_uint(r)));
    } else {
      const int dg = int((Key<ET>::of(z) - lo[q]) >> shift[q]);
      atomicAdd(&sh.count[q][dg], 1u);
      if (shift[q] > 0)
        atomicAdd(reinterpret_cast<unsigned long long*>(&sh.mass[q][dg]),
                  static_cast<unsigned long long>(fixed_mass(z, c, mc)));
    }
  };
  auto one_search = [&](int q, auto cells_t) {
    const float l = zlo[q], h = zhi[q];
#pragma unroll
    for (int k = 0; k < kFV; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float z = Elem<ET>::get(v[k], j);
        if (z >= l && z <= h) digit_add(q, z, cells_t);
      }
  };
  // Weight cells are only a bf16 row's first key level, where every open
  // search of the row has them over the same interval (the keys below the
  // window): one histogram serves both.
  const int q1 = on[0] ? 0 : 1;
  if (kKeyWindow<ET> && cells[q1]) {
    one_search(q1, std::true_type{});
  } else if (on[0] && on[1]) {
#pragma unroll
    for (int k = 0; k < kFV; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float z = Elem<ET>::get(v[k], j);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (z >= zlo[q] && z <= zhi[q]) digit_add(q, z, std::false_type{});
      }
  } else {
    one_search(q1, std::false_type{});
  }
  __syncthreads();
  // only the interval's digits are stored: the digits below ((hi - lo) >> shift) + 1
  const size_t seg = row * n + s;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (!on[q] || tid > (cells[q] ? kBins - 1 : int((hi[q] - lo[q]) >> shift[q]))) continue;
    const bool wide = cells[q] || shift[q] > 0;
    const int hq = cells[q] ? q1 : q;  // a weight-cell histogram was built once
    const uint64_t mw = sh.mass[hq][tid];
    const uint32_t cw = cells[q] ? uint32_t(mw >> kCountShift0) : sh.count[hq][tid];
    if (LATER) {
      if (wide) store_dev64(&a.hmass[(seg * 2 + q) * kBins + tid], mw);
      store_dev(&a.hcount[seg * 2 * kBins0 + q * kBins0 + tid], cw);
    } else {
      if (wide) a.hmass[(seg * 2 + q) * kBins + tid] = mw;
      a.hcount[seg * 2 * kBins0 + q * kBins0 + tid] = cw;
    }
  }
  if (!LATER) return;
  if (!arrive_last_all(&a.tickets[row], uint32_t(n), &sh.last)) return;
  if (tid == 0) sh.more = 0;
  __syncthreads();
  if (select_row_wg<ET>(a, c, mc, row, sh, tid)) list_row(a, row, level, levels, &sh.base, tid);
  if (tid == 0) store_dev(&a.tickets[row], 0u);
}

// The first key level.  fp32: one workgroup per 32 KiB segment of every row
// slot, its selection a kernel of its own.  bf16: the segments listed by the
// level-0 selection, in list order, each row's selection made by its last
// arriving segment workgroup as at the later levels.
template <typename ET>
__global__ __launch_bounds__(kFT) void filt_keys_first_kernel(FiltArgs a, int levels) {
  __shared__ HistShared sh;
  const int n = a.nseg2, R = a.R;
  if constexpr (kKeyWindow<ET>) {
    const uint32_t count = a.wcount[kFirstList];
    const uint32_t* list = a.work + size_t(a.B) * R * n;
    for (uint32_t e = blockIdx.x; e < count; e += gridDim.x) {
      const uint32_t item = list[e];
      const int s = int(item % uint32_t(n));
      const int rs = int((item / uint32_t(n)) % uint32_t(R));
      const int b = int(item / (uint32_t(n) * uint32_t(R)));
      keys_segment<ET, true>(a, b, rs, s, 1, levels, sh, threadIdx.x);
      __syncthreads();  // the shared arrays are reused by the next segment
    }
  } else {
    const uint32_t item = blockIdx.x;
    const int s = int(item % uint32_t(n));
    const int rs = int((item / uint32_t(n)) % uint32_t(R));
    const int b = int(item / (uint32_t(n) * uint32_t(R)));
    keys_segment<ET, false>(a, b, rs, s, 1, 1, sh, threadIdx.x);
  }
}

// Selection of an fp32 row's first key level: one wave per row slot; a row
// still searching is listed for the second.  Also clears the row's arrival
// counter, used by the later levels.
template <typename ET>
__global__ __launch_bounds__(64) void filt_select_kernel(FiltArgs a, int levels) {
  __shared__ uint32_t base;
  const int tid = threadIdx.x;
  const int R = a.R;
  const int rs = int(blockIdx.x % uint32_t(R));
  const int b = int(blockIdx.x / uint32_t(R));
  const size_t row = size_t(b) * R + rs;
  const int n = a.nseg2;
  if (tid == 0) a.tickets[row] = 0u;
  // the row's segment maxima (the first 64), its search states and the
  // request's scalars in one round trip
  float m = a.partials[row * n + min(tid, n - 1)].m;
  const uint32_t s0 = a.search[row * 2].state, s1 = a.search[row * 2 + 1].state;
  const ReqFilter f = req_filter(a, b);
  pin_all(m, s0, s1, f.K, f.T, f.top_k, f.top_p);
  if (!row_filtered(a, f, rs) || (s0 != 1u && s1 != 1u)) return;
  for (int q = tid + 64; q < n; q += 64) m = fmaxf(m, a.partials[row * n + q].m);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float c = kLog2e / f.T;
  if (select_row<ET>(a, c, m * c, row, tid)) list_row(a, row, 1, levels, &base, tid);
}

// Later key levels: the segments listed by the previous level's selections,
// taken in list order by a grid of workgroups (most levels list none).
template <typename ET>
__global__ __launch_bounds__(kFT) void filt_keys_next_kernel(FiltArgs a, int level, int levels) {
  __shared__ HistShared sh;
  const int n = a.nseg2, R = a.R;
  const uint32_t count = a.wcount[level - 2];
  const uint32_t* list = a.work + size_t(level & 1) * (size_t(a.B) * R * n);
  for (uint32_t e = blockIdx.x; e < count; e += gridDim.x) {
    const uint32_t item = list[e];
    const int s = int(item % uint32_t(n));
    const int rs = int((item / uint32_t(n)) % uint32_t(R));
    const int b = int(item / (uint32_t(n) * uint32_t(R)));
    keys_segment<ET, true>(a, b, rs, s, level, levels, sh, threadIdx.x);
    __syncthreads();  // the shared arrays are reused by the next segment
  }
}

// ---------------------------------------------------------------------------
// verdict and draw
// ---------------------------------------------------------------------------
//
// Three kernels, as the unfiltered path: the verdict (one wave per request:
// row normalisers and thresholds, accept walk, outputs), the draw weights
// (one workgroup per 32 KiB segment of the draw rows: the weights of its 8
// slices of 4 KiB, for the residual and for the target row alone, the
// fallback when the residual has no mass), and the search (one workgroup per
// request: the slice sums scanned in token order, then the crossing slice).

struct RowInfo {
  float kk;    // log2 normaliser: p'(v) = exp2(z c - kk) for kept v
  uint32_t t;  // threshold key (0: every token kept)
  int idx;     // lowest-index argmax (greedy target rows)
  int pad;
};

static_assert(sizeof(RowInfo) == kFilterRowBytes, "row info layout");

struct DrawDesc {
  int acc;    // accept length
  int mode;   // 0: greedy (token emitted), 1: residual at acc, 2: bonus from target row acc
  float u;
  int pad;
};

static_assert(sizeof(DrawDesc) == kFilterDescBytes, "draw descriptor layout");
static_assert(kFV == kDrawSlices, "slices per draw segment");
constexpr int kMaxSlices = int(int64_t(SV_MAX_V) * 4 / (kFT * 16));  // 4 KiB slices of the longest row

template <typename ET>
__global__ __launch_bounds__(64) void filt_verdict_kernel(FiltArgs a, RowInfo* info, DrawDesc* desc) {
  __shared__ RowInfo row[2 * SV_MAX_K + 1];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int max_k = a.max_k, R = a.R, n = a.nseg2;
  const ReqFilter f = req_filter(a, b);
  const int K = f.K;
  const bool greedy = !(f.T > 0.f);
  const float c = kLog2e / (greedy ? 1.f : f.T);
  // lane i's position (i < max_k): token, logits at it, uniform, fetched now
  // so that they arrive with the rows' statistics
  const size_t o = size_t(b) * max_k + min(tid, max(max_k - 1, 0));
  int d = 0;
  float zd = 0.f, zt = 0.f, ua = 1.f;
  if (tid < max_k) {
    d = a.tokens[o];
    zd = a.zval[size_t(b) * R + tid];
    zt = a.zval[size_t(b) * R + max_k + tid];
    ua = a.u_accept[o];
  }
  if (tid < R) {
    const int rs = tid;
    const bool valid = rs < max_k ? (rs < K && !greedy) : (rs - max_k <= K);
    RowInfo r{0.f, 0u, 0, 0};
    int kept = -1;
    if (valid) {
      // the row's segment statistics, eight at a time, every load of them
      // issued before any merge
      const Partial* p = a.partials + (size_t(b) * R + rs) * n;
      float m = -INFINITY, sum = 0.f, cnt = 0.f;
      int idx = 0x7fffffff;
      for (int s0 = 0; s0 < n; s0 += 8) {
        Partial x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = p[min(s0 + u, n - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (s0 + u >= n) break;
          if (greedy) merge_argmax(m, idx, x[u].m, x[u].idx);
          else merge_ms(m, sum, cnt, x[u].m, x[u].s + x[u].cnt, 0.f, c);
        }
      }
      if (greedy) {
        r.idx = idx;
      } else {
        const float mc = m * c;
        r.kk = mc + fast_log2(sum);
        if (row_filtered(a, f, rs)) {
          const FSearch* st = a.search + (size_t(b) * R + rs) * 2;
          const FSearch& sk = st[0];
          const FSearch& sp = st[1];
          const FSearch& use = !f.on_k ? sp : !f.on_p ? sk : (sk.key >= sp.key ? sk : sp);
          r.t = use.key;
          r.kk = mc + fast_log2(float(use.mfinal));
          kept = int(use.kept);
        }
      }
    }
    row[rs] = r;
    info[size_t(b) * R + rs] = r;
    if (a.kept) a.kept[size_t(b) * R + rs] = kept;
  }
  __syncthreads();
  // the accept tests, one position per lane; the accept length is the first
  // rejection (K_b if none)
  const int i = tid;
  float pd = NAN, pt = NAN;
  bool ok = true;
  if (i < K) {
    if (greedy) {
      ok = d == row[max_k + i].idx;
      pt = ok ? 1.f : 0.f;
    } else {
      const RowInfo& id = row[i];
      const RowInfo& it = row[max_k + i];
      const uint32_t kd = Key<ET>::of(zd), kt = Key<ET>::of(zt);
      const float ld = kd >= id.t ? fmaf(zd, c, -id.kk) : -INFINITY;
      const float lt = kt >= it.t ? fmaf(zt, c, -it.kk) : -INFINITY;
      pd = fast_exp2(ld);
      pt = fast_exp2(lt);
      const float ratio = ld == -INFINITY ? INFINITY : fast_exp2(lt - ld);
      ok = ua < fminf(1.f, ratio);
    }
  }
  const unsigned long long rej = __ballot(i < K && !ok);
  const int acc = rej ? __ffsll(static_cast<long long>(rej)) - 1 : K;
  if (i < max_k) {
    if (a.p_draft) a.p_draft[o] = pd;
    if (a.p_target) a.p_target[o] = pt;
    if (a.labels) a.labels[o] = int8_t(i < acc ? 1 : (i == acc && i < K ? 0 : -1));
  }
  if (i <= max_k) a.out_tokens[size_t(b) * (max_k + 1) + i] = i < acc ? d : -1;
  if (tid != 0) return;
  a.accept_len[b] = acc;
  DrawDesc dd{acc, 0, 0.f, 0};
  if (greedy) {
    a.out_tokens[size_t(b) * (max_k + 1) + acc] = row[max_k + acc].idx;
  } else {
    dd.mode = acc < K ? 1 : 2;
    dd.u = acc < K ? a.u_residual[b] : a.u_bonus[b];
  }
  desc[b] = dd;
}

// A row's kept set {key(z) >= t} as a value test z >= value(t): the key
// order is the value order (-0 and +0 one value), so the two agree on every
// non-NaN logit, and the compare is one instruction.
struct KeptRow {
  float zt;  // value(t)
  float kk;  // log2 of the normaliser
};
template <typename ET>
__device__ __forceinline__ KeptRow kept_row(const RowInfo& r) {
  // keys up to kMin (-inf; below it only NaN patterns, 0 for an unfiltered
  // row) keep every logit
  return KeptRow{r.t <= Key<ET>::kMin ? -INFINITY : Key<ET>::value(r.t), r.kk};
}

// Weight of one element pair: (pt' - pd')+ (residual) or pt'.
__device__ __forceinline__ void pair_w(float zt, float zd, const KeptRow& it, const KeptRow& id, float c, bool resid,
                                       float* wr, float* wt) {
  const float x = zt >= it.zt ? fast_exp2(fmaf(zt, c, -it.kk)) : 0.f;
  *wt = x;
  if (resid) {
    const float y = zd >= id.zt ? fast_exp2(fmaf(zd, c, -id.kk)) : 0.f;
    *wr = fmaxf(x - y, 0.f);
  } else {
    *wr = x;
  }
}

// Slice sums of one segment of the draw rows into red (residual and target
// weights), read in two halves of kFV / 2 vectors so that a workgroup holds
// 16 KiB of each row at a time.  Elements past the end of the row load as
// -inf and weigh 0.
template <typename ET, bool RESID>
__device__ __forceinline__ void weight_slices(const ET* rt, const ET* rd, int hb, int V, bool full, bool al,
                                              const KeptRow& it, const KeptRow& id, float c,
                                              float (*red)[kFV][kFT / 64], int tid) {
  constexpr int N = Elem<ET>::N;
  constexpr int H = kFV / 2;
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    uint4 vt[H], vd[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const int e0 = hb + ((h * H + k) * kFT + tid) * N;
      vt[k] = full ? load_stream16(rt + e0) : load_raw<ET>(rt, e0, V, al);
      if (RESID) vd[k] = full ? load_stream16(rd + e0) : load_raw<ET>(rd, e0, V, al);
    }
#pragma unroll
    for (int k = 0; k < H; ++k) {
      float sr = 0.f, st = 0.f;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        float wr, wt;
        const float zt = Elem<ET>::get(vt[k], j);
        pair_w(zt, RESID ? Elem<ET>::get(vd[k], j) : zt, it, id, c, RESID, &wr, &wt);
        sr += wr;
        st += wt;
      }
      sr = wave_sum(sr);
      st = wave_sum(st);
      if (lane == 0) {
        red[0][h * H + k][wv] = sr;
        red[1][h * H + k][wv] = st;
      }
    }
  }
}

// Draw weights: workgroup (b, s) sums its 32 KiB segment of the draw rows per
// slice (slice k = vector k of every thread: 4 KiB of contiguous tokens).
template <typename ET>
__global__ __launch_bounds__(kFT) void filt_weight_kernel(FiltArgs a, const RowInfo* info, const DrawDesc* desc,
                                                          float* slices) {
  __shared__ float red[2][kFV][kFT / 64];
  constexpr int N = Elem<ET>::N;
  const int tid = threadIdx.x;
  const int n = a.nseg2;
  const int b = int(blockIdx.x / uint32_t(n)), s = int(blockIdx.x % uint32_t(n));
  // the request's scalars in one round trip, then the rows
  const DrawDesc dd = desc[b];
  const int64_t ds = a.draft_start[b], ts = a.target_start[b];
  const float T = a.temperature[b];
  if (dd.mode == 0) return;
  const bool resid = dd.mode == 1;
  const int R = a.R, max_k = a.max_k;
  const ET* rt = static_cast<const ET*>(a.target) + (ts + dd.acc) * a.target_stride;
  const ET* rd = resid ? static_cast<const ET*>(a.draft) + (ds + dd.acc) * a.draft_stride : rt;
  const bool al = is_aligned16(rt) && is_aligned16(rd);
  const int hb = s * kFT * kFV * N;
  const bool full = al && hb + kFT * kFV * N <= a.V;
  const float c = kLog2e / T;
  const KeptRow it = kept_row<ET>(info[size_t(b) * R + max_k + dd.acc]);
  const KeptRow id = resid ? kept_row<ET>(info[size_t(b) * R + dd.acc]) : it;
  if (resid)
    weight_slices<ET, true>(rt, rd, hb, a.V, full, al, it, id, c, red, tid);
  else
    weight_slices<ET, false>(rt, rd, hb, a.V, full, al, it, id, c, red, tid);
  __syncthreads();
  if (tid < 2 * kFV) {
    const int q = tid / kFV, k = tid % kFV;
    float x = 0.f;
    for (int w = 0; w < kFT / 64; ++w) x += red[q][k][w];
    slices[((size_t(b) * n + s) * 2 + q) * kFV + k] = x;
  }
}

__device__ __forceinline__ int ft_max_int(int x, int* part, int tid) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  if ((tid & 63) == 0) part[tid >> 6] = x;
  __syncthreads();
  int m = part[0];
  for (int q = 1; q < kFT / 64; ++q) m = max(m, part[q]);
  __syncthreads();
  return m;
}

// The draw: running sums of the slice weights in token order locate the slice
// where u Z is crossed, a scan of that slice the token.  If rounding leaves
// no crossing, the last positive-weight token (of the row, or of the slice).
template <typename ET>
__global__ __launch_bounds__(kFT) void filt_search_kernel(FiltArgs a, const RowInfo* info, const DrawDesc* desc,
                                                          const float* slices) {
  __shared__ float part[kFT / 64];
  __shared__ int ip[kFT / 64];
  __shared__ int pick, last, mode;
  __shared__ float rem;
  __shared__ float sw[2][kMaxSlices];
  constexpr int N = Elem<ET>::N;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x, n = a.nseg2;
  const DrawDesc dd = desc[b];
  if (dd.mode == 0) return;
  const int ns = n * kFV;  // slices of a row
  const int R = a.R, max_k = a.max_k;
  // everything the draw needs besides the crossing slice, in one round trip:
  // the slice weights (slice j = (segment j / kFV, vector j % kFV); its
  // weights of kind q sit at ((j / kFV) * 2 + q) * kFV + j % kFV of the
  // request's block), both candidate rows' thresholds and starts, T
  const float* sl = slices + size_t(b) * n * 2 * kFV;
  for (int e = tid; e < 2 * ns; e += kFT) {
    const int seg = e / (2 * kFV), q = (e / kFV) & 1, k = e % kFV;
    sw[q][seg * kFV + k] = sl[e];
  }
  const RowInfo it = info[size_t(b) * R + max_k + dd.acc];
  const RowInfo idr = info[size_t(b) * R + dd.acc];
  const ET* rt = row_ptr<ET>(a, b, max_k + dd.acc);
  const ET* rdr = row_ptr<ET>(a, b, dd.acc);
  const float c = kLog2e / a.temperature[b];
  __syncthreads();
  if (wv == 0) {
    // wave 0: lane l sums slices l * per .. in order, a prefix over the
    // lanes places each lane's run; the crossing lane scans its run
    const int per = (ns + 63) / 64;
    const int j0 = min(lane * per, ns), j1 = min(j0 + per, ns);
    int q = dd.mode == 1 ? 0 : 1;
    auto lane_sum = [&](int qq) {
      float x = 0.f;
      for (int j = j0; j < j1; ++j) x += sw[qq][j];
      return x;
    };
    float ls = lane_sum(q);
    float incl = wave_inclusive_scan(ls, lane);
    float Z = __shfl(incl, 63, 64);
    if (q == 0 && !(Z > 0.f)) {  // the residual has no mass: draw from the target row
      q = 1;
      ls = lane_sum(q);
      incl = wave_inclusive_scan(ls, lane);
      Z = __shfl(incl, 63, 64);
    }
    const float t = dd.u * Z;
    float before = __shfl_up(incl, 1, 64);  // weight of the slices ahead of this lane's run
    if (lane == 0) before = 0.f;
    const unsigned long long hit = __ballot(incl > t && j1 > j0);
    int ch = -1, want_last = 0;
    float cum = 0.f;
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      if (lane == l) {
        // the crossing slice of the run; if rounding leaves none there, the
        // run's last slice with positive weight
        cum = before;
        int lastj = -1;
        float cum_last = before;
        for (int j = j0; j < j1; ++j) {
          const float w = sw[q][j];
          if (w > 0.f) {
            lastj = j;
            cum_last = cum;
          }
          if (cum + w > t) {
            ch = j;
            break;
          }
          cum += w;
        }
        if (ch < 0) {
          ch = max(lastj, j0);
          cum = cum_last;
        }
      }
      ch = __shfl(ch, l, 64);
      cum = __shfl(cum, l, 64);
    }
    if (ch < 0) {
      // rounding left no crossing: the last slice with positive weight
      want_last = 1;
      int lastp = -1;
      for (int j = j0; j < j1; ++j)
        if (sw[q][j] > 0.f) lastp = j;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) lastp = max(lastp, __shfl_xor(lastp, o, 64));
      ch = max(lastp, 0);
      cum = t;
    }
    if (lane == 0) {
      pick = ch;
      last = want_last;
      mode = q;
      rem = t - cum;
    }
  }
  __syncthreads();
  const int ch = pick;
  const bool resid = mode == 0;
  const RowInfo id = resid ? idr : it;
  const KeptRow kit = kept_row<ET>(it), kid = kept_row<ET>(id);
  const ET* rd = resid ? rdr : rt;
  const bool al = is_aligned16(rt) && is_aligned16(rd);
  // the slice: kFT * N contiguous tokens, thread t holding N of them
  const int first = (ch / kFV) * kFT * kFV * N + (ch % kFV) * kFT * N + tid * N;
  const uint4 vt = load_raw<ET>(rt, first, a.V, al);
  const uint4 vd = resid ? load_raw<ET>(rd, first, a.V, al) : vt;
  float w[N];
  float own = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float wr, wt;
    pair_w(Elem<ET>::get(vt, j), Elem<ET>::get(vd, j), kit, kid, c, resid, &wr, &wt);
    w[j] = first + j < a.V ? wr : 0.f;
    own += w[j];
  }
  float incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) part[wv] = incl;
  __syncthreads();
  float run = incl - own;
  for (int q = 0; q < wv; ++q) run += part[q];
  int fst = 0x7fffffff, lastpos = -1;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    run += w[j];
    if (w[j] > 0.f) {
      lastpos = first + j;
      if (fst == 0x7fffffff && run > rem) fst = first + j;
    }
  }
  const int fmin = -ft_max_int(-fst, ip, tid);
  const int lmax = ft_max_int(lastpos, ip, tid);
  if (tid == 0) a.out_tokens[size_t(b) * (max_k + 1) + dd.acc] = (!last && fmin != 0x7fffffff) ? fmin : lmax;
}

}  // namespace

hipError_t launch_filtered(VerifyArgs va, const FilterIO& io, int dtype, hipStream_t stream) {
  const uint64_t n1 = uint64_t(va.B) * uint64_t(va.R) * uint64_t(va.nseg2);
  if (n1 >= (uint64_t(1) << 31)) return hipErrorInvalidValue;
  FiltArgs a{va.B, va.V, va.max_k, va.R, va.nseg2, va.draft, va.draft_start, va.draft_stride, va.target,
             va.target_start, va.target_stride, va.num_draft, va.tokens, va.temperature, io.top_k, io.top_p,
             va.u_accept, va.u_residual, va.u_bonus, va.accept_len, va.out_tokens, va.labels, va.p_draft,
             va.p_target, io.kept, va.partials, va.zval, io.hmass, io.hcount,
             reinterpret_cast<FSearch*>(io.search), io.tickets, io.work, io.wcount};
  const unsigned g1 = unsigned(n1), g2 = unsigned(va.B) * unsigned(va.R);
  const unsigned gw = unsigned(va.B) * unsigned(va.nseg2);
  const unsigned gn = unsigned(min(n1, uint64_t(2048)));  // workgroups of the later key levels
  RowInfo* info = reinterpret_cast<RowInfo*>(io.info);
  DrawDesc* desc = reinterpret_cast<DrawDesc*>(io.desc);
  float* slices = io.slices;
  // key levels after level 0: bf16, a weight-cell level (below the window)
  // then two of 8-bit digits; fp32, four of 8-bit digits
  const int levels = dtype == SV_BF16 ? 3 : kMaxKeyLevels;
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL(filt_stats0_kernel<uint16_t>, dim3(g1), dim3(kFT), 0, stream, a);
    hipLaunchKernelGGL(filt_select0_kernel<uint16_t>, dim3(g2), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(filt_keys_first_kernel<uint16_t>, dim3(gn), dim3(kFT), 0, stream, a, levels);
    for (int l = 2; l <= levels; ++l)
      hipLaunchKernelGGL(filt_keys_next_kernel<uint16_t>, dim3(gn), dim3(kFT), 0, stream, a, l, levels);
    hipLaunchKernelGGL(filt_verdict_kernel<uint16_t>, dim3(unsigned(va.B)), dim3(64), 0, stream, a, info, desc);
    hipLaunchKernelGGL(filt_weight_kernel<uint16_t>, dim3(gw), dim3(kFT), 0, stream, a, info, desc, slices);
    hipLaunchKernelGGL(filt_search_kernel<uint16_t>, dim3(unsigned(va.B)), dim3(kFT), 0, stream, a, info, desc,
                       slices);
  } else {
    hipLaunchKernelGGL(filt_stats0_kernel<float>, dim3(g1), dim3(kFT), 0, stream, a);
    hipLaunchKernelGGL(filt_select0_kernel<float>, dim3(g2), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(filt_keys_first_kernel<float>, dim3(g1), dim3(kFT), 0, stream, a, levels);
    hipLaunchKernelGGL(filt_select_kernel<float>, dim3(g2), dim3(64), 0, stream, a, levels);
    for (int l = 2; l <= levels; ++l)
      hipLaunchKernelGGL(filt_keys_next_kernel<float>, dim3(gn), dim3(kFT), 0, stream, a, l, levels);
    hipLaunchKernelGGL(filt_verdict_kernel<float>, dim3(unsigned(va.B)), dim3(64), 0, stream, a, info, desc);
    hipLaunchKernelGGL(filt_weight_kernel<float>, dim3(gw), dim3(kFT), 0, stream, a, info, desc, slices);
    hipLaunchKernelGGL(filt_search_kernel<float>, dim3(unsigned(va.B)), dim3(kFT), 0, stream, a, info, desc,
                       slices);
  }
  return hipGetLastError();
}

}  // namespace sv
