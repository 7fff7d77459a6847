// Batched draft-token verification for gfx950: two streaming kernels.
//
// Method: [CS] "Speculative Decoding: Draft, EAGLE, MTP", sections "One
// speculative step" and "Algorithm loop in code" (accept with
// min(1, pt/pd), first rejection -> normalised residual (pt - pd)+, all
// accepted -> bonus token from the last target row); estimator feature and
// score from [AV] "Adaptive Verification ohne Confidence Head", sections
// "Solution: online acceptance estimator" and "Scoring the distribution".
//
// statistics kernel: one workgroup per 32 KiB segment of every row read
//   (draft rows 0..K_b-1, target rows 0..K_b).  Each reduces its segment to
//   (max, sum of exp2((z - max) * c)) - or (max, lowest argmax) for greedy
//   target rows - stores it, and leaves; the segment holding a draft token
//   also stores the logit at that token.  Nothing waits and nothing is
//   counted: the kernel is a plain streaming reduction.
// verdict + draw kernel: one workgroup per 32 KiB segment of the rows the
//   emitted token is drawn from.  Every workgroup of a request first merges
//   the request's segment statistics (a few KiB, from L2) into row
//   statistics and evaluates the accept tests; all of them reach the same
//   accept length a, as they compute the same function of the same data.
//   The first one writes the request's outputs.  Then each reads its
//   segment of the draw rows (residual: draft and target row a; bonus:
//   target row K_b) and hands off the segment's weight; the request's last
//   segment collects the weights, scans them, re-reads the segment where the
//   running weight crosses u * total and searches it.
//
// Workgroups are dispatched in index order, so the last segment of a
// request only ever waits for workgroups that already hold a compute unit:
// the wait ends.  A hand-off slot is 8 bytes written in one store (ready
// marker, value) and is cleared by the workgroup that takes it, so no slot
// holds the marker between calls and replays of a captured call need no
// reset.
//
// Both kernels are plain grids: the hardware dispatcher keeps every compute
// unit busy, and the statistics kernel's small register footprint (8 x 16
// bytes of data per thread) gives 8 waves per SIMD to hide memory latency
// behind the exp2 arithmetic.
#include "sv_segment.hpp"

namespace sv {

namespace {

constexpr int kSleep = 2;  // s_sleep argument while polling a slot

// Hand a 32-bit value off in slot p.
__device__ __forceinline__ void put_slot(uint64_t* p, uint32_t bits) {
  __hip_atomic_store(p, ready_slot(bits), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for slot p (at most spin_limit polls), clear it, return its value.  An
// expired wait (a broken dispatch order) sets the error word and gives NaN.
__device__ __forceinline__ uint32_t take_slot(uint64_t* p, const VerifyArgs& a) {
  uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t k = 0; uint32_t(v) != kSlotReady && k < a.spin_limit; ++k) {
    __builtin_amdgcn_s_sleep(kSleep);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (uint32_t(v) != kSlotReady) {
    store_dev(&a.ctrl[kCtrlError], 1u);
    return 0x7fc00000u;
  }
  __hip_atomic_store(p, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return uint32_t(v >> 32);
}

// Slot of request b's slice q of the draw rows (slice q: vector q % kNV of
// segment q / kNV), see WsLayout::tagged.
static_assert(kNV == kDrawSlices, "one weight slot per vector of a draw segment");
constexpr int kMaxDrawSegs = 256;  // 32 KiB segments of the longest row: 2^21 fp32 elements
static_assert(int64_t(SV_MAX_V) * 4 / kHalfBytes <= kMaxDrawSegs, "draw segments per row");
__device__ __forceinline__ uint64_t* weight_slot(const VerifyArgs& a, int b, int q) {
  return a.tagged + (size_t(b) * a.nseg2) * kNV + q;
}

// ---------------------------------------------------------------------------
// the statistics kernel
// ---------------------------------------------------------------------------

// Workgroup = segment s of row slot r (position order: draft i, target i,
// ..., target max_k) of request b.
template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void stats_kernel(VerifyArgs a) {
  __shared__ Partial red[kWaves];
  const int tid = threadIdx.x;
  const int n = a.nseg2, R = a.R, max_k = a.max_k;
  const uint32_t item = blockIdx.x;
  const int s = int(item % uint32_t(n));
  const int rp = int((item / uint32_t(n)) % uint32_t(R));
  const int b = int(item / (uint32_t(n) * uint32_t(R)));
  const bool draft = rp < 2 * max_k && (rp & 1) == 0;
  const int i = rp < 2 * max_k ? rp >> 1 : max_k;
  // every scalar of the request in one round trip, before the early exit
  const int kraw = a.num_draft[b];
  const float T = a.temperature[b];
  const int64_t start = draft ? a.draft_start[b] : a.target_start[b];
  const int d = i < max_k ? a.tokens[size_t(b) * max_k + i] : -1;
  const int K = min(max(kraw, 0), max_k);
  const bool greedy = !(T > 0.f);
  const int nd = (!greedy || a.av_feature != nullptr) ? K : 0;  // draft rows read
  if (draft ? (i >= nd) : (i > K)) return;
  const float c = uniform(kLog2e / (greedy ? 1.f : T));
  const ET* row = draft ? static_cast<const ET*>(a.draft) + (start + i) * a.draft_stride
                        : static_cast<const ET*>(a.target) + (start + i) * a.target_stride;
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  const bool ztok = !greedy && i < K && d >= s * E && d < (s + 1) * E && d < a.V;
  const int rs = draft ? i : max_k + i;
  if (!draft && greedy)
    stats_segment<ET, kArgmax>(a, red, b, rs, s, ztok, c, row, d, tid);
  else
    stats_segment<ET, kSumInclusive>(a, red, b, rs, s, ztok, c, row, d, tid);
}

// ---------------------------------------------------------------------------
// the verdict and the draw
// ---------------------------------------------------------------------------

// Statistics of a whole row.
struct RowStat {
  float m;  // maximum logit
  float s;  // sum of exp2((z - m) * c) (sum rows)
  int idx;  // lowest-index argmax (greedy target rows)
  float z;  // logit at the draft token (rows of a test position)
};

struct DrawShared {
  float wt[kWaves];
  float sw[kWaves][kNV];
  int wi[2 * kWaves];
  float cum[kDrawSlices * kMaxDrawSegs];  // running slice weights (slices of a draw segment, or of a row)
  Partial red[kWaves];
  RowStat row[2 * SV_MAX_K + 1];  // by row slot: draft i at i, target j at max_k + j
  int word;
  float fv;
  float fz, ft, fb4;
  int fk, ffb;
};

// Weight of element j of vector k: residual max(0, pt - pd), or pt.
template <typename ET, bool RESID>
__device__ __forceinline__ float elem_w(const uint4& zt, const uint4& zd, int j, float c, float kt, float kd) {
  const float pt = fast_exp2(fmaf(Elem<ET>::get(zt, j), c, -kt));
  if (RESID) return fmaxf(pt - fast_exp2(fmaf(Elem<ET>::get(zd, j), c, -kd)), 0.f);
  return pt;
}

// Weights of the kNV / 2 slices K0 .. of a segment (slice k: vector k of
// every thread, a contiguous kThreads * N elements), per wave into sh.sw.
template <typename ET, bool RESID, int K0>
__device__ __forceinline__ void half_weights(const uint4 (&t)[kNV / 2], const uint4 (&d)[kNV / 2], float c, float kt,
                                             float kd, DrawShared& sh, int tid) {
  constexpr int N = Elem<ET>::N;
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int k = 0; k < kNV / 2; ++k) {
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) r += elem_w<ET, RESID>(t[k], d[k], j, c, kt, kd);
    r = wave_sum(r);
    if (lane == 0) sh.sw[wave][K0 + k] = r;
  }
}

// Weights of the segment's kNV slices, handed off to the request's search in
// slots[0 .. kNV-1]; the segment is read in two halves, so that a workgroup
// holds 16 KiB of it at a time.  Each slice's sum takes the same order in
// every call.
template <typename ET, bool RESID>
__device__ __forceinline__ void slice_weights(const ET* rt, const ET* rd, int hb, int V, float c, float kt, float kd,
                                              uint64_t* slots, DrawShared& sh, int tid) {
  {
    uint4 t[kNV / 2], d[kNV / 2];
    load_vecs<ET, kNV / 2, 0>(rt, hb, V, t);
    if (RESID) load_vecs<ET, kNV / 2, 0>(rd, hb, V, d);
    half_weights<ET, RESID, 0>(t, d, c, kt, kd, sh, tid);
  }
  {
    uint4 t[kNV / 2], d[kNV / 2];
    load_vecs<ET, kNV / 2, kNV / 2>(rt, hb, V, t);
    if (RESID) load_vecs<ET, kNV / 2, kNV / 2>(rd, hb, V, d);
    half_weights<ET, RESID, kNV / 2>(t, d, c, kt, kd, sh, tid);
  }
  __syncthreads();
  if (tid < kNV) {
    float W = sh.sw[0][tid];
    for (int x = 1; x < kWaves; ++x) W += sh.sw[x][tid];
    put_slot(slots + tid, __float_as_uint(W));
  }
}

// Scan the m weights in sh.cum (in place, in token order) and find the
// crossing entry k: the first whose running weight exceeds u * Z (-1 if Z is
// not positive; if rounding leaves u * Z at or above the last running
// weight, the last entry with positive weight, flagged), the weight before
// it, u * Z.
__device__ __forceinline__ void scan_cum(int m, float u, DrawShared& sh, int tid) {
  const int lane = tid & 63;
  __syncthreads();
  if (tid < 64) {
    float carry = 0.f;
    for (int base = 0; base < m; base += 64) {
      const int q = base + lane;
      float x = (q < m) ? sh.cum[q] : 0.f;
      x = wave_inclusive_scan(x, lane) + carry;
      if (q < m) sh.cum[q] = x;
      carry = __shfl(x, 63, 64);
    }
    if (lane == 0) {
      const float Z = carry;
      int k = -1, fb = 0;
      float thr = 0.f;
      if (Z > 0.f) {
        thr = u * Z;
        int lo = 0, hi = m;  // first k with cum[k] > thr
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (sh.cum[mid] > thr)
            hi = mid;
          else
            lo = mid + 1;
        }
        k = lo;
        if (k == m) {
          k = m - 1;
          while (k > 0 && !(sh.cum[k] > sh.cum[k - 1])) --k;
          fb = 1;
        }
      }
      sh.fk = k;
      sh.ffb = fb;
      sh.ft = thr;
      sh.fb4 = k > 0 ? sh.cum[k - 1] : 0.f;
    }
  }
  __syncthreads();
}

// Collect the m slice weights of request b from their slots and scan them.
__device__ __forceinline__ void scan_slices(const VerifyArgs& a, int b, int m, float u, DrawShared& sh, int tid) {
  if (tid < 64) {
    uint64_t* slots = weight_slot(a, b, 0);
    for (int q = tid; q < m; q += 64) sh.cum[q] = __uint_as_float(take_slot(slots + q, a));
  }
  scan_cum(m, u, sh, tid);
}

// Within one slice (thread t holds elements first + t*N .. + N-1): the first
// element whose running weight from `before` exceeds thr; if none (rounding,
// or `fallback`), the slice's last positive-weight element.  The same value
// in every thread.
template <typename ET, bool RESID>
__device__ __forceinline__ int slice_search(const ET* rt, const ET* rd, int first, int V, float c, float kt, float kd,
                                            float before, float thr, bool fallback, DrawShared& sh, int tid) {
  constexpr int N = Elem<ET>::N;
  const int wave = tid >> 6, lane = tid & 63;
  const int e0 = first + tid * N;
  const uint4 zt = load_raw<ET>(rt, e0, V, is_aligned16(rt));
  const uint4 zd = RESID ? load_raw<ET>(rd, e0, V, is_aligned16(rd)) : zt;
  float w[N], vt = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    w[j] = elem_w<ET, RESID>(zt, zd, j, c, kt, kd);
    vt += w[j];
  }
  const float incl = wave_inclusive_scan(vt, lane);
  if (lane == 63) sh.wt[wave] = incl;
  float excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.f;
  __syncthreads();
  float run = before + excl;
  for (int x = 0; x < wave; ++x) run += sh.wt[x];
  int mine = -1, last = -1;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    run += w[j];
    if (w[j] > 0.f) {
      last = e0 + j;
      if (mine < 0 && !fallback && run > thr) mine = e0 + j;
    }
  }
  const unsigned long long hit = __ballot(mine >= 0);
  const int found = hit ? __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1, 64) : -1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) {
    sh.wi[wave] = found;
    sh.wi[kWaves + wave] = last;
  }
  __syncthreads();
  int result = -1, lastall = -1;
  for (int x = 0; x < kWaves; ++x) {
    if (result < 0) result = sh.wi[x];
    lastall = max(lastall, sh.wi[kWaves + x]);
  }
  __syncthreads();
  return uniform(result >= 0 ? result : lastall);
}

// The draw from pt itself (the residual has no mass, reachable only
// through rounding): the row's slices are weighed by the waves in turn (wave
// w takes slices w, w + kWaves, ...), then scanned and searched like the
// residual's.  Slow and rarely taken; it holds one vector per lane.
template <typename ET>
__device__ __forceinline__ int draw_from_target(const ET* rt, int V, float c, float kt, float u, DrawShared& sh,
                                                int tid) {
  constexpr int N = Elem<ET>::N;
  constexpr int EV = kThreads * N;  // elements per slice
  const int wave = tid >> 6, lane = tid & 63;
  const int m = (V + EV - 1) / EV;  // at most kDrawSlices * kMaxDrawSegs
  const bool al = is_aligned16(rt);
  for (int q = wave; q < m; q += kWaves) {
    float w = 0.f;
    for (int x = 0; x < kThreads / 64; ++x) {
      const uint4 z = load_raw<ET>(rt, q * EV + (x * 64 + lane) * N, V, al);
#pragma unroll
      for (int j = 0; j < N; ++j) w += elem_w<ET, false>(z, z, j, c, kt, kt);
    }
    w = wave_sum(w);
    if (lane == 0) sh.cum[q] = w;
  }
  scan_cum(m, u, sh, tid);
  const int k = uniform(sh.fk);
  if (k < 0) return -1;
  return slice_search<ET, false>(rt, rt, k * EV, V, c, kt, kt, uniform(sh.fb4), uniform(sh.ft), uniform(sh.ffb) != 0,
                                 sh, tid);
}

// Weights of segment s of the draw rows, handed off to the request's search.
template <typename ET, bool RESID>
__device__ __forceinline__ void weight_segment(const VerifyArgs& a, DrawShared& sh, int b, int s, float c, float kt,
                                               float kd, const ET* rt, const ET* rd, int tid) {
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  slice_weights<ET, RESID>(rt, rd, s * E, a.V, c, kt, kd, weight_slot(a, b, s * kNV), sh, tid);
}

// The draw of request b once its slices' weights are in: scan them, read the
// crossing slice again and search it.
template <typename ET, bool RESID>
__device__ __forceinline__ void search_request(const VerifyArgs& a, DrawShared& sh, int b, int aa, float c, float kt,
                                               float kd, float u, const ET* rt, const ET* rd, int tid) {
  constexpr int EV = kThreads * Elem<ET>::N;  // elements per slice
  scan_slices(a, b, a.nseg2 * kNV, u, sh, tid);
  const int k = uniform(sh.fk);
  int tok = -1;
  if (k < 0) {
    // the residual has no mass (reachable only through rounding): draw from pt itself
    if (RESID) tok = draw_from_target<ET>(rt, a.V, c, kt, u, sh, tid);
  } else {
    tok = slice_search<ET, RESID>(rt, rd, k * EV, a.V, c, kt, kd, uniform(sh.fb4), uniform(sh.ft), uniform(sh.ffb) != 0,
                                  sh, tid);
  }
  if (tid == 0) a.out_tokens[size_t(b) * (a.max_k + 1) + aa] = tok;
}

// Merge the segment statistics of the request's rows into sh.row, by row
// slot (draft i at i, target j at max_k + j; slots of rows the statistics
// kernel skipped hold stale values that nothing reads).  A row takes G lanes
// (G the smallest power of two >= the segments per row, at most 64), so a
// wave merges 64 / G rows at a time: lane j of a row's group merges
// segments j, j + G, ... in order, then a butterfly over the group combines
// the lanes.  Every workgroup of the request evaluates the same function of
// the same data, so all reach the same statistics.  The first pass's loads
// (MergeFirst) are issued beforehand, with the request's scalars.
struct MergeFirst {
  Partial p;  // the lane's first segment of its row in the first pass
  float z;    // the row's logit at the draft token
};
__device__ __forceinline__ int merge_lanes(int n) {
  int G = 1;
  while (G < n && G < 64) G <<= 1;
  return G;
}
__device__ __forceinline__ MergeFirst merge_first(const VerifyArgs& a, int b, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int n = a.nseg2, R = a.R;
  const int G = merge_lanes(n);
  const int q = min(wave * (64 / G) + lane / G, R - 1), x = min(lane & (G - 1), n - 1);
  return MergeFirst{a.partials[(size_t(b) * R + q) * n + x], a.zval[size_t(b) * R + q]};
}
__device__ __forceinline__ void merge_rows(const VerifyArgs& a, DrawShared& sh, int b, bool greedy, float c,
                                           const MergeFirst& first, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int n = a.nseg2, max_k = a.max_k, R = a.R;
  const int G = merge_lanes(n);
  const int RW = 64 / G;  // rows per wave and pass
  const int g = lane / G, j = lane & (G - 1);
  const Partial* base = a.partials + size_t(b) * R * n;
  for (int q0 = wave * RW; q0 < R; q0 += kWaves * RW) {
    const int q = q0 + g;
    const bool amax = greedy && q >= max_k;
    const bool pass0 = q0 == wave * RW;
    const float z = (q < R && j == 0) ? (pass0 ? first.z : a.zval[size_t(b) * R + q]) : NAN;
    Partial acc{-INFINITY, 0.f, 0.f, 0x7fffffff};
    if (q < R)
      for (int x = j; x < n; x += G) {
        const Partial p = (pass0 && x == j) ? first.p : base[size_t(q) * n + x];
        if (amax)
          merge_argmax(acc.m, acc.idx, p.m, p.idx);
        else
          merge_ms(acc.m, acc.s, acc.cnt, p.m, p.s, p.cnt, c);
      }
    for (int o = G >> 1; o >= 1; o >>= 1) {
      Partial y;
      y.m = __shfl_xor(acc.m, o, 64);
      y.s = __shfl_xor(acc.s, o, 64);
      y.cnt = __shfl_xor(acc.cnt, o, 64);
      y.idx = __shfl_xor(acc.idx, o, 64);
      if (amax)
        merge_argmax(acc.m, acc.idx, y.m, y.idx);
      else
        merge_ms(acc.m, acc.s, acc.cnt, y.m, y.s, y.cnt, c);
    }
    if (j == 0 && q < R) sh.row[q] = RowStat{acc.m, acc.s + acc.cnt, acc.idx, z};
  }
  __syncthreads();
}

// Estimator feature of a confident draft row i (sum of the non-maximal
// probabilities below kRecomputeBelow - 1): the first segment holding the
// row maximum is summed again leaving out one maximal term exactly, and the
// other segments' sums are added at the row maximum's scale.
template <typename ET>
__device__ __forceinline__ void confident_feature(const VerifyArgs& a, DrawShared& sh, int b, int i, float c,
                                                  int tid) {
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = a.nseg2;
  const float M = sh.row[i].m;
  if (wave == 0) {
    const Partial* pp = a.partials + (size_t(b) * a.R + i) * n;
    int first = 0x7fffffff;
    float rest = 0.f;
    for (int s0 = 0; s0 < n; s0 += 64) {
      const int q = s0 + lane;
      const Partial p = q < n ? pp[q] : Partial{-INFINITY, 0.f, 0.f, 0x7fffffff};
      const uint64_t hit = __ballot(q < n && p.m == M);
      if (first == 0x7fffffff && hit) first = s0 + __ffsll(static_cast<long long>(hit)) - 1;
      const float x = (p.m != -INFINITY && q != first) ? (p.s + p.cnt) * fast_exp2((p.m - M) * c) : 0.f;
      rest += wave_sum(x);
    }
    if (lane == 0) {
      sh.fk = first;
      sh.fv = rest;
    }
  }
  __syncthreads();
  const int seg = uniform(sh.fk);
  const float rest = sh.fv;
  float x = kFeatureClamp;
  if (seg != 0x7fffffff) {
    const ET* rd = static_cast<const ET*>(a.draft) + (a.draft_start[b] + i) * a.draft_stride;
    uint4 v[kNV];
    load_seg<ET>(rd, seg * E, a.V, v, tid);
    const Partial e = block_reduce<kSumExclusive>(thread_stats<ET, kSumExclusive>(v, seg * E, c, tid), c, sh.red, tid);
    x = feature_from_other(e.s + (e.cnt - 1.f) + rest);
  }
  if (tid == 0) {
    const size_t o = size_t(b) * a.max_k + i;
    a.av_feature[o] = x;
    if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, x);
  }
  __syncthreads();
}

// Workgroup = segment s of the draw rows of request b (weights); the
// request's last segment then collects all the weights and searches.
// Requests in order; every workgroup derives its request's verdict first.
template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void draw_kernel(VerifyArgs a) {
  __shared__ DrawShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.nseg2, max_k = a.max_k;
  const int s = int(blockIdx.x % uint32_t(n));
  const int b = int(blockIdx.x / uint32_t(n));
  // Everything the verdict needs in one round trip: the request's scalars,
  // lane i's token and uniform, the merge's first loads.  The scalars are
  // loaded by every lane (indexed through an opaque zero), so that they are
  // vector loads: scalar loads would share one counter with the reloads of
  // the kernel arguments, and each reload's wait would wait for them too.
  const int z0 = fresh_tid() >> 16;  // 0
  const int kraw_l = a.num_draft[b + z0];
  const float T_l = a.temperature[b + z0];
  const int64_t ts = a.target_start[b + z0];
  const int64_t dsl = (max_k > 0 ? a.draft_start : a.target_start)[b + z0];
  const float ures = a.u_residual[b + z0], ubon = a.u_bonus[b + z0];
  // lane i of wave 0 tests position i: its token and uniform (loaded for
  // every i < max_k, so that the loads need not wait for K)
  int dl = -1;
  float ul = 0.f;
  if (wave == 0 && lane < max_k) {
    dl = a.tokens[size_t(b) * max_k + lane];
    ul = a.u_accept[size_t(b) * max_k + lane];
  }
  const MergeFirst mf = merge_first(a, b, tid);
  pin_all(kraw_l, T_l, ts, dsl, ures, ubon, dl, ul, mf.p.m, mf.p.s, mf.p.cnt, mf.p.idx, mf.z);
  const int kraw = uniform(kraw_l);
  const float T = uniform(T_l);
  const int64_t ds = max_k > 0 ? dsl : 0;
  const int K = min(max(kraw, 0), max_k);
  const bool greedy = !(T > 0.f);
  const bool want_feat = a.av_feature != nullptr;
  const int nd = (!greedy || want_feat) ? K : 0;  // draft rows read
  const float c = uniform(kLog2e / (greedy ? 1.f : T));
  merge_rows(a, sh, b, greedy, c, mf, tid);

  // the accept tests, and the accept length a: the first rejection, else K
  float pd = NAN, pt = NAN;
  if (wave == 0) {
    bool rej = false;
    if (lane < K) {
      const RowStat tr = sh.row[max_k + lane];
      if (greedy) {
        rej = dl != tr.idx;
        pt = rej ? 0.f : 1.f;
      } else {
        const RowStat dr = sh.row[lane];
        const float l2d = (dr.z - dr.m) * c - fast_log2(dr.s);
        const float l2t = (tr.z - tr.m) * c - fast_log2(tr.s);
        pd = fast_exp2(l2d);
        pt = fast_exp2(l2t);
        rej = !((l2d == -INFINITY) || (ul < fast_exp2(l2t - l2d)));
      }
    }
    const uint64_t rm = __ballot(rej);
    if (lane == 0) sh.word = rm ? __ffsll(static_cast<long long>(rm)) - 1 : K;
  }
  __syncthreads();
  const int aa = uniform(sh.word);
  const bool resid = aa < K;
  const float u = resid ? ures : ubon;
  const ET* rt = static_cast<const ET*>(a.target) + (ts + aa) * a.target_stride;
  const ET* rd = resid ? static_cast<const ET*>(a.draft) + (ds + aa) * a.draft_stride : rt;
  const RowStat tr = sh.row[max_k + aa];
  const RowStat dr = sh.row[resid ? aa : max_k + aa];
  const float kt = tr.m * c + fast_log2(tr.s);
  const float kd = dr.m * c + fast_log2(dr.s);

  // the request's outputs, by its first workgroup (the token at a of a
  // stochastic request comes from the search)
  if (s == 0 && wave == 0) {
    const int j = lane;
    if (j < max_k) {
      const size_t o = size_t(b) * max_k + j;
      if (a.labels) a.labels[o] = (j < aa) ? 1 : ((j == aa && aa < K) ? 0 : -1);
      if (a.p_draft) a.p_draft[o] = j < K ? pd : NAN;
      if (a.p_target) a.p_target[o] = j < K ? pt : NAN;
      if (want_feat && !(j < nd && sh.row[j].s < kRecomputeBelow)) {  // confident rows: below
        const float x = j < nd ? feature_from_other(sh.row[j].s - 1.f) : NAN;
        a.av_feature[o] = x;
        if (a.av_score) a.av_score[o] = j < nd ? sigmoid_score(a.av_params, j, x) : NAN;
      }
    }
    if (j <= max_k && j != aa) a.out_tokens[size_t(b) * (max_k + 1) + j] = (j < aa) ? dl : -1;
    if (j == 0) {
      a.accept_len[b] = aa;
      if (greedy) a.out_tokens[size_t(b) * (max_k + 1) + aa] = tr.idx;
    }
  }
  if (!greedy) {
    // the last segment waits only for workgroups dispatched before it
    if (resid) {
      weight_segment<ET, true>(a, sh, b, s, c, kt, kd, rt, rd, tid);
      if (s == n - 1) search_request<ET, true>(a, sh, b, aa, c, kt, kd, u, rt, rd, tid);
    } else {
      weight_segment<ET, false>(a, sh, b, s, c, kt, kd, rt, rd, tid);
      if (s == n - 1) search_request<ET, false>(a, sh, b, aa, c, kt, kd, u, rt, rd, tid);
    }
  }
  // features of confident draft rows: position i by the workgroup of segment i mod n
  if (want_feat)
    for (int i = s; i < nd; i += n)
      if (sh.row[i].s < kRecomputeBelow) confident_feature<ET>(a, sh, b, i, c, tid);
}

// ---------------------------------------------------------------------------
// the estimator's scoring pass: statistics of the draft rows, then one
// workgroup per request for feature, score, survival and the kept count
// ---------------------------------------------------------------------------

// Workgroup = segment s of draft row i of request b (the statistics kernel's
// access pattern and partials layout).  Greedy requests are scored at T = 1.
template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void score_stats_kernel(
    VerifyArgs a) {
  __shared__ Partial red[kWaves];
  const int tid = threadIdx.x;
  const int n = a.nseg2, max_k = a.max_k;
  const uint32_t item = blockIdx.x;
  const int s = int(item % uint32_t(n));
  const int i = int((item / uint32_t(n)) % uint32_t(max_k));
  const int b = int(item / (uint32_t(n) * uint32_t(max_k)));
  const int kraw = a.num_draft[b];
  const float T = a.temperature[b];
  const int64_t start = a.draft_start[b];
  const int K = min(max(kraw, 0), max_k);
  if (i >= K) return;
  const float c = uniform(kLog2e / ((T > 0.f) ? T : 1.f));
  const ET* row = static_cast<const ET*>(a.draft) + (start + i) * a.draft_stride;
  stats_segment<ET, kSumInclusive>(a, red, b, i, s, false, c, row, -1, tid);
}

// Workgroup = request b: merge each draft row's segment statistics (lane
// groups, as in the verdict), feature and score of every position (confident
// rows re-summed exactly, as in the verification), then the survival prune.
template <typename ET>
__global__ __launch_bounds__(kThreads) void score_finish_kernel(VerifyArgs a, float threshold, int32_t* num_kept) {
  __shared__ DrawShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.nseg2, max_k = a.max_k, R = a.R;
  const int b = blockIdx.x;
  const int K = min(max(a.num_draft[b], 0), max_k);
  const float T = a.temperature[b];
  const float c = uniform(kLog2e / ((T > 0.f) ? T : 1.f));
  int G = 1;
  while (G < n && G < 64) G <<= 1;
  const int RW = 64 / G;
  const int g = lane / G, j = lane & (G - 1);
  const Partial* base = a.partials + size_t(b) * R * n;
  for (int q0 = wave * RW; q0 < K; q0 += kWaves * RW) {
    const int q = q0 + g;
    Partial acc{-INFINITY, 0.f, 0.f, 0x7fffffff};
    if (q < K)
      for (int x = j; x < n; x += G) {
        const Partial p = base[size_t(q) * n + x];
        merge_ms(acc.m, acc.s, acc.cnt, p.m, p.s, p.cnt, c);
      }
    for (int o = G >> 1; o >= 1; o >>= 1) {
      const float m2 = __shfl_xor(acc.m, o, 64), s2 = __shfl_xor(acc.s, o, 64), c2 = __shfl_xor(acc.cnt, o, 64);
      merge_ms(acc.m, acc.s, acc.cnt, m2, s2, c2, c);
    }
    if (j == 0 && q < K) sh.row[q] = RowStat{acc.m, acc.s + acc.cnt, 0x7fffffff, NAN};
  }
  __syncthreads();
  if (tid < max_k) {
    const size_t o = size_t(b) * max_k + tid;
    const bool conf = tid < K && sh.row[tid].s < kRecomputeBelow;  // below, exactly
    if (!conf) {
      const float x = tid < K ? feature_from_other(sh.row[tid].s - 1.f) : NAN;
      a.av_feature[o] = x;
      a.av_score[o] = tid < K ? sigmoid_score(a.av_params, tid, x) : NAN;
    }
  }
  __syncthreads();
  for (int i = 0; i < K; ++i)
    if (sh.row[i].s < kRecomputeBelow) confident_feature<ET>(a, sh, b, i, c, tid);
  if (tid == 0 && num_kept) {
    // survival: the running product of the scores, kept while >= threshold
    int kept = K;
    if (threshold > 0.f) {
      float surv = 1.f;
      kept = 0;
      for (int i = 0; i < K; ++i) {
        surv *= a.av_score[size_t(b) * max_k + i];
        if (!(surv >= threshold)) break;
        ++kept;
      }
    }
    num_kept[b] = kept;
  }
}

}  // namespace

hipError_t launch_score(VerifyArgs a, float threshold, int32_t* num_kept, int dtype, hipStream_t stream) {
  const uint64_t n1 = uint64_t(a.B) * uint64_t(a.max_k) * uint64_t(a.nseg2);
  if (a.B == 0) return hipSuccess;
  if (n1 >= (uint64_t(1) << 31)) return hipErrorInvalidValue;
  const bool bf = dtype == SV_BF16;
  if (n1 > 0) {
    if (bf)
      hipLaunchKernelGGL(score_stats_kernel<uint16_t>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(score_stats_kernel<float>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
  }
  if (bf)
    hipLaunchKernelGGL(score_finish_kernel<uint16_t>, dim3(unsigned(a.B)), dim3(kThreads), 0, stream, a, threshold,
                       num_kept);
  else
    hipLaunchKernelGGL(score_finish_kernel<float>, dim3(unsigned(a.B)), dim3(kThreads), 0, stream, a, threshold,
                       num_kept);
  return hipGetLastError();
}

hipError_t launch_streaming(VerifyArgs a, int dtype, hipStream_t stream) {
  const uint64_t n1 = uint64_t(a.B) * uint64_t(a.R) * uint64_t(a.nseg2);
  const uint64_t n2 = uint64_t(a.B) * uint64_t(a.nseg2);  // one workgroup per segment of the draw rows
  if (n1 == 0) return hipSuccess;
  if (n1 >= (uint64_t(1) << 31)) return hipErrorInvalidValue;
  a.spin_limit = 1u << 18;  // a fraction of a second of polling: reached only if dispatch order were broken
  const bool bf = dtype == SV_BF16;
  if (bf)
    hipLaunchKernelGGL(stats_kernel<uint16_t>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(stats_kernel<float>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
  if (bf)
    hipLaunchKernelGGL(draw_kernel<uint16_t>, dim3(unsigned(n2)), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(draw_kernel<float>, dim3(unsigned(n2)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

namespace {

__global__ void status_kernel(uint32_t* ctrl, int32_t* status, int clear) {
  status[0] = int32_t(__hip_atomic_load(&ctrl[kCtrlError], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  if (clear) store_dev(&ctrl[kCtrlError], 0u);
}

}  // namespace

hipError_t launch_status(uint32_t* ctrl, int32_t* status, int clear, hipStream_t stream) {
  hipLaunchKernelGGL(status_kernel, dim3(1), dim3(1), 0, stream, ctrl, status, clear);
  return hipGetLastError();
}

}  // namespace sv
