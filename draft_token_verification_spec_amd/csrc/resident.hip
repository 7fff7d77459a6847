// Batched draft-token verification for gfx950, register-resident variant.
//
// Method: [CS] "Speculative Decoding: Draft, EAGLE, MTP", sections "One
// speculative step" and "Algorithm loop in code" (accept with
// min(1, pt/pd), first rejection -> normalised residual (pt - pd)+, all
// accepted -> bonus token from the last target row); estimator feature and
// score from [AV] "Adaptive Verification ohne Confidence Head", sections
// "Solution: online acceptance estimator" and "Scoring the distribution".
//
// Request b owns `stride`
// item slots; an item is one of
//
//   pair item (i, s):   half segment s (32 KiB) of draft row i and the same
//                       half segment of target row i, for i < K_b;
//   single item (i, s): segment s (64 KiB) of target row i, for target rows
//                       read without a draft row beside them (the bonus row
//                       K_b; every row of a greedy request whose draft rows
//                       are not needed).
//
// An item loads its data (16 x 16 bytes per thread), reduces it to partial
// statistics, publishes them, parks its first half in LDS (the second stays
// in registers) and counts itself into its row.  Items that may draw, the
// item that may hold a confident draft row's maximum, and the row's leader
// (its item 0) wait until the row is complete, then each combines the row's
// partials itself: row statistics, the accept test of position i, the
// normalisers.  The leader writes the row's outputs and sets the row's bits
// in the request's verdict mask (bit i: known; bit 32 + i: rejected); the
// leader whose bit fixes the accept length writes the request's outputs.
//
// The token is drawn from row a: the first rejected row, or the bonus row K_b
// when every draft was accepted.  An item knows from its own row whether it
// was rejected, so the items of a rejected row 0 go straight to the draw;
// those of a later rejected row (or of the bonus row) wait only for the
// verdicts of the rows before it.  The draw items compute their segment's
// weight from registers and publish it; once all are in, each scans the
// weights, and the item holding the segment where the running weight crosses
// u * total searches its registers for the token.  Every logit is read from
// memory once.
//
// Progress: items are claimed in slot order (rows in order, the items of a
// row consecutive) from one of `parts` counters (partition p owns requests
// b = p mod parts).  An item waits only for items of its own row and of
// earlier rows of its request, all claimed before it or with it: a row whose
// items are all claimed completes once the rows before it have.  Taking the
// smallest unfinished item of a partition, either its row is fully claimed
// (and completes) or the partition holds at most (row items - 1) waiting
// items; with more than parts * (row items - 1) resident workgroups one is
// then free to claim - the launcher picks `parts` to make that hold.  A
// workgroup claims its next item only once its current item has nothing
// left to wait for.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kWaitSleep = 8;   // s_sleep argument while polling a request word
constexpr int kMaxCum = 256;    // half segments per row: 2^21 fp32 elements / 32 KiB
static_assert(int64_t(SV_MAX_V) * 4 / kHalfBytes <= kMaxCum, "segment weight prefix");
constexpr uint32_t kNoClaim = 0xffffffffu;
constexpr uint32_t kPlainMismatch = 0xfffffffeu;  // run the item with the other load kind

// What every item of row i learns once the row is complete.
struct RowView {
  Partial D, Tg;  // draft (pair rows) and target row statistics
  float kt, kd;   // log2 normalisers: log2 p(v) = z * c - k
  float pd, pt;   // probabilities of the draft token (stochastic rows i < K)
  int acc;        // accept test of position i (1 for the bonus row)
};

// Outcome of the draw's scan over its segment weights.
struct Choice {
  float Z, t, before;
  int k;      // -1 if Z is not positive
  int fb;     // no running sum crossed t (rounding): k is the last segment with weight
};

struct RShared {
  uint4 park[kHalfVecs][kThreads];  // the item's first 32 KiB half, parked after the statistics
  Partial part[2][kWaves];
  float sw[kWaves][kVecsPerThread];  // per-wave sweep totals of the search
  float wt[kWaves];
  int wi[2 * kWaves];
  float cum[kMaxCum];
  Partial cp[2][64];  // partials of one row being combined
  float zv[2];        // logits at the draft token: draft, target
  RowView rv;
  Choice ch;
  float fv;
  uint64_t mask;
  int word;
  uint32_t next;
};

__device__ __forceinline__ uint32_t claim(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The thread index, opaque to the optimiser: lane-dependent addresses are
// computed inside each item instead of being hoisted out of the persistent
// loop, where dozens of them would stay live for the whole kernel.
__device__ __forceinline__ int item_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// A workgroup-uniform value, moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return uint32_t(__builtin_amdgcn_readfirstlane(int(v))); }
__device__ __forceinline__ float uniform(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// data in registers
// ---------------------------------------------------------------------------
//
// An item's data is two 32 KiB halves: `lo` (pair: the draft half; single:
// the first half of the segment) and `hi` (pair: the target half; single: the
// second half).  Vector k of thread t of a half starting at element hb holds
// elements hb + (k * kThreads + t) * N .. + N-1 of its row, so token order is
// vector, then thread, then element.  Elements past the end of the row read
// as -inf.  After the statistics `lo` is parked in LDS (sh.park[k][t]) and
// only `hi` stays in registers.

// True when both halves are 16-byte aligned and inside the row: then they are
// read with plain 16-byte loads.
template <typename ET>
__device__ __forceinline__ bool plain_halves(const ET* r0, int h0, const ET* r1, int h1, int V) {
  constexpr int E2 = kThreads * kHalfVecs * Elem<ET>::N;
  return is_aligned16(r0) && is_aligned16(r1) && h0 + E2 <= V && h1 + E2 <= V;
}

// Loads half lo from (r0, h0) and half hi from (r1, h1).  The whole item is
// instantiated once per load kind, so the careful path's branches never merge
// into the plain path's registers.
template <typename ET, bool PLAIN>
__device__ __forceinline__ void load_halves(const ET* r0, int h0, const ET* r1, int h1, int V,
                                            uint4 (&lo)[kHalfVecs], uint4 (&hi)[kHalfVecs], int tid) {
  constexpr int N = Elem<ET>::N;
  const bool a0 = is_aligned16(r0), a1 = is_aligned16(r1);
  if (PLAIN) {
#pragma unroll
    for (int k = 0; k < kHalfVecs; ++k) {
      lo[k] = load_vec16<ET>(r0 + h0 + (k * kThreads + tid) * N);
      hi[k] = load_vec16<ET>(r1 + h1 + (k * kThreads + tid) * N);
    }
  } else {
#pragma unroll
    for (int k = 0; k < kHalfVecs; ++k) {
      lo[k] = load_raw<ET>(r0, h0 + (k * kThreads + tid) * N, V, a0);
      hi[k] = load_raw<ET>(r1, h1 + (k * kThreads + tid) * N, V, a1);
    }
  }
}

// Opaque to the optimiser: values computed from the registers before a fence
// are not reused after it (they would stay live across the waits, which
// spills), so every phase decodes the raw vectors again.
__device__ __forceinline__ void fence_regs(uint4 (&v)[kHalfVecs]) {
#pragma unroll
  for (int k = 0; k < kHalfVecs; ++k) keep_raw(v[k]);
}

// Per-thread statistics of one half starting at element hb (see Partial).
template <typename ET, int MODE>
__device__ __forceinline__ Partial thread_stats(uint4 (&v)[kHalfVecs], int hb, float c, int tid) {
  constexpr int N = Elem<ET>::N;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kHalfVecs; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) m = fmaxf(m, Elem<ET>::get(v[k], j));
  if (N == 8) fence_regs(v);
  float s = 0.f, cnt = 0.f;
  int idx = 0x7fffffff;
  if (MODE == kArgmax) {
#pragma unroll
    for (int k = kHalfVecs - 1; k >= 0; --k)
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (Elem<ET>::get(v[k], j) == m) idx = hb + (k * kThreads + tid) * N + j;
    if (m == -INFINITY) idx = 0x7fffffff;
  } else if (m != -INFINITY) {
    const float mc = m * c;
#pragma unroll
    for (int k = 0; k < kHalfVecs; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float z = Elem<ET>::get(v[k], j);
        const float e = fast_exp2(fmaf(z, c, -mc));
        if (MODE == kSumExclusive) {
          s += (z < m) ? e : 0.f;
          cnt += (z == m) ? 1.f : 0.f;
        } else {
          s += e;
        }
      }
  }
  return Partial{m, s, cnt, idx};
}

template <int MODE>
__device__ __forceinline__ void merge_partial(Partial& p, const Partial& q, float c) {
  if (MODE == kArgmax)
    merge_argmax(p.m, p.idx, q.m, q.idx);
  else
    merge_ms(p.m, p.s, p.cnt, q.m, q.s, q.cnt, c);
}

template <int MODE>
__device__ __forceinline__ Partial wave_reduce(Partial p, float c) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(p.m, o, 64);
    if (MODE == kArgmax) {
      merge_argmax(p.m, p.idx, m2, __shfl_xor(p.idx, o, 64));
    } else {
      const float s2 = __shfl_xor(p.s, o, 64);
      const float c2 = __shfl_xor(p.cnt, o, 64);
      merge_ms(p.m, p.s, p.cnt, m2, s2, c2, c);
    }
  }
  return p;
}

template <int MODE>
__device__ __forceinline__ Partial merge_waves(const Partial* lds, float c) {
  Partial p = lds[0];
  for (int w = 1; w < kWaves; ++w) {
    if (MODE == kArgmax)
      merge_argmax(p.m, p.idx, lds[w].m, lds[w].idx);
    else
      merge_ms(p.m, p.s, p.cnt, lds[w].m, lds[w].s, lds[w].cnt, c);
  }
  return p;
}

// ---------------------------------------------------------------------------
// draw weights from registers
// ---------------------------------------------------------------------------

enum WeightKind {
  kWResid = 0,   // pair item: max(0, pt - pd); sweep k = lo[k] (draft) with hi[k] (target)
  kWTarget = 1,  // pair item: pt from hi[k]
  kWPlain = 2,   // single item: pt; sweeps 0..7 = lo, 8..15 = hi
};

template <int WK>
struct Sweeps {
  static constexpr int n = WK == kWPlain ? 2 * kHalfVecs : kHalfVecs;
};

// The target (zt) and draft (zd) vectors of sweep k.
template <int WK>
__device__ __forceinline__ void sweep_vecs(const RShared& sh, const uint4 (&hi)[kHalfVecs], int k, int tid, uint4& zt,
                                           uint4& zd) {
  if (WK == kWResid) {
    zt = hi[k];
    zd = sh.park[k][tid];
  } else if (WK == kWTarget) {
    zt = hi[k];
  } else {
    zt = k < kHalfVecs ? sh.park[k][tid] : hi[k - kHalfVecs];
  }
}

template <typename ET, int WK>
__device__ __forceinline__ float elem_weight(const uint4& zt, const uint4& zd, int j, float c, float kt, float kd) {
  const float pt = fast_exp2(fmaf(Elem<ET>::get(zt, j), c, -kt));
  if (WK == kWResid) return fmaxf(pt - fast_exp2(fmaf(Elem<ET>::get(zd, j), c, -kd)), 0.f);
  return pt;
}

// Total draw weight of the item's range, the same value in every thread.
template <typename ET, int WK>
__device__ __forceinline__ float range_weight(uint4 (&hi)[kHalfVecs], float c, float kt, float kd, RShared& sh,
                                              int tid) {
  constexpr int N = Elem<ET>::N;
  const int wave = tid >> 6, lane = tid & 63;
  fence_regs(hi);
  float ls = 0.f;
#pragma unroll
  for (int k = 0; k < Sweeps<WK>::n; ++k) {
    uint4 zt, zd;
    sweep_vecs<WK>(sh, hi, k, tid, zt, zd);
#pragma unroll
    for (int j = 0; j < N; ++j) ls += elem_weight<ET, WK>(zt, zd, j, c, kt, kd);
  }
  ls = wave_sum(ls);
  if (lane == 0) sh.wt[wave] = ls;
  __syncthreads();
  float W = sh.wt[0];
  for (int w = 1; w < kWaves; ++w) W += sh.wt[w];
  __syncthreads();
  return W;
}

// First element of the item's range (token order: sweep, thread, element)
// whose running weight, starting from `before`, exceeds t; with `fallback`,
// or if rounding leaves no crossing, the range's last positive-weight
// element.  The same value in every thread.
template <typename ET, int WK>
__device__ __forceinline__ int range_search(uint4 (&hi)[kHalfVecs], int base, float c, float kt, float kd,
                                            float before, float t, bool fallback, RShared& sh, int tid) {
  constexpr int N = Elem<ET>::N;
  constexpr int NS = Sweeps<WK>::n;
  const int wave = tid >> 6, lane = tid & 63;
  fence_regs(hi);
  float r[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    r[k] = 0.f;
    uint4 zt, zd;
    sweep_vecs<WK>(sh, hi, k, tid, zt, zd);
#pragma unroll
    for (int j = 0; j < N; ++j) r[k] += elem_weight<ET, WK>(zt, zd, j, c, kt, kd);
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const float v = wave_sum(r[k]);
    if (lane == 0) sh.sw[wave][k] = v;
  }
  __syncthreads();

  // the crossing sweep, with the running sum before it
  int J = -1;
  float run = before, runJ = before;
  if (!fallback) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      float Tk = sh.sw[0][k];
      for (int w = 1; w < kWaves; ++w) Tk += sh.sw[w][k];
      if (J < 0) {
        if (run + Tk > t) {
          J = k;
          runJ = run;
        } else {
          run += Tk;
        }
      }
    }
  }
  int result = -1;
  fence_regs(hi);
  if (J >= 0) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (k == J) v = r[k];
    const float incl = wave_inclusive_scan(v, lane);
    if (lane == 63) sh.wt[wave] = incl;
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    __syncthreads();
    float wb = runJ;
    for (int w = 0; w < wave; ++w) wb += sh.wt[w];
    const float b0 = wb + excl;
    // the vectors of sweep J: lo from LDS, hi selected from registers
    const int kh = (WK == kWPlain) ? J - kHalfVecs : J;
    uint4 zt = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kHalfVecs; ++k)
      if (k == kh) zt = hi[k];
    if (WK == kWResid) zd = sh.park[J][tid];
    if (WK == kWPlain && J < kHalfVecs) zt = sh.park[J][tid];
    keep_raw(zt);  // recompute the weights rather than keep the first pass's alive
    keep_raw(zd);
    int mine = -1;
    float pre = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float w = elem_weight<ET, WK>(zt, zd, j, c, kt, kd);
      pre += w;
      if (mine < 0 && w > 0.f && b0 + pre > t) mine = base + (J * kThreads + tid) * N + j;
    }
    const unsigned long long hit = __ballot(mine >= 0);
    const int found = hit ? __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1, 64) : -1;
    if (lane == 0) sh.wi[wave] = found;
    __syncthreads();
    for (int w = 0; w < kWaves && result < 0; ++w)
      if (sh.wi[w] >= 0) result = sh.wi[w];
  }
  result = uniform(result);
  if (result < 0) {
    // no crossing (rounding, or the chooser's fallback): the last positive-weight element
    fence_regs(hi);
    int last = -1;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      uint4 zt, zd;
      sweep_vecs<WK>(sh, hi, k, tid, zt, zd);
#pragma unroll
      for (int j = 0; j < N; ++j)
        if (elem_weight<ET, WK>(zt, zd, j, c, kt, kd) > 0.f) last = base + (k * kThreads + tid) * N + j;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    __syncthreads();
    if (lane == 0) sh.wi[kWaves + wave] = last;
    __syncthreads();
    result = sh.wi[kWaves];
    for (int w = 1; w < kWaves; ++w) result = max(result, sh.wi[kWaves + w]);
    result = uniform(result);
  }
  __syncthreads();
  return result;
}

// ---------------------------------------------------------------------------
// request words
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t load_mask(const uint32_t* w) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<uint32_t*>(w + kWMask)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_word(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Accept length fixed by the row verdicts in `mask` (bit i: row i has its
// verdict; bit 32 + i: row i was rejected), or -1 while it is open: the first
// rejected row once every row before it was accepted, or K once rows 0..K-1
// were accepted and row K (the bonus row) has its statistics.
__device__ __forceinline__ int decided_a(uint64_t mask, int K) {
  const uint32_t known = uint32_t(mask), rej = uint32_t(mask >> 32);
  const uint32_t acc = known & ~rej;
  const int f = __builtin_ctz(~acc);  // first row not known to be accepted
  if (f < K) return ((known >> f) & (rej >> f) & 1u) ? f : -1;
  return ((known >> K) & 1u) ? K : -1;
}

// Polls (thread 0) the request's verdict mask until `done(mask)`, at most
// spin_limit times; returns the last mask read, in every thread.  Expiry
// (never expected) raises the error flag.
template <typename Done>
__device__ __forceinline__ uint64_t wait_mask(const VerifyArgs& a, const uint32_t* w, Done done, RShared& sh) {
  if (threadIdx.x == 0) {
    uint64_t m = load_mask(w);
    for (uint32_t n = 0; !done(m) && n < a.spin_limit; ++n) {
      __builtin_amdgcn_s_sleep(kWaitSleep);
      m = load_mask(w);
    }
    if (!done(m)) store_dev(&a.ctrl[kCtrlError], 1u);
    sh.mask = m;
  }
  __syncthreads();
  const uint64_t m = sh.mask;
  __syncthreads();
  return (uint64_t(uniform(uint32_t(m >> 32))) << 32) | uniform(uint32_t(m));
}

// Polls (thread 0) the counter *p until it reaches `target`; as wait_mask.
__device__ __forceinline__ void wait_count(const VerifyArgs& a, const uint32_t* p, uint32_t target) {
  if (threadIdx.x == 0) {
    uint32_t v = load_word(p);
    for (uint32_t n = 0; v < target && n < a.spin_limit; ++n) {
      __builtin_amdgcn_s_sleep(kWaitSleep);
      v = load_word(p);
    }
    if (v < target) store_dev(&a.ctrl[kCtrlError], 1u);
  }
  __syncthreads();
}

// Adds one to *p once this workgroup's published stores are complete;
// returns the previous value (thread 0).
__device__ __forceinline__ uint32_t arrive_count(uint32_t* p) {
  drain_stores();
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// row statistics, verdicts and the decision
// ---------------------------------------------------------------------------


// Combines the row's published partials in segment order (loads spread over
// waves 0-2, merged by thread 0) and evaluates position i; the same view in
// every thread.
__device__ __forceinline__ RowView row_view(const VerifyArgs& a, RShared& sh, int b, int i, bool pair, int K,
                                            bool greedy, float c, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int max_k = a.max_k;
  const Partial* pp = &a.partials[(size_t(b) * a.R + i) * a.nseg2];
  const Partial* tp = &a.partials[(size_t(b) * a.R + max_k + i) * a.nseg2];
  const int n = pair ? a.nseg2 : a.nseg;
  const bool test = i < K;
  Partial D{-INFINITY, 0.f, 0.f, 0x7fffffff}, Tg = D;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int m = min(64, n - s0);
    if (wave == 0 && pair && lane < m) sh.cp[0][lane] = fetch(&pp[s0 + lane]);
    if (wave == 1 && lane < m) sh.cp[1][lane] = fetch(&tp[s0 + lane]);
    if (wave == 2 && s0 == 0 && lane < 2 && test && !greedy)
      sh.zv[lane] = load_dev(&a.zval[size_t(b) * a.R + (lane == 0 ? i : max_k + i)]);
    __syncthreads();
    if (tid == 0) {
      for (int k = 0; k < m; ++k) {
        if (pair) merge_ms(D.m, D.s, D.cnt, sh.cp[0][k].m, sh.cp[0][k].s, sh.cp[0][k].cnt, c);
        if (greedy)
          merge_argmax(Tg.m, Tg.idx, sh.cp[1][k].m, sh.cp[1][k].idx);
        else
          merge_ms(Tg.m, Tg.s, Tg.cnt, sh.cp[1][k].m, sh.cp[1][k].s, sh.cp[1][k].cnt, c);
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    RowView v;
    v.D = D;
    v.Tg = Tg;
    v.kt = Tg.m * c + fast_log2(Tg.s + Tg.cnt);
    v.kd = pair ? D.m * c + fast_log2(D.s + D.cnt) : 0.f;
    v.pd = NAN;
    v.pt = NAN;
    v.acc = 1;
    if (test) {
      const int d = a.tokens[size_t(b) * max_k + i];
      if (greedy) {
        v.acc = (d == Tg.idx);
        v.pt = v.acc ? 1.f : 0.f;
      } else {
        const float l2d = (sh.zv[0] - D.m) * c - fast_log2(D.s + D.cnt);
        const float l2t = (sh.zv[1] - Tg.m) * c - fast_log2(Tg.s + Tg.cnt);
        v.pd = fast_exp2(l2d);
        v.pt = fast_exp2(l2t);
        v.acc = (l2d == -INFINITY) || (a.u_accept[size_t(b) * max_k + i] < fast_exp2(l2t - l2d));
      }
    }
    sh.rv = v;
  }
  __syncthreads();
  RowView v = sh.rv;
  __syncthreads();
  v.acc = uniform(v.acc);
  v.kt = uniform(v.kt);
  v.kd = uniform(v.kd);
  return v;
}

// Lowest-index argmax of target row j of request b (thread 0).
__device__ __forceinline__ int row_argmax(const VerifyArgs& a, int b, int j, int n) {
  const Partial* tp = &a.partials[(size_t(b) * a.R + a.max_k + j) * a.nseg2];
  Partial p = fetch(&tp[0]);
  for (int s = 1; s < n; ++s) {
    const Partial q = fetch(&tp[s]);
    merge_argmax(p.m, p.idx, q.m, q.idx);
  }
  return p.idx;
}

// Outputs fixed by the accept length a (run once per request, by the row
// leader whose verdict completed the prefix).  The emitted token of a
// stochastic request is written by the draw.
__device__ __forceinline__ void publish_decision(const VerifyArgs& a, int b, int K, int nd, int aa, bool greedy,
                                                 bool want_feat, int tid) {
  const int max_k = a.max_k;
  if (tid < 64) {
    const int j = tid;
    if (j < max_k) {
      const size_t o = size_t(b) * max_k + j;
      if (a.labels) a.labels[o] = (j < aa) ? 1 : ((j == aa && aa < K) ? 0 : -1);
      if (j >= K) {
        if (a.p_draft) a.p_draft[o] = NAN;
        if (a.p_target) a.p_target[o] = NAN;
        if (want_feat) {
          a.av_feature[o] = NAN;
          if (a.av_score) a.av_score[o] = NAN;
        }
      }
    }
    if (j <= max_k && j != aa) a.out_tokens[size_t(b) * (max_k + 1) + j] = (j < aa) ? a.tokens[size_t(b) * max_k + j] : -1;
    if (j == 0) {
      a.accept_len[b] = aa;
      if (greedy) a.out_tokens[size_t(b) * (max_k + 1) + aa] = row_argmax(a, b, aa, aa < nd ? a.nseg2 : a.nseg);
    }
  }
}


// Weight scan of the draw (wave 0): Z, and the first segment whose running
// weight exceeds u * Z, with the weight before it; every draw item computes
// the same values from the same published weights.
__device__ __forceinline__ Choice scan_segments(const float* segsum, int n, float u, RShared& sh, int tid) {
  const int lane = tid & 63;
  if (tid < 64) {
    float carry = 0.f;
    for (int base = 0; base < n; base += 64) {
      float v = (base + lane < n) ? load_dev(&segsum[base + lane]) : 0.f;
      v = wave_inclusive_scan(v, lane) + carry;
      if (base + lane < n) sh.cum[base + lane] = v;
      carry = __shfl(v, 63, 64);
    }
    if (lane == 0) {
      Choice ch{carry, 0.f, 0.f, -1, 0};
      if (ch.Z > 0.f) {
        ch.t = u * ch.Z;
        int lo = 0, hi = n;  // first k with cum[k] > t
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (sh.cum[mid] > ch.t)
            hi = mid;
          else
            lo = mid + 1;
        }
        int k = lo;
        if (k == n) {  // rounding: the last segment with positive weight
          k = n - 1;
          while (k > 0 && !(sh.cum[k] > sh.cum[k - 1])) --k;
          ch.fb = 1;
        }
        ch.k = k;
        ch.before = k > 0 ? sh.cum[k - 1] : 0.f;
      }
      sh.ch = ch;
    }
  }
  __syncthreads();
  Choice ch = sh.ch;
  __syncthreads();
  ch.k = uniform(ch.k);
  ch.fb = uniform(ch.fb);
  return ch;
}

// ---------------------------------------------------------------------------
// one item
// ---------------------------------------------------------------------------

// Returns, in thread 0, the next claim number taken ahead, kNoClaim, or
// kPlainMismatch (the item needs the other load kind; nothing was done).
template <typename ET, bool PLAIN, bool GREEDY>
__device__ __forceinline__ uint32_t run_item(const VerifyArgs& a, RShared& sh, int b, int slot, uint32_t* counter) {
  const int tid = item_tid(), wave = tid >> 6, lane = tid & 63;
  const int max_k = a.max_k;
  const int K = min(max(a.num_draft[b], 0), max_k);
  const float T = a.temperature[b];
  constexpr bool greedy = GREEDY;
  const bool want_feat = a.av_feature != nullptr;
  const int nd = (!greedy || want_feat) ? K : 0;  // rows read as pairs
  constexpr int E2 = kHalfBytes / int(sizeof(ET));
  const int npair = nd * a.nseg2;
  bool pair;
  int i, s;
  if (slot < npair) {
    pair = true;
    i = slot / a.nseg2;
    s = slot % a.nseg2;
  } else {
    pair = false;
    const int q = slot - npair;
    i = nd + q / a.nseg;
    s = q % a.nseg;
    if (i > K) return kNoClaim;  // slot unused by this request
  }
  const uint32_t n_items = uint32_t(npair) + uint32_t(K + 1 - nd) * uint32_t(a.nseg);
  const float c = kLog2e / (greedy ? 1.f : T);
  const int base = pair ? s * E2 : 2 * s * E2;
  const int hb = pair ? base : base + E2;  // element base of the hi half
  const ET* rt = static_cast<const ET*>(a.target) + (a.target_start[b] + i) * a.target_stride;
  const ET* rd = pair ? static_cast<const ET*>(a.draft) + (a.draft_start[b] + i) * a.draft_stride : rt;
  if (plain_halves<ET>(rd, base, rt, hb, a.V) != PLAIN) return kPlainMismatch;

  uint4 lo[kHalfVecs], hi[kHalfVecs];
  load_halves<ET, PLAIN>(rd, base, rt, hb, a.V, lo, hi, tid);

  // ---- statistics ----
  // Both halves are reduced the same way (lo of a pair item is a draft row,
  // summed even for greedy requests: its sums feed the estimator feature);
  // a single item's two partials are merged afterwards.
  {
    constexpr int MODE = GREEDY ? kArgmax : kSumInclusive;
    Partial p0 = (GREEDY && pair) ? thread_stats<ET, kSumInclusive>(lo, base, c, tid)
                                  : thread_stats<ET, MODE>(lo, base, c, tid);
    Partial p1 = thread_stats<ET, MODE>(hi, hb, c, tid);
    p0 = (GREEDY && pair) ? wave_reduce<kSumInclusive>(p0, c) : wave_reduce<MODE>(p0, c);
    p1 = wave_reduce<MODE>(p1, c);
    if (lane == 0) {
      sh.part[0][wave] = p0;
      sh.part[1][wave] = p1;
    }
    __syncthreads();
    if (tid == 0) {
      p1 = merge_waves<MODE>(sh.part[1], c);
      if (pair) {
        p0 = merge_waves<GREEDY ? kSumInclusive : MODE>(sh.part[0], c);
        publish(&a.partials[(size_t(b) * a.R + i) * a.nseg2 + s], p0);
        if (!GREEDY) {
          const int d = a.tokens[size_t(b) * max_k + i];
          if (d >= base && d < base + E2 && d < a.V) {
            store_dev(&a.zval[size_t(b) * a.R + i], Elem<ET>::one(rd + d));
            store_dev(&a.zval[size_t(b) * a.R + max_k + i], Elem<ET>::one(rt + d));
          }
        }
      } else {
        p0 = merge_waves<MODE>(sh.part[0], c);
        merge_partial<MODE>(p0, p1, c);  // lo precedes hi: ties keep the lower index
        p1 = p0;
      }
      publish(&a.partials[(size_t(b) * a.R + max_k + i) * a.nseg2 + s], p1);
    }
  }
  // park the first half in LDS: only `hi` stays in registers from here on
#pragma unroll
  for (int k = 0; k < kHalfVecs; ++k) sh.park[k][tid] = lo[k];
  fence_regs(hi);

  // ---- the row ----
  // Item 0 of each row leads it: it writes the row's outputs and its verdict
  // bit.  Items that may draw, or may hold a confident row's maximum, wait
  // for their row, then combine its partials themselves.
  uint32_t* w = &a.reqw[size_t(b) * kReqWords];
  const uint32_t n_row = pair ? uint32_t(a.nseg2) : uint32_t(a.nseg);
  const bool leader = s == 0;
  const bool may_draw = !GREEDY && (pair || i == K);
  const bool may_hold = want_feat && pair;
  if (tid == 0) sh.word = int(arrive_count(&w[kWRow + i]));
  __syncthreads();
  const uint32_t before_me = uniform(uint32_t(sh.word));
  __syncthreads();
  uint32_t ahead = kNoClaim;
  bool draw = false;
  float kt = 0.f, kd = 0.f;
  if (leader || may_draw || may_hold) {
    if (before_me + 1 < n_row) wait_count(a, &w[kWRow + i], n_row);
    const RowView v = row_view(a, sh, b, i, pair, K, greedy, c, tid);
    kt = v.kt;
    kd = v.kd;
    const size_t o = size_t(b) * max_k + i;

    // confident draft row: the item holding the first maximum re-sums its half exactly
    if (may_hold && v.D.s < kRecomputeBelow) {
      if (tid == 0) {
        const Partial* pp = &a.partials[(size_t(b) * a.R + i) * a.nseg2];
        int seg = -1;
        float rest = 0.f;
        for (int q = 0; q < a.nseg2; ++q) {
          const Partial p = fetch(&pp[q]);
          if (p.m == v.D.m && seg < 0)
            seg = q;
          else if (p.m != -INFINITY)
            rest += (p.s + p.cnt) * fast_exp2((p.m - v.D.m) * c);
        }
        sh.word = seg;
        sh.fv = rest;
      }
      __syncthreads();
      const int seg = uniform(sh.word);
      const float rest = sh.fv;
      __syncthreads();
      if (seg == s) {
        uint4 u[kHalfVecs];
#pragma unroll
        for (int k = 0; k < kHalfVecs; ++k) u[k] = sh.park[k][tid];
        Partial e = wave_reduce<kSumExclusive>(thread_stats<ET, kSumExclusive>(u, base, c, tid), c);
        if (lane == 0) sh.part[0][wave] = e;
        __syncthreads();
        if (tid == 0) {
          e = merge_waves<kSumExclusive>(sh.part[0], c);
          const float xf = feature_from_other(e.s + (e.cnt - 1.f) + rest);
          a.av_feature[o] = xf;
          if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, xf);
        }
        __syncthreads();
      }
    }

    if (leader) {
      if (tid == 0) {
        if (i < K) {
          if (a.p_draft) a.p_draft[o] = v.pd;
          if (a.p_target) a.p_target[o] = v.pt;
          if (want_feat && pair && v.D.s >= kRecomputeBelow) {
            const float x = feature_from_other(v.D.s - 1.f);
            a.av_feature[o] = x;
            if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, x);
          }
        }
        const uint64_t bits = (uint64_t(1) << i) | ((i < K && !v.acc) ? (uint64_t(1) << (32 + i)) : 0);
        const uint64_t old = __hip_atomic_fetch_or(reinterpret_cast<uint64_t*>(w + kWMask), bits, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        const int an = decided_a(old | bits, K);
        sh.word = (an >= 0 && decided_a(old, K) < 0) ? an : -1;
      }
      __syncthreads();
      const int aa = uniform(sh.word);
      __syncthreads();
      if (aa >= 0) publish_decision(a, b, K, nd, aa, greedy, want_feat, tid);
    }

    // is this row the one the token is drawn from?
    if (may_draw) {
      if (pair && v.acc) {
        draw = false;
      } else if (i == 0) {
        draw = true;  // row 0 rejected, or the bonus row of a request without drafts
      } else {
        // every earlier row must have been accepted
        const uint32_t need = (1u << i) - 1u;
        const uint64_t m = wait_mask(a, w, [&](uint64_t mm) {
          return ((uint32_t(mm) & need) == need) || ((uint32_t(mm >> 32) & uint32_t(mm) & need) != 0);
        }, sh);
        draw = (uint32_t(m) & need) == need && (uint32_t(m >> 32) & need) == 0;
      }
    }
  }
  if (!draw && tid == 0) ahead = claim(counter);  // nothing left to wait for

  // ---- the draw, from registers ----
  if (draw) {
    const int n = pair ? a.nseg2 : a.nseg;
    const float u = pair ? a.u_residual[b] : a.u_bonus[b];
    int wk = pair ? kWResid : kWPlain;
    Choice ch;
    for (int round = 0; round < 2; ++round) {
      const float W = wk == kWResid    ? range_weight<ET, kWResid>(hi, c, kt, kd, sh, tid)
                      : wk == kWTarget ? range_weight<ET, kWTarget>(hi, c, kt, kd, sh, tid)
                                       : range_weight<ET, kWPlain>(hi, c, kt, kd, sh, tid);
      float* seg = &a.segsum[(size_t(round) * a.B + b) * a.nseg2];
      if (tid == 0) {
        store_dev(&seg[s], W);
        arrive_count(&w[kWDraw + round]);
      }
      wait_count(a, &w[kWDraw + round], uint32_t(n));
      ch = scan_segments(seg, n, u, sh, tid);
      if (ch.k >= 0 || wk != kWResid) break;
      wk = kWTarget;  // the residual had no mass (rounding): draw from the target row itself
    }
    if (tid == 0) ahead = claim(counter);
    if (ch.k < 0) {
      if (s == 0 && tid == 0) a.out_tokens[size_t(b) * (max_k + 1) + i] = -1;  // no positive weight at all
    } else if (ch.k == s) {
      const int tok = wk == kWResid    ? range_search<ET, kWResid>(hi, base, c, kt, kd, ch.before, ch.t, ch.fb, sh, tid)
                      : wk == kWTarget ? range_search<ET, kWTarget>(hi, base, c, kt, kd, ch.before, ch.t, ch.fb, sh, tid)
                                       : range_search<ET, kWPlain>(hi, base, c, kt, kd, ch.before, ch.t, ch.fb, sh, tid);
      if (tid == 0) a.out_tokens[size_t(b) * (max_k + 1) + i] = tok;
    }
  }

  // ---- leave the request; the last item out clears its words ----
  if (tid == 0) {
    const uint32_t out = arrive_count(&w[kWDepart]);
    if (out == n_items - 1) {
      for (int k = 0; k <= K; ++k) store_dev(&w[kWRow + k], 0u);
      store_dev(&w[kWMask], 0u);
      store_dev(&w[kWMask + 1], 0u);
      store_dev(&w[kWDepart], 0u);
      store_dev(&w[kWDraw], 0u);
      store_dev(&w[kWDraw + 1], 0u);
    }
  }
  return ahead;
}

template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void resident_kernel(VerifyArgs a) {
  __shared__ RShared sh;
  const int tid = threadIdx.x;
  int p = int(blockIdx.x % uint32_t(a.parts));
  for (int visited = 0; visited < a.parts; ++visited, p = (p + 1) % a.parts) {
    const uint32_t nreq = uint32_t((a.B - p + a.parts - 1) / a.parts);
    const uint32_t total = nreq * uint32_t(a.stride);
    uint32_t* counter = &a.ctrl[kCtrlWork + p * kLineWords];
    if (tid == 0) sh.next = claim(counter);
    __syncthreads();
    uint32_t id = uniform(sh.next);
    __syncthreads();
    while (id < total) {
      const int b = p + int(id / uint32_t(a.stride)) * a.parts;
      const int slot = int(id % uint32_t(a.stride));
      uint32_t ahead;
      if (a.temperature[b] > 0.f) {
        ahead = run_item<ET, true, false>(a, sh, b, slot, counter);
        if (ahead == kPlainMismatch) ahead = run_item<ET, false, false>(a, sh, b, slot, counter);
      } else {
        ahead = run_item<ET, true, true>(a, sh, b, slot, counter);
        if (ahead == kPlainMismatch) ahead = run_item<ET, false, true>(a, sh, b, slot, counter);
      }
      if (tid == 0) sh.next = (ahead == kNoClaim) ? claim(counter) : ahead;
      __syncthreads();
      id = uniform(sh.next);
      __syncthreads();
    }
  }
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kCtrlExit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      for (int q = 0; q < a.parts; ++q) store_dev(&a.ctrl[kCtrlWork + q * kLineWords], 0u);
      store_dev(&a.ctrl[kCtrlExit], 0u);
    }
  }
}

int g_capacity[64][2];

int resident_capacity(int dtype) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int slot = dtype == SV_BF16 ? 1 : 0;
  int cap = __atomic_load_n(&g_capacity[dev][slot], __ATOMIC_RELAXED);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    const hipError_t e1 =
        dtype == SV_BF16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_kernel<uint16_t>, kThreads, 0)
                         : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, resident_kernel<float>, kThreads, 0);
    const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cap = (e1 == hipSuccess && e2 == hipSuccess && per_cu > 0 && cus > 0) ? per_cu * cus : -1;
    __atomic_store_n(&g_capacity[dev][slot], cap, __ATOMIC_RELAXED);
  }
  return cap;
}

}  // namespace

// Item slots a request may need: pair items for rows 0..max_k-1, single
// items for the bonus row.  Requests with fewer pair rows need fewer slots
// (nseg <= nseg2).
int resident_stride(int max_k, int nseg, int nseg2) { return max_k * nseg2 + nseg; }

// Launches the register-resident kernel if the request's items fit the
// resident workgroups with room for progress; returns false otherwise (the
// caller then uses the streaming kernel).
bool launch_resident(VerifyArgs a, int dtype, hipStream_t stream, hipError_t* err) {
  const int cap = resident_capacity(dtype);
  if (cap <= 0) return false;
  a.stride = resident_stride(a.max_k, a.nseg, a.nseg2);
  if (a.nseg2 > kMaxCum) return false;
  // an item waits only for items of its own row and of earlier rows: with
  // more resident workgroups than parts * (row items - 1), one is always free
  const int row_items = a.nseg2;  // >= a.nseg
  int parts = a.B < kParts ? a.B : kParts;
  if (row_items > 1) parts = min(parts, (cap - 1) / (row_items - 1));
  if (parts < 1) return false;
  a.parts = parts;
  a.group = 0;
  const uint64_t nreq = (uint64_t(a.B) + parts - 1) / parts;
  const uint64_t per_part = nreq * uint64_t(a.stride);
  if (per_part + uint64_t(cap) >= (uint64_t(1) << 32)) return false;
  a.spin_limit = 1u << 20;
  const uint64_t all = per_part * uint64_t(parts);
  const unsigned grid = unsigned(all < uint64_t(cap) ? all : uint64_t(cap));
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(resident_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(resident_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, a);
  *err = hipGetLastError();
  return true;
}

}  // namespace sv
