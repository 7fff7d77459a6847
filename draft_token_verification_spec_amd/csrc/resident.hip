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
constexpr uint32_t kPrefetched = 0xfffffffdu;     // the next item's Meta is in sh.meta

// What every item of row i learns once the row is complete.
struct RowView {
  Partial D, Tg;  // draft (pair rows) and target row statistics
  float kt, kd;   // log2 normalisers: log2 p(v) = z * c - k
  float pd, pt;   // probabilities of the draft token (stochastic rows i < K)
  int acc;        // accept test of position i (1 for the bonus row)
};

// A partition's claim schedule (see decode_claim).
struct Sched {
  int p;              // partition: requests b = p + j * parts
  uint32_t nreq;      // requests of the partition
  uint32_t A, C, L;   // statistics slots, sampling slots per request; sampling lag in requests
  uint32_t total;     // claim numbers of the partition
};

// An item, decoded from its claim number, with its request's scalars.
struct Meta {
  uint32_t id;  // claim number; >= total: the partition is exhausted
  int b, slot, stats;
  int K;
  float T;
  int64_t ts, ds;  // target_row_start[b], draft_row_start[b]
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
  Meta meta;
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

// Loads one half from (r, hb).
template <typename ET, bool PLAIN>
__device__ __forceinline__ void load_half(const ET* r, int hb, int V, uint4 (&v)[kHalfVecs], int tid) {
  constexpr int N = Elem<ET>::N;
  const bool al = is_aligned16(r);
#pragma unroll
  for (int k = 0; k < kHalfVecs; ++k)
    v[k] = PLAIN ? load_vec16<ET>(r + hb + (k * kThreads + tid) * N) : load_raw<ET>(r, hb + (k * kThreads + tid) * N, V, al);
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

// Zeroes request b's words (by its last departing item).
__device__ __forceinline__ void clear_request(uint32_t* w, int K) {
  for (int k = 0; k <= K; ++k) store_dev(&w[kWRow + k], 0u);
  store_dev(&w[kWMask], 0u);
  store_dev(&w[kWMask + 1], 0u);
  store_dev(&w[kWDepart], 0u);
  store_dev(&w[kWDraw], 0u);
  store_dev(&w[kWDraw + 1], 0u);
}

// Departure of a streaming request's row evaluator or sampling item (thread
// 0): the last of the n of them clears the verdict mask.
__device__ __forceinline__ void depart(uint32_t* w, uint32_t n) {
  const uint32_t out = __hip_atomic_fetch_add(&w[kWDepart], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (out == n - 1) {
    store_dev(&w[kWMask], 0u);
    store_dev(&w[kWMask + 1], 0u);
    store_dev(&w[kWDepart], 0u);
  }
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

// The row's outputs and its verdict bit (run once per row, by its leader);
// publishes the request's outputs when this verdict fixed the accept length.
__device__ __forceinline__ void row_verdict(const VerifyArgs& a, RShared& sh, int b, int i, bool pair, int K, int nd,
                                            bool greedy, bool want_feat, const RowView& v, uint32_t* w, int tid) {
  if (tid == 0) {
    const size_t o = size_t(b) * a.max_k + i;
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

// Confident draft row (inclusive sum below kRecomputeBelow): the first half
// segment holding the row maximum, and the other halves' sums scaled to it
// (thread 0; the same values in every thread).
__device__ __forceinline__ void confident_split(const VerifyArgs& a, RShared& sh, int b, int i, float m, float c,
                                                int& seg, float& rest) {
  if (threadIdx.x == 0) {
    const Partial* pp = &a.partials[(size_t(b) * a.R + i) * a.nseg2];
    int sg = -1;
    float r = 0.f;
    for (int q = 0; q < a.nseg2; ++q) {
      const Partial p = fetch(&pp[q]);
      if (p.m == m && sg < 0)
        sg = q;
      else if (p.m != -INFINITY)
        r += (p.s + p.cnt) * fast_exp2((p.m - m) * c);
    }
    sh.word = sg;
    sh.fv = r;
  }
  __syncthreads();
  seg = uniform(sh.word);
  rest = uniform(sh.fv);
  __syncthreads();
}

// Exact feature of draft row i from its half segment `seg` (starting at
// element hb, data in v) and the other halves' sums.
template <typename ET>
__device__ __forceinline__ void exact_feature(const VerifyArgs& a, RShared& sh, int b, int i, uint4 (&v)[kHalfVecs],
                                              int hb, float rest, float c, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  Partial e = wave_reduce<kSumExclusive>(thread_stats<ET, kSumExclusive>(v, hb, c, tid), c);
  if (lane == 0) sh.part[0][wave] = e;
  __syncthreads();
  if (tid == 0) {
    e = merge_waves<kSumExclusive>(sh.part[0], c);
    const float xf = feature_from_other(e.s + (e.cnt - 1.f) + rest);
    const size_t o = size_t(b) * a.max_k + i;
    a.av_feature[o] = xf;
    if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, xf);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// claims
// ---------------------------------------------------------------------------

// Claim number -> item of a partition with nreq requests of A statistics
// slots and C sampling slots: statistics of requests 0..L-1, then statistics
// of request j + L followed by the sampling of request j, then the sampling
// of the last L requests.
__device__ __forceinline__ void decode_claim(uint32_t id, uint32_t nreq, uint32_t A, uint32_t C, uint32_t L,
                                             bool& stats, uint32_t& j, uint32_t& off) {
  if (C == 0) {
    stats = true;
    j = id / A;
    off = id % A;
    return;
  }
  L = min(L, nreq);
  if (id < L * A) {
    stats = true;
    j = id / A;
    off = id % A;
    return;
  }
  const uint32_t q = id - L * A, blk = q / (A + C), r = q % (A + C);
  if (blk < nreq - L) {
    stats = r < A;
    j = stats ? L + blk : blk;
    off = stats ? r : r - A;
    return;
  }
  const uint32_t q2 = q - (nreq - L) * (A + C);
  stats = false;
  j = (nreq - L) + q2 / C;
  off = q2 % C;
}

// Decodes claim number id of partition S and loads its request's scalars
// (thread 0).
__device__ __forceinline__ Meta load_meta(const VerifyArgs& a, const Sched& S, uint32_t id) {
  Meta m;
  m.id = id;
  m.b = -1;
  m.slot = m.stats = m.K = 0;
  m.T = 0.f;
  m.ts = m.ds = 0;
  if (id >= S.total) return m;
  bool st;
  uint32_t j, off;
  decode_claim(id, S.nreq, S.A, S.C, S.L, st, j, off);
  m.b = S.p + int(j) * a.parts;
  m.slot = int(off);
  m.stats = st ? 1 : 0;
  m.K = min(max(a.num_draft[m.b], 0), a.max_k);
  m.T = a.temperature[m.b];
  m.ts = a.target_start[m.b];
  m.ds = a.max_k > 0 ? a.draft_start[m.b] : 0;
  return m;
}

// sh.meta in every thread, as scalars.
__device__ __forceinline__ Meta read_meta(const RShared& sh) {
  Meta m = sh.meta;
  m.id = uniform(m.id);
  m.b = uniform(m.b);
  m.slot = uniform(m.slot);
  m.stats = uniform(m.stats);
  m.K = uniform(m.K);
  m.T = uniform(m.T);
  m.ts = (int64_t(uniform(uint32_t(uint64_t(m.ts) >> 32))) << 32) | uniform(uint32_t(m.ts));
  m.ds = (int64_t(uniform(uint32_t(uint64_t(m.ds) >> 32))) << 32) | uniform(uint32_t(m.ds));
  return m;
}

// ---------------------------------------------------------------------------
// one statistics item
// ---------------------------------------------------------------------------

// HOLD: the register-resident kernel (the item keeps its data until its
// row's verdict, and draws from it); otherwise the item leaves once counted
// in, the last item of the row evaluating it, and the draw re-reads row a in
// separate sampling items.
// Returns, in thread 0, the next claim number taken ahead, kNoClaim, or
// kPlainMismatch (the item needs the other load kind; nothing was done).
template <typename ET, bool PLAIN, bool GREEDY, bool HOLD>
__device__ __forceinline__ uint32_t run_item(const VerifyArgs& a, RShared& sh, const Meta& me, const Sched& S,
                                             uint32_t* counter) {
  const int tid = item_tid(), wave = tid >> 6, lane = tid & 63;
  const int max_k = a.max_k;
  const int b = me.b, slot = me.slot, K = me.K;
  const float T = me.T;
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
  const ET* rt = static_cast<const ET*>(a.target) + (me.ts + i) * a.target_stride;
  const ET* rd = pair ? static_cast<const ET*>(a.draft) + (me.ds + i) * a.draft_stride : rt;
  if (plain_halves<ET>(rd, base, rt, hb, a.V) != PLAIN) return kPlainMismatch;
  uint32_t ahead = kNoClaim;
  if (!HOLD && tid == 0) ahead = claim(counter);  // a streaming item never waits

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
  uint32_t* w = &a.reqw[size_t(b) * kReqWords];
  const uint32_t n_row = pair ? uint32_t(a.nseg2) : uint32_t(a.nseg);
  if (!HOLD) {
    // ---- streaming: count in; the row's last item evaluates it ----
    // Thread 0 loads the next item's scalars while its arrival is in flight.
    Meta nx;
    if (tid == 0) {
      nx = load_meta(a, S, ahead);
      sh.word = int(arrive_count(&w[kWRow + i]));
    }
    __syncthreads();
    const bool last = uniform(uint32_t(sh.word)) + 1 == n_row;
    __syncthreads();
    if (last) {
      const RowView v = row_view(a, sh, b, i, pair, K, greedy, c, tid);
      if (want_feat && pair && v.D.s < kRecomputeBelow) {
        int seg;
        float rest;
        confident_split(a, sh, b, i, v.D.m, c, seg, rest);
        uint4 u[kHalfVecs];
#pragma unroll
        for (int k = 0; k < kHalfVecs; ++k)
          u[k] = load_raw<ET>(rd, seg * E2 + (k * kThreads + tid) * Elem<ET>::N, a.V, is_aligned16(rd));
        exact_feature<ET>(a, sh, b, i, u, seg * E2, rest, c, tid);
      }
      row_verdict(a, sh, b, i, pair, K, nd, greedy, want_feat, v, w, tid);
      // every item of the row has counted in: the counter is free again
      if (tid == 0) {
        store_dev(&w[kWRow + i], 0u);
        depart(w, uint32_t(K + 1) + (GREEDY ? 0u : uint32_t(a.nseg2)));
      }
    }
    if (tid == 0) sh.meta = nx;
    return kPrefetched;
  }

  // park the first half in LDS: only `hi` stays in registers from here on
#pragma unroll
  for (int k = 0; k < kHalfVecs; ++k) sh.park[k][tid] = lo[k];
  fence_regs(hi);

  // ---- the row ----
  // Item 0 of each row leads it: it writes the row's outputs and its verdict
  // bit.  Items that may draw, or may hold a confident row's maximum, wait
  // for their row, then combine its partials themselves.
  const bool leader = s == 0;
  const bool may_draw = !GREEDY && (pair || i == K);
  const bool may_hold = want_feat && pair;
  if (tid == 0) sh.word = int(arrive_count(&w[kWRow + i]));
  __syncthreads();
  const uint32_t before_me = uniform(uint32_t(sh.word));
  __syncthreads();
  bool draw = false;
  float kt = 0.f, kd = 0.f;
  if (leader || may_draw || may_hold) {
    if (before_me + 1 < n_row) wait_count(a, &w[kWRow + i], n_row);
    const RowView v = row_view(a, sh, b, i, pair, K, greedy, c, tid);
    kt = v.kt;
    kd = v.kd;
    // confident draft row: the item holding the first maximum re-sums its half exactly
    if (may_hold && v.D.s < kRecomputeBelow) {
      int seg;
      float rest;
      confident_split(a, sh, b, i, v.D.m, c, seg, rest);
      if (seg == s) {
        uint4 u[kHalfVecs];
#pragma unroll
        for (int k = 0; k < kHalfVecs; ++k) u[k] = sh.park[k][tid];
        exact_feature<ET>(a, sh, b, i, u, base, rest, c, tid);
      }
    }
    if (leader) row_verdict(a, sh, b, i, pair, K, nd, greedy, want_feat, v, w, tid);

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
    if (out == n_items - 1) clear_request(w, K);
  }
  return ahead;
}


// ---------------------------------------------------------------------------
// one sampling item (streaming kernel)
// ---------------------------------------------------------------------------

// Half segment s of the rows request b's token is drawn from: the draft and
// target rows a (residual) or the target row K (bonus).  Publishes its draw
// weight; the request's last sampling item scans the weights, re-reads the
// half segment where the running weight crosses u * total and searches it.
template <typename ET, bool PLAIN>
__device__ __forceinline__ void sample_body(const VerifyArgs& a, RShared& sh, int b, int s, int K, int aa, float c,
                                            uint32_t* w, int tid) {
  constexpr int E2 = kHalfBytes / int(sizeof(ET));
  const int max_k = a.max_k;
  const bool pair = aa < K;
  const ET* rt = static_cast<const ET*>(a.target) + (a.target_start[b] + aa) * a.target_stride;
  const ET* rd = pair ? static_cast<const ET*>(a.draft) + (a.draft_start[b] + aa) * a.draft_stride : rt;
  uint4 lo[kHalfVecs], hi[kHalfVecs];
  if (pair)
    load_halves<ET, PLAIN>(rd, s * E2, rt, s * E2, a.V, lo, hi, tid);
  else
    load_half<ET, PLAIN>(rt, s * E2, a.V, hi, tid);
  const RowView v = row_view(a, sh, b, aa, pair, K, false, c, tid);
  if (pair) {
#pragma unroll
    for (int k = 0; k < kHalfVecs; ++k) sh.park[k][tid] = lo[k];
  }
  const float W = pair ? range_weight<ET, kWResid>(hi, c, v.kt, v.kd, sh, tid)
                       : range_weight<ET, kWTarget>(hi, c, v.kt, v.kd, sh, tid);
  float* seg = &a.segsum[size_t(b) * a.nseg2];
  if (tid == 0) {
    store_dev(&seg[s], W);
    sh.word = int(arrive_count(&w[kWDraw]));
  }
  __syncthreads();
  const bool last = uniform(uint32_t(sh.word)) + 1 == uint32_t(a.nseg2);
  __syncthreads();
  if (!last) return;
  if (tid == 0) store_dev(&w[kWDraw], 0u);  // every sampling item has counted in

  const float u = pair ? a.u_residual[b] : a.u_bonus[b];
  const Choice ch = scan_segments(seg, a.nseg2, u, sh, tid);
  int tok = -1;
  if (ch.k < 0) {
    // the residual has no mass (reachable only through rounding): draw from pt itself
    if (pair)
      tok = cdf_sample<ET, false>(rt, c, v.kt, rt, c, v.kt, a.V, u, reinterpret_cast<float*>(&sh.park[0][0]), sh.wi);
  } else {
    if (ch.k != s) {  // re-read the crossing half segment
      if (plain_halves<ET>(rd, ch.k * E2, rt, ch.k * E2, a.V)) {
        if (pair) load_halves<ET, true>(rd, ch.k * E2, rt, ch.k * E2, a.V, lo, hi, tid);
        else load_half<ET, true>(rt, ch.k * E2, a.V, hi, tid);
      } else {
        if (pair) load_halves<ET, false>(rd, ch.k * E2, rt, ch.k * E2, a.V, lo, hi, tid);
        else load_half<ET, false>(rt, ch.k * E2, a.V, hi, tid);
      }
      __syncthreads();
      if (pair) {
#pragma unroll
        for (int k = 0; k < kHalfVecs; ++k) sh.park[k][tid] = lo[k];
      }
    }
    tok = pair ? range_search<ET, kWResid>(hi, ch.k * E2, c, v.kt, v.kd, ch.before, ch.t, ch.fb, sh, tid)
               : range_search<ET, kWTarget>(hi, ch.k * E2, c, v.kt, v.kd, ch.before, ch.t, ch.fb, sh, tid);
  }
  if (tid == 0) a.out_tokens[size_t(b) * (max_k + 1) + aa] = tok;
}

// Returns, in thread 0, the next claim number taken ahead, or kNoClaim.
template <typename ET>
__device__ __forceinline__ uint32_t sample_item(const VerifyArgs& a, RShared& sh, const Meta& me, const Sched& S,
                                                uint32_t* counter) {
  const int tid = item_tid();
  const int b = me.b, s = me.slot, K = me.K;
  const float T = me.T;
  if (!(T > 0.f)) return kNoClaim;  // greedy requests draw nothing
  constexpr int E2 = kHalfBytes / int(sizeof(ET));
  uint32_t ahead = kNoClaim;
  if (tid == 0) ahead = claim(counter);
  uint32_t* w = &a.reqw[size_t(b) * kReqWords];
  const uint64_t m = wait_mask(a, w, [&](uint64_t mm) { return decided_a(mm, K) >= 0; }, sh);
  const int aa = decided_a(m, K);
  Meta nx;
  if (tid == 0) nx = load_meta(a, S, ahead);
  if (aa >= 0) {  // (an expired wait leaves the token unwritten)
    const bool pair = aa < K;
    const ET* rt = static_cast<const ET*>(a.target) + (me.ts + aa) * a.target_stride;
    const ET* rd = pair ? static_cast<const ET*>(a.draft) + (me.ds + aa) * a.draft_stride : rt;
    if (plain_halves<ET>(rd, s * E2, rt, s * E2, a.V))
      sample_body<ET, true>(a, sh, b, s, K, aa, kLog2e / T, w, tid);
    else
      sample_body<ET, false>(a, sh, b, s, K, aa, kLog2e / T, w, tid);
  }
  if (tid == 0) {
    depart(w, uint32_t(K + 1) + uint32_t(a.nseg2));
    sh.meta = nx;
  }
  return kPrefetched;
}

template <typename ET, bool HOLD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void verify_kernel(VerifyArgs a) {
  __shared__ RShared sh;
  const int tid = threadIdx.x;
  int p = int(blockIdx.x % uint32_t(a.parts));
  for (int visited = 0; visited < a.parts; ++visited, p = (p + 1) % a.parts) {
    Sched S;
    S.p = p;
    S.nreq = uint32_t((a.B - p + a.parts - 1) / a.parts);
    S.A = uint32_t(a.stride);
    S.C = HOLD ? 0u : uint32_t(a.nseg2);
    S.L = 0;
    S.total = S.nreq * (S.A + S.C);
    uint32_t* counter = &a.ctrl[kCtrlWork + p * kLineWords];
    if (tid == 0) sh.meta = load_meta(a, S, claim(counter));
    __syncthreads();
    Meta m = read_meta(sh);
    __syncthreads();
    while (m.id < S.total) {
      uint32_t r;
      if (!m.stats) {
        r = sample_item<ET>(a, sh, m, S, counter);
      } else if (m.T > 0.f) {
        r = run_item<ET, true, false, HOLD>(a, sh, m, S, counter);
        if (r == kPlainMismatch) r = run_item<ET, false, false, HOLD>(a, sh, m, S, counter);
      } else {
        r = run_item<ET, true, true, HOLD>(a, sh, m, S, counter);
        if (r == kPlainMismatch) r = run_item<ET, false, true, HOLD>(a, sh, m, S, counter);
      }
      if (tid == 0 && r != kPrefetched) sh.meta = load_meta(a, S, r == kNoClaim ? claim(counter) : r);
      __syncthreads();
      m = read_meta(sh);
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

// Resident workgroups of the kernel on the current device (occupancy x CUs).
int capacity(int dtype) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int slot = dtype == SV_BF16 ? 1 : 0;
  int cap = __atomic_load_n(&g_capacity[dev][slot], __ATOMIC_RELAXED);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    const hipError_t e1 =
        dtype == SV_BF16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<uint16_t, true>, kThreads, 0)
                         : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, verify_kernel<float, true>, kThreads, 0);
    const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cap = (e1 == hipSuccess && e2 == hipSuccess && per_cu > 0 && cus > 0) ? per_cu * cus : -1;
    __atomic_store_n(&g_capacity[dev][slot], cap, __ATOMIC_RELAXED);
  }
  return cap;
}

}  // namespace

// Statistics slots a request may need: pair items for rows 0..max_k-1, single
// items for the bonus row.  Requests with fewer pair rows need fewer slots
// (nseg <= nseg2).
int stats_stride(int max_k, int nseg, int nseg2) { return max_k * nseg2 + nseg; }

bool launch_verify(VerifyArgs a, int dtype, hipStream_t stream, hipError_t* err, const hipEvent_t* ev) {
  const int cap = capacity(dtype);
  if (cap <= 0) return false;
  a.stride = stats_stride(a.max_k, a.nseg, a.nseg2);
  if (a.nseg2 > kMaxCum) return false;
  int parts = a.B < kParts ? a.B : kParts;
  // an item waits only for items of its own row and of earlier rows: with
  // more resident workgroups than parts * (row items - 1), one is always free
  const int row_items = a.nseg2;  // >= a.nseg
  if (row_items > 1) parts = min(parts, (cap - 1) / (row_items - 1));
  if (parts < 1) return false;
  a.parts = parts;
  const uint64_t nreq = (uint64_t(a.B) + parts - 1) / parts;
  const uint64_t per_part = nreq * uint64_t(a.stride);
  if (per_part + uint64_t(cap) >= (uint64_t(1) << 32)) return false;
  a.spin_limit = 1u << 20;
  const uint64_t all = per_part * uint64_t(parts);
  const unsigned grid = unsigned(all < uint64_t(cap) ? all : uint64_t(cap));
  if (ev) (void)hipEventRecord(ev[0], stream);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL((verify_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((verify_kernel<float, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  *err = hipGetLastError();
  if (ev) {
    (void)hipEventRecord(ev[1], stream);
    (void)hipEventRecord(ev[2], stream);
  }
  return true;
}

}  // namespace sv
