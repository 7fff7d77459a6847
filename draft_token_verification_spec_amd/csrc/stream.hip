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
//   (draft rows 0..K_b-1, target rows 0..K_b), in position order.  Each
//   reduces its segment to (max, sum of exp2((z - max) * c)) - or (max,
//   lowest argmax) for greedy target rows - and publishes it.  The last
//   segment of position i to arrive combines the position's partials,
//   evaluates the accept test of position i, writes the position's outputs
//   and sets the position's bits in the request's verdict mask (bit i:
//   known; bit 32 + i: rejected).  The verdict that fixes the accept length
//   (the first rejection once every earlier position was accepted, or all
//   accepted once the bonus row is known) writes the request's outputs.
//   Nothing waits: a few workgroups per row live slightly longer.
// draw kernel: one workgroup per 32 KiB segment of the rows the token is
//   drawn from (residual: draft and target row a; bonus: target row K_b),
//   read again now that every decision is final.  Each publishes its
//   segment's weight; the request's last one scans the weights, re-reads
//   the segment where the running weight crosses u * total and searches it.
//
// Both kernels are plain grids: the hardware dispatcher keeps every
// compute unit busy, and the statistics kernel's small register footprint
// (8 x 16 bytes of data per thread) gives 8 waves per SIMD to hide memory
// latency behind the exp2 arithmetic.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kNV = 8;  // 16-byte vectors per thread: 32 KiB per workgroup

__device__ __forceinline__ void drain_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// The thread index, opaque to the optimiser: lane addresses are recomputed
// where needed instead of being kept live (and spilled) across the kernel.
__device__ __forceinline__ int fresh_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Vector k of thread t holds elements hb + (k * kThreads + t) * N .. + N-1 of
// its row (token order: vector, thread, element); past the end: -inf.
template <typename ET>
__device__ __forceinline__ void load_seg(const ET* row, int hb, int V, uint4 (&v)[kNV], int) {
  constexpr int N = Elem<ET>::N;
  const int tid = fresh_tid();
  const bool al = is_aligned16(row);
  if (al && hb + kThreads * kNV * N <= V) {
#pragma unroll
    for (int k = 0; k < kNV; ++k) v[k] = load_vec16<ET>(row + hb + (k * kThreads + tid) * N);
  } else {
#pragma unroll
    for (int k = 0; k < kNV; ++k) v[k] = load_raw<ET>(row, hb + (k * kThreads + tid) * N, V, al);
  }
}

__device__ __forceinline__ void fence_regs(uint4 (&v)[kNV]) {
#pragma unroll
  for (int k = 0; k < kNV; ++k) keep_raw(v[k]);
}

// Per-thread statistics of a segment (see Partial).
template <typename ET, int MODE>
__device__ __forceinline__ Partial thread_stats(uint4 (&v)[kNV], int hb, float c, int tid) {
  constexpr int N = Elem<ET>::N;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kNV; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) m = fmaxf(m, Elem<ET>::get(v[k], j));
  if (N == 8) fence_regs(v);
  float s = 0.f, cnt = 0.f;
  int idx = 0x7fffffff;
  if (MODE == kArgmax) {
#pragma unroll
    for (int k = kNV - 1; k >= 0; --k)
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (Elem<ET>::get(v[k], j) == m) idx = hb + (k * kThreads + tid) * N + j;
    if (m == -INFINITY) idx = 0x7fffffff;
  } else if (m != -INFINITY) {
    const float mc = m * c;
#pragma unroll
    for (int k = 0; k < kNV; ++k)
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

// Workgroup reduction of a per-thread Partial; the result in thread 0.
template <int MODE>
__device__ __forceinline__ Partial block_reduce(Partial p, float c, Partial* lds, int tid) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    Partial q;
    q.m = __shfl_xor(p.m, o, 64);
    q.s = __shfl_xor(p.s, o, 64);
    q.cnt = __shfl_xor(p.cnt, o, 64);
    q.idx = __shfl_xor(p.idx, o, 64);
    merge_partial<MODE>(p, q, c);
  }
  if ((tid & 63) == 0) lds[tid >> 6] = p;
  __syncthreads();
  if (tid == 0) {
    p = lds[0];
    for (int w = 1; w < kWaves; ++w) merge_partial<MODE>(p, lds[w], c);
  }
  return p;
}

// ---------------------------------------------------------------------------
// request words and decisions
// ---------------------------------------------------------------------------

// Accept length fixed by the verdict mask, or -1 while it is open.
__device__ __forceinline__ int decided_a(uint64_t mask, int K) {
  const uint32_t known = uint32_t(mask), rej = uint32_t(mask >> 32);
  const uint32_t acc = known & ~rej;
  const int f = __builtin_ctz(~acc);  // first position not known to be accepted
  if (f < K) return ((known >> f) & (rej >> f) & 1u) ? f : -1;
  return ((known >> K) & 1u) ? K : -1;
}

struct StatsShared {
  Partial red[kWaves];
  Partial cp[2][64];
  float zv[2];
  int word;
  float fv;
};

// Outputs fixed by the accept length a (once per request, by the position
// verdict that fixed it).  The token at a of a stochastic request is written
// by the draw kernel; a greedy request's is the argmax of target row a.
__device__ __forceinline__ void publish_decision(const VerifyArgs& a, int b, int K, int aa, bool greedy,
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
      const RowRec* rr = &a.rowrec[size_t(b) * (max_k + 1) + aa];
      Record* rec = &a.records[b];  // read by the draw kernel
      rec->a = aa;
      if (greedy) {
        a.out_tokens[size_t(b) * (max_k + 1) + aa] = load_dev(&rr->argmax);
        rec->mode = kNoDraw;
      } else {
        rec->mode = aa < K ? kResidual : kBonus;
        rec->kt = load_dev(&rr->kt);
        rec->kd = load_dev(&rr->kd);
        rec->u = aa < K ? a.u_residual[b] : a.u_bonus[b];
      }
    }
  }
}

// The last segment of position i: combine, test, outputs, verdict.
template <typename ET>
__device__ __forceinline__ void finish_position(const VerifyArgs& a, StatsShared& sh, int b, int i, int K, bool greedy,
                                                bool want_feat, bool has_draft, float c, uint32_t* w, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int max_k = a.max_k, n = a.nseg2;
  const Partial* pp = &a.partials[(size_t(b) * a.R + i) * a.nseg2];
  const Partial* tp = &a.partials[(size_t(b) * a.R + max_k + i) * a.nseg2];
  const bool test = i < K;
  Partial D{-INFINITY, 0.f, 0.f, 0x7fffffff}, Tg = D;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const int m = min(64, n - s0);
    if (wave == 0 && has_draft && lane < m) sh.cp[0][lane] = fetch(&pp[s0 + lane]);
    if (wave == 1 && lane < m) sh.cp[1][lane] = fetch(&tp[s0 + lane]);
    if (wave == 2 && s0 == 0 && lane < 2 && test && !greedy)
      sh.zv[lane] = load_dev(&a.zval[size_t(b) * a.R + (lane == 0 ? i : max_k + i)]);
    __syncthreads();
    if (tid == 0) {
      for (int k = 0; k < m; ++k) {
        if (has_draft) merge_ms(D.m, D.s, D.cnt, sh.cp[0][k].m, sh.cp[0][k].s, sh.cp[0][k].cnt, c);
        if (greedy)
          merge_argmax(Tg.m, Tg.idx, sh.cp[1][k].m, sh.cp[1][k].idx);
        else
          merge_ms(Tg.m, Tg.s, Tg.cnt, sh.cp[1][k].m, sh.cp[1][k].s, sh.cp[1][k].cnt, c);
      }
    }
    __syncthreads();
  }

  // confident draft row: re-sum the first segment holding the maximum exactly
  if (want_feat && has_draft) {
    if (tid == 0) {
      sh.word = -1;
      sh.fv = 0.f;
      if (D.s < kRecomputeBelow) {
        int seg = -1;
        float rest = 0.f;
        for (int q = 0; q < n; ++q) {
          const Partial p = fetch(&pp[q]);
          if (p.m == D.m && seg < 0)
            seg = q;
          else if (p.m != -INFINITY)
            rest += (p.s + p.cnt) * fast_exp2((p.m - D.m) * c);
        }
        sh.word = seg;
        sh.fv = rest;
      }
    }
    __syncthreads();
    const int seg = uniform(sh.word);
    const float rest = sh.fv;
    __syncthreads();
    if (seg >= 0) {
      constexpr int E = kThreads * kNV * Elem<ET>::N;
      const ET* rd = static_cast<const ET*>(a.draft) + (a.draft_start[b] + i) * a.draft_stride;
      uint4 v[kNV];
      load_seg<ET>(rd, seg * E, a.V, v, tid);
      Partial e = block_reduce<kSumExclusive>(thread_stats<ET, kSumExclusive>(v, seg * E, c, tid), c, sh.red, tid);
      if (tid == 0) {
        const float x = feature_from_other(e.s + (e.cnt - 1.f) + rest);
        const size_t o = size_t(b) * max_k + i;
        a.av_feature[o] = x;
        if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, x);
      }
      __syncthreads();
    }
  }

  if (tid == 0) {
    const size_t o = size_t(b) * max_k + i;
    bool acc = true;
    if (test) {
      const int d = a.tokens[o];
      float pd = NAN, pt;
      if (greedy) {
        acc = (d == Tg.idx);
        pt = acc ? 1.f : 0.f;
      } else {
        const float l2d = (sh.zv[0] - D.m) * c - fast_log2(D.s + D.cnt);
        const float l2t = (sh.zv[1] - Tg.m) * c - fast_log2(Tg.s + Tg.cnt);
        pd = fast_exp2(l2d);
        pt = fast_exp2(l2t);
        acc = (l2d == -INFINITY) || (a.u_accept[o] < fast_exp2(l2t - l2d));
      }
      if (a.p_draft) a.p_draft[o] = pd;
      if (a.p_target) a.p_target[o] = pt;
      if (want_feat && has_draft && D.s >= kRecomputeBelow) {
        const float x = feature_from_other(D.s - 1.f);
        a.av_feature[o] = x;
        if (a.av_score) a.av_score[o] = sigmoid_score(a.av_params, i, x);
      }
    }
    RowRec* rr = &a.rowrec[size_t(b) * (max_k + 1) + i];
    store_dev(&rr->kt, Tg.m * c + fast_log2(Tg.s + Tg.cnt));
    store_dev(&rr->kd, has_draft ? D.m * c + fast_log2(D.s + D.cnt) : 0.f);
    store_dev(&rr->argmax, Tg.idx);
    store_dev(&w[kWRow + i], 0u);  // every segment of the position has arrived
    drain_stores();
    const uint64_t bits = (uint64_t(1) << i) | ((test && !acc) ? (uint64_t(1) << (32 + i)) : 0);
    const uint64_t old = __hip_atomic_fetch_or(reinterpret_cast<uint64_t*>(w + kWMask), bits, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    const int an = decided_a(old | bits, K);
    sh.word = (an >= 0 && decided_a(old, K) < 0) ? an : -1;
  }
  __syncthreads();
  const int aa = uniform(sh.word);
  __syncthreads();
  if (aa >= 0) publish_decision(a, b, K, aa, greedy, want_feat, tid);
}

// One segment: statistics, publication, arrival at its position; the last
// segment of the position finishes it.  Instantiated per statistics mode so
// that the mode choice is taken before the loads.
template <typename ET, int MODE>
__device__ __forceinline__ void stats_segment(const VerifyArgs& a, StatsShared& sh, int b, int i, int s, bool draft,
                                              int K, int nd, bool greedy, bool want_feat, float c, const ET* row,
                                              int d, int tid) {
  const int n = a.nseg2, R = a.R, max_k = a.max_k;
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  const int hb = s * E;
  uint4 v[kNV];
  load_seg<ET>(row, hb, a.V, v, tid);
  const Partial p = block_reduce<MODE>(thread_stats<ET, MODE>(v, hb, c, tid), c, sh.red, tid);

  uint32_t* w = &a.reqw[size_t(b) * kReqWords];
  if (tid == 0) {
    publish(&a.partials[(size_t(b) * R + (draft ? i : max_k + i)) * n + s], p);
    if (!greedy && i < K) {
      if (d >= hb && d < hb + E && d < a.V)
        store_dev(&a.zval[size_t(b) * R + (draft ? i : max_k + i)], Elem<ET>::one(row + d));
    }
    const uint32_t want = uint32_t(n) * (i < nd ? 2u : 1u);
    drain_stores();
    const uint32_t old = __hip_atomic_fetch_add(&w[kWRow + i], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.word = (old + 1 == want) ? 1 : 0;
  }
  __syncthreads();
  if (uniform(sh.word) == 0) return;
  __syncthreads();
  finish_position<ET>(a, sh, b, i, K, greedy, want_feat, i < nd, c, w, tid);
}

// Workgroup = segment s of row slot r (position order: draft i, target i,
// ..., target max_k) of request b.
template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void stats_kernel(VerifyArgs a) {
  __shared__ StatsShared sh;
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
  const bool want_feat = a.av_feature != nullptr;
  const int nd = (!greedy || want_feat) ? K : 0;  // draft rows read
  if (draft ? (i >= nd) : (i > K)) return;
  const float c = kLog2e / (greedy ? 1.f : T);
  const ET* row = draft ? static_cast<const ET*>(a.draft) + (start + i) * a.draft_stride
                        : static_cast<const ET*>(a.target) + (start + i) * a.target_stride;
  if (!draft && greedy)
    stats_segment<ET, kArgmax>(a, sh, b, i, s, draft, K, nd, greedy, want_feat, c, row, d, tid);
  else
    stats_segment<ET, kSumInclusive>(a, sh, b, i, s, draft, K, nd, greedy, want_feat, c, row, d, tid);
}

// ---------------------------------------------------------------------------
// the draw
// ---------------------------------------------------------------------------

struct DrawShared {
  float wt[kWaves];
  float sw[kWaves][kNV];
  int wi[2 * kWaves];
  float cum[256];
  float chunk[kMaxChunks];
  int li[4];
  int word;
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

// Total weight of the segment (same value in every thread).
template <typename ET, bool RESID>
__device__ __forceinline__ float seg_weight(const uint4 (&t)[kNV], const uint4 (&d)[kNV], float c, float kt, float kd,
                                            DrawShared& sh, int tid) {
  constexpr int N = Elem<ET>::N;
  float ls = 0.f;
#pragma unroll
  for (int k = 0; k < kNV; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) ls += elem_w<ET, RESID>(t[k], d[k], j, c, kt, kd);
  ls = wave_sum(ls);
  if ((tid & 63) == 0) sh.wt[tid >> 6] = ls;
  __syncthreads();
  float W = sh.wt[0];
  for (int x = 1; x < kWaves; ++x) W += sh.wt[x];
  __syncthreads();
  return W;
}

// First element of the segment (starting at hb) whose running weight from
// `before` exceeds t; if none (rounding, or `fallback`), the segment's last
// positive-weight element.  The same value in every thread.
template <typename ET, bool RESID>
__device__ __forceinline__ int seg_search(uint4 (&t)[kNV], uint4 (&d)[kNV], int hb, float c, float kt, float kd,
                                          float before, float thr, bool fallback, DrawShared& sh, int tid) {
  constexpr int N = Elem<ET>::N;
  const int wave = tid >> 6, lane = tid & 63;
  float r[kNV];
#pragma unroll
  for (int k = 0; k < kNV; ++k) {
    r[k] = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) r[k] += elem_w<ET, RESID>(t[k], d[k], j, c, kt, kd);
  }
#pragma unroll
  for (int k = 0; k < kNV; ++k) {
    const float x = wave_sum(r[k]);
    if (lane == 0) sh.sw[wave][k] = x;
  }
  __syncthreads();
  int J = -1;
  float run = before, runJ = before;
  if (!fallback) {
#pragma unroll
    for (int k = 0; k < kNV; ++k) {
      float Tk = sh.sw[0][k];
      for (int x = 1; x < kWaves; ++x) Tk += sh.sw[x][k];
      if (J < 0) {
        if (run + Tk > thr) {
          J = k;
          runJ = run;
        } else {
          run += Tk;
        }
      }
    }
  }
  int result = -1;
  if (J >= 0) {
    float vJ = 0.f;
    uint4 zt = {0u, 0u, 0u, 0u}, zd = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kNV; ++k)
      if (k == J) {
        vJ = r[k];
        zt = t[k];
        zd = d[k];
      }
    keep_raw(zt);
    keep_raw(zd);
    const float incl = wave_inclusive_scan(vJ, lane);
    if (lane == 63) sh.wt[wave] = incl;
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    __syncthreads();
    float wb = runJ;
    for (int x = 0; x < wave; ++x) wb += sh.wt[x];
    const float b0 = wb + excl;
    int mine = -1;
    float pre = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float wj = elem_w<ET, RESID>(zt, zd, j, c, kt, kd);
      pre += wj;
      if (mine < 0 && wj > 0.f && b0 + pre > thr) mine = hb + (J * kThreads + tid) * N + j;
    }
    const unsigned long long hit = __ballot(mine >= 0);
    const int found = hit ? __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1, 64) : -1;
    if (lane == 0) sh.wi[wave] = found;
    __syncthreads();
    for (int x = 0; x < kWaves && result < 0; ++x)
      if (sh.wi[x] >= 0) result = sh.wi[x];
  }
  result = uniform(result);
  if (result < 0) {
    fence_regs(t);
    fence_regs(d);
    int last = -1;
#pragma unroll
    for (int k = 0; k < kNV; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j)
        if (elem_w<ET, RESID>(t[k], d[k], j, c, kt, kd) > 0.f) last = hb + (k * kThreads + tid) * N + j;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    __syncthreads();
    if (lane == 0) sh.wi[kWaves + wave] = last;
    __syncthreads();
    result = sh.wi[kWaves];
    for (int x = 1; x < kWaves; ++x) result = max(result, sh.wi[kWaves + x]);
    result = uniform(result);
  }
  __syncthreads();
  return result;
}

// Segment weights published; the last segment scans them: Z, the crossing
// segment k (-1 if Z is not positive), the weight before it, u * Z.
__device__ __forceinline__ void scan_weights(const float* segsum, int n, float u, DrawShared& sh, int tid) {
  const int lane = tid & 63;
  if (tid < 64) {
    float carry = 0.f;
    for (int base = 0; base < n; base += 64) {
      float x = (base + lane < n) ? load_dev(&segsum[base + lane]) : 0.f;
      x = wave_inclusive_scan(x, lane) + carry;
      if (base + lane < n) sh.cum[base + lane] = x;
      carry = __shfl(x, 63, 64);
    }
    if (lane == 0) {
      const float Z = carry;
      int k = -1, fb = 0;
      float thr = 0.f;
      if (Z > 0.f) {
        thr = u * Z;
        int lo = 0, hi = n;  // first k with cum[k] > thr
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (sh.cum[mid] > thr)
            hi = mid;
          else
            lo = mid + 1;
        }
        k = lo;
        if (k == n) {  // rounding: the last segment with positive weight
          k = n - 1;
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

template <typename ET, bool RESID>
__device__ __forceinline__ void draw_segment(const VerifyArgs& a, DrawShared& sh, int b, int s, int aa, float c,
                                             float kt, float kd, float u, const ET* rt, const ET* rd, uint32_t* w,
                                             int tid) {
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  uint4 t[kNV], d[kNV];
  load_seg<ET>(rt, s * E, a.V, t, tid);
  if (RESID) load_seg<ET>(rd, s * E, a.V, d, tid);
  const float W = seg_weight<ET, RESID>(t, d, c, kt, kd, sh, tid);
  float* segsum = &a.segsum[size_t(b) * a.nseg2];
  if (tid == 0) {
    store_dev(&segsum[s], W);
    drain_stores();
    const uint32_t old = __hip_atomic_fetch_add(&w[kWDraw], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.word = (old + 1 == uint32_t(a.nseg2)) ? 1 : 0;
  }
  __syncthreads();
  if (uniform(sh.word) == 0) return;
  if (tid == 0) store_dev(&w[kWDraw], 0u);  // every segment has arrived

  scan_weights(segsum, a.nseg2, u, sh, tid);
  const int k = uniform(sh.fk);
  int tok = -1;
  if (k < 0) {
    // the residual has no mass (reachable only through rounding): draw from pt itself
    if (RESID) tok = cdf_sample<ET, false>(rt, c, kt, rt, c, kt, a.V, u, sh.chunk, sh.li);
  } else {
    if (k != s) {
      load_seg<ET>(rt, k * E, a.V, t, tid);
      if (RESID) load_seg<ET>(rd, k * E, a.V, d, tid);
    }
    tok = seg_search<ET, RESID>(t, d, k * E, c, kt, kd, uniform(sh.fb4), uniform(sh.ft), uniform(sh.ffb) != 0, sh, tid);
  }
  if (tid == 0) a.out_tokens[size_t(b) * (a.max_k + 1) + aa] = tok;
}

// Workgroup = segment s of the draw rows of request b (requests in reverse
// order: the last ones read by the statistics kernel are the likeliest to be
// cached).
template <typename ET>
__global__ __launch_bounds__(kThreads) void draw_kernel(VerifyArgs a) {
  __shared__ DrawShared sh;
  const int tid = threadIdx.x;
  const int n = a.nseg2, max_k = a.max_k;
  const int s = int(blockIdx.x % uint32_t(n));
  const int b = a.B - 1 - int(blockIdx.x / uint32_t(n));
  uint32_t* w = &a.reqw[size_t(b) * kReqWords];
  if (s == 0 && tid == 0) {  // the statistics kernel is over: the verdict mask is free again
    store_dev(&w[kWMask], 0u);
    store_dev(&w[kWMask + 1], 0u);
  }
  // the decision record and the row starts in one round trip
  const Record rec = a.records[b];
  const float T = a.temperature[b];
  const int64_t ts = a.target_start[b];
  const int64_t ds = max_k > 0 ? a.draft_start[b] : 0;
  if (rec.mode != kResidual && rec.mode != kBonus) return;  // greedy requests draw nothing
  const int aa = rec.a;
  const float c = kLog2e / T;
  const ET* rt = static_cast<const ET*>(a.target) + (ts + aa) * a.target_stride;
  if (rec.mode == kResidual) {
    const ET* rd = static_cast<const ET*>(a.draft) + (ds + aa) * a.draft_stride;
    draw_segment<ET, true>(a, sh, b, s, aa, c, rec.kt, rec.kd, rec.u, rt, rd, w, tid);
  } else {
    draw_segment<ET, false>(a, sh, b, s, aa, c, rec.kt, rec.kd, rec.u, rt, rt, w, tid);
  }
}

}  // namespace

hipError_t launch_streaming(VerifyArgs a, int dtype, hipStream_t stream) {
  const uint64_t n1 = uint64_t(a.B) * uint64_t(a.R) * uint64_t(a.nseg2);
  const uint64_t n2 = uint64_t(a.B) * uint64_t(a.nseg2);
  if (n1 == 0) return hipSuccess;
  if (n1 >= (uint64_t(1) << 31)) return hipErrorInvalidValue;
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL(stats_kernel<uint16_t>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(draw_kernel<uint16_t>, dim3(unsigned(n2)), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(stats_kernel<float>, dim3(unsigned(n1)), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(draw_kernel<float>, dim3(unsigned(n2)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sv
