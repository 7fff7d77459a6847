// Device building blocks for the verification and scoring kernels (gfx950).
//
// Rows are streamed with 16-byte loads; one thread handles kVecsPerThread
// vectors of a 64 KiB segment, strided by the workgroup so that a wave's
// load covers 1 KiB of contiguous memory.  Statistics are kept in fp32 in the
// base-2 domain: exp((z - m) / T) = exp2((z - m) * c) with c = log2(e) / T.
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "sv_internal.hpp"

namespace sv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------
//
// A 16-byte vector is kept raw (uint4) and decoded element by element, which
// keeps register use at 4 VGPRs per vector.  Positions past the end of a row
// hold the bit pattern of -inf.

template <typename ET>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bit patterns: 8 per vector
  static constexpr int N = 8;
  static constexpr uint32_t kNegInf = 0xff80u;
  __device__ __forceinline__ static float get(const uint4& w, int j) {
    const uint32_t v = (j >> 1) == 0 ? w.x : (j >> 1) == 1 ? w.y : (j >> 1) == 2 ? w.z : w.w;
    return __uint_as_float((j & 1) ? (v & 0xffff0000u) : (v << 16));
  }
  __device__ __forceinline__ static float one(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
  __device__ __forceinline__ static uint32_t raw(const uint16_t* p) { return *p; }
  __device__ __forceinline__ static void put(uint4& w, int j, uint32_t bits) {
    uint32_t& v = (j >> 1) == 0 ? w.x : (j >> 1) == 1 ? w.y : (j >> 1) == 2 ? w.z : w.w;
    v = (j & 1) ? ((v & 0xffffu) | (bits << 16)) : ((v & 0xffff0000u) | bits);
  }
};

template <>
struct Elem<float> {  // 4 per vector
  static constexpr int N = 4;
  static constexpr uint32_t kNegInf = 0xff800000u;
  __device__ __forceinline__ static float get(const uint4& w, int j) {
    return __uint_as_float(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w);
  }
  __device__ __forceinline__ static float one(const float* p) { return *p; }
  __device__ __forceinline__ static uint32_t raw(const float* p) { return __float_as_uint(*p); }
  __device__ __forceinline__ static void put(uint4& w, int j, uint32_t bits) {
    (j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w) = bits;
  }
};

// The vector holding elements first..first+N-1 of a row; positions >= limit
// read as -inf.  `aligned` says the row start is 16-byte aligned (then a full
// vector is one 16-byte load).
template <typename ET>
__device__ __forceinline__ uint4 load_raw(const ET* row, int first, int limit, bool aligned) {
  constexpr int N = Elem<ET>::N;
  if (aligned && first + N <= limit) return *reinterpret_cast<const uint4*>(row + first);
  uint4 w;
#pragma unroll
  for (int j = 0; j < N; ++j)
    Elem<ET>::put(w, j, (first + j < limit) ? Elem<ET>::raw(row + first + j) : Elem<ET>::kNegInf);
  return w;
}

// Unconditional 16-byte load: the caller guarantees alignment and bounds.
template <typename ET>
__device__ __forceinline__ uint4 load_vec16(const ET* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// The same, streaming: marked non-temporal, for data read once (the
// logit rows of a verification or a distillation step), so that it does not
// displace what the caches hold for other work.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 x = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ bool is_aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// ---------------------------------------------------------------------------
// merging statistics
// ---------------------------------------------------------------------------

// Combine (m, s, cnt) pairs.  Symmetric: both orders give bit-identical
// results, so butterfly reductions leave every lane with the same value.
__device__ __forceinline__ void merge_ms(float& m, float& s, float& cnt, float m2, float s2, float cnt2,
                                         float c) {
  const bool keep = m >= m2;
  const float mh = keep ? m : m2, ml = keep ? m2 : m;
  const float sh = keep ? s : s2, sl = keep ? s2 : s;
  const float ch = keep ? cnt : cnt2, cl = keep ? cnt2 : cnt;
  float ns, nc;
  if (ml == -INFINITY) {
    ns = sh;
    nc = ch;
  } else if (ml == mh) {
    ns = sh + sl;
    nc = ch + cl;
  } else {
    ns = sh + (sl + cl) * fast_exp2((ml - mh) * c);
    nc = ch;
  }
  m = mh;
  s = ns;
  cnt = nc;
}

__device__ __forceinline__ void merge_argmax(float& m, int& idx, float m2, int idx2) {
  if (m2 > m || (m2 == m && idx2 < idx)) {
    m = m2;
    idx = idx2;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Inclusive prefix sum across the wave (Hillis-Steele).
__device__ __forceinline__ float wave_inclusive_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// ---------------------------------------------------------------------------
// one 64 KiB segment of a row -> Partial (valid in thread 0 of the block)
// ---------------------------------------------------------------------------

enum SegMode { kSumInclusive = 0, kSumExclusive = 1, kArgmax = 2 };

// Issue the loads of one segment: thread t takes vectors t, t + kThreads, ...
// of the segment.  Returns true when the fast path (kVecsPerThread plain
// 16-byte loads, nothing else) was taken.
template <typename ET>
__device__ __forceinline__ bool load_segment(const ET* row, int seg_base, int V, bool aligned,
                                             uint4 (&x)[kVecsPerThread]) {
  constexpr int N = Elem<ET>::N;
  const int tid = threadIdx.x;
  if (aligned && seg_base + kThreads * kVecsPerThread * N <= V) {
#pragma unroll
    for (int k = 0; k < kVecsPerThread; ++k) x[k] = load_vec16<ET>(row + seg_base + (k * kThreads + tid) * N);
    return true;
  }
#pragma unroll
  for (int k = 0; k < kVecsPerThread; ++k) x[k] = load_raw<ET>(row, seg_base + (k * kThreads + tid) * N, V, aligned);
  return false;
}

// Reduce a loaded segment to its Partial (valid in thread 0).
// Opaque to the optimiser: the raw vectors are decoded again after it instead
// of keeping every decoded value alive between the two passes (for bf16 that
// would double the registers held per thread).
__device__ __forceinline__ void keep_raw(uint4& w) { asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w)); }

template <typename ET, int MODE>
__device__ __forceinline__ Partial stats_from_regs(uint4 (&x)[kVecsPerThread], int seg_base, float c,
                                                   Partial* lds /* kWaves entries */) {
  constexpr int N = Elem<ET>::N;
  const int tid = threadIdx.x;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kVecsPerThread; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) m = fmaxf(m, Elem<ET>::get(x[k], j));
  if (N == 8) {
#pragma unroll
    for (int k = 0; k < kVecsPerThread; ++k) keep_raw(x[k]);
  }

  float s = 0.f, cnt = 0.f;
  int idx = 0x7fffffff;
  if (MODE == kArgmax) {
#pragma unroll
    for (int k = kVecsPerThread - 1; k >= 0; --k)
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (Elem<ET>::get(x[k], j) == m) idx = seg_base + (k * kThreads + tid) * N + j;
    if (m == -INFINITY) idx = 0x7fffffff;
  } else if (m != -INFINITY) {
    const float mc = m * c;
#pragma unroll
    for (int k = 0; k < kVecsPerThread; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float z = Elem<ET>::get(x[k], j);
        const float e = fast_exp2(fmaf(z, c, -mc));
        if (MODE == kSumExclusive) {
          s += (z < m) ? e : 0.f;
          cnt += (z == m) ? 1.f : 0.f;
        } else {
          s += e;
        }
      }
  }

  // wave butterfly
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    if (MODE == kArgmax) {
      const int i2 = __shfl_xor(idx, o, 64);
      merge_argmax(m, idx, m2, i2);
    } else {
      const float s2 = __shfl_xor(s, o, 64);
      const float c2 = __shfl_xor(cnt, o, 64);
      merge_ms(m, s, cnt, m2, s2, c2, c);
    }
  }
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) lds[wave] = Partial{m, s, cnt, idx};
  __syncthreads();
  Partial p = lds[0];
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) {
      if (MODE == kArgmax)
        merge_argmax(p.m, p.idx, lds[w].m, lds[w].idx);
      else
        merge_ms(p.m, p.s, p.cnt, lds[w].m, lds[w].s, lds[w].cnt, c);
    }
  }
  return p;
}

// Load and reduce one segment (used where no prefetch is needed).
template <typename ET, int MODE>
__device__ __forceinline__ Partial segment_stats(const ET* row, int seg_base, int V, bool aligned, float c,
                                                 Partial* lds) {
  uint4 x[kVecsPerThread];
  load_segment<ET>(row, seg_base, V, aligned, x);
  return stats_from_regs<ET, MODE>(x, seg_base, c, lds);
}

// ---------------------------------------------------------------------------
// publishing results across workgroups
// ---------------------------------------------------------------------------
//
// Workgroups of one request run on different XCDs, whose L2 caches are not
// coherent with each other.  Data handed from one workgroup to another is
// written and read with device-scope (agent) atomic stores and loads, which
// the compiler emits as plain loads/stores with device coherence (sc1):
// written through to, and read from, the device coherence point.  No fence
// is used: an agent-scope release/acquire fence would write back and
// invalidate the whole L2 of the XCD for every workgroup.

__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_dev(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish(Partial* dst, const Partial& p) {
  store_dev(&dst->m, p.m);
  store_dev(&dst->s, p.s);
  store_dev(&dst->cnt, p.cnt);
  store_dev(&dst->idx, p.idx);
}

__device__ __forceinline__ Partial fetch(const Partial* src) {
  return Partial{load_dev(&src->m), load_dev(&src->s), load_dev(&src->cnt), load_dev(&src->idx)};
}

// Arrival counter.  Thread 0 of every workgroup of a request has published
// its results (device-scope stores above); it waits until they are complete,
// then takes a ticket.  The workgroup taking the last ticket (want - 1)
// finishes the request; it reads the published data with device-scope loads
// issued after its ticket returned.  Returns the verdict in all threads.
__device__ __forceinline__ bool arrive_last(uint32_t* ticket, uint32_t want, int* lds_flag) {
  if (threadIdx.x == 0) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0): the published stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    *lds_flag = (__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want - 1) ? 1 : 0;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// Combine the nseg published partials of one row in segment order.
__device__ __forceinline__ Partial combine_published(const Partial* parts, int nseg, float c, bool argmax) {
  Partial p = fetch(&parts[0]);
  for (int s = 1; s < nseg; ++s) {
    const Partial q = fetch(&parts[s]);
    if (argmax)
      merge_argmax(p.m, p.idx, q.m, q.idx);
    else
      merge_ms(p.m, p.s, p.cnt, q.m, q.s, q.cnt, c);
  }
  return p;
}

// ---------------------------------------------------------------------------
// estimator feature of a draft row
// ---------------------------------------------------------------------------
//
// x = logit(q_max) = -log(sum_{v != argmax} exp((z_v - z_max) / T)).  The row
// statistics are inclusive sums S (all terms, the maximum contributing 1), and
// S - 1 is accurate whenever S >= 1.5 (q_max <= 2/3): its relative error is at
// most 3x that of S.  For more confident rows the sum of the other tokens is
// rebuilt exactly: segments whose maximum is below the row maximum keep their
// inclusive partials, and the segment(s) holding the maximum are summed again
// with the maximum's terms counted instead of added.

constexpr float kFeatureClamp = 80.f;
constexpr float kRecomputeBelow = 1.5f;

__device__ __forceinline__ float feature_from_other(float so) {
  return (so > 0.f) ? fminf(-fast_log2(so) * kLn2, kFeatureClamp) : kFeatureClamp;
}

// sigmoid(omega * x + beta_i), params = [omega, beta_0, ...]
__device__ __forceinline__ float sigmoid_score(const float* params, int i, float x) {
  const float t = params[0] * x + params[1 + i];
  return 1.f / (1.f + fast_exp2(-t * kLog2e));
}

// Exact sum of the non-maximal terms of one row (row max m); all threads
// participate, the result is valid in thread 0.  lds: kWaves Partials.
template <typename ET>
__device__ __forceinline__ float exact_other_sum(const ET* row, const Partial* parts, int nseg, int V, float m,
                                                 float c, Partial* lds) {
  constexpr int SEG = kSegBytes / int(sizeof(ET));
  const bool aligned = is_aligned16(row);
  float other = 0.f, cnt = 0.f;
  for (int s = 0; s < nseg; ++s) {
    const Partial q = fetch(&parts[s]);
    if (q.m == m) {
      const Partial e = segment_stats<ET, kSumExclusive>(row, s * SEG, V, aligned, c, lds);
      other += e.s;  // thread 0 holds the reduced value
      cnt += e.cnt;
      __syncthreads();
    } else if (q.m != -INFINITY) {
      other += q.s * fast_exp2((q.m - m) * c);
    }
  }
  return other + (cnt - 1.f);
}

// ---------------------------------------------------------------------------
// inverse-CDF sampling over a full row, by one workgroup
// ---------------------------------------------------------------------------
//
// Weights: w_v = exp2(z_t[v] * ct - kt)                        (bonus / plain)
//          w_v = max(0, exp2(z_t[v] * ct - kt) - exp2(z_d[v] * cd - kd))  (residual)
// i.e. target and draft probabilities when kt = m_t*c + log2(S_t), etc.
// Returns the first v (ascending) whose running sum exceeds u * Z, Z the
// total; if rounding leaves none, the last v with positive weight; -1 if
// Z is not positive.
//
// Layout: a "block" is 64 lanes x N consecutive elements; a "chunk" is cb
// consecutive blocks (a multiple of kGroup) summed by one wave, kGroup blocks
// at a time with all their loads issued together.  Chunk sums go to LDS,
// their prefix locates the chunk holding the crossing, and one wave rescans
// that chunk.

constexpr int kMaxChunks = 1024;

template <typename ET, bool RESID>
__device__ __forceinline__ void cdf_weights(const uint4& zt, const uint4& zd, float ct, float kt, float cd, float kd,
                                            float (&w)[Elem<ET>::N]) {
  constexpr int N = Elem<ET>::N;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float pt = fast_exp2(fmaf(Elem<ET>::get(zt, j), ct, -kt));
    w[j] = RESID ? fmaxf(pt - fast_exp2(fmaf(Elem<ET>::get(zd, j), cd, -kd)), 0.f) : pt;
  }
}

// Loads blocks g..g+kGroup-1 (lane's vector of each) of the target row and,
// for the residual, of the draft row.  When the rows are 16-byte aligned and
// the group lies inside `limit`, all loads are issued back to back.
template <typename ET, bool RESID>
__device__ __forceinline__ void load_group(const ET* rt, const ET* rd, bool fast, int g, int lane, int limit,
                                           uint4 (&zt)[kGroup], uint4 (&zd)[kGroup]) {
  constexpr int N = Elem<ET>::N;
  constexpr int BLK = 64 * N;
  if (fast && (g + kGroup) * BLK <= limit) {
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int first = (g + q) * BLK + lane * N;
      zt[q] = load_vec16<ET>(rt + first);
      if (RESID) zd[q] = load_vec16<ET>(rd + first);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const int first = (g + q) * BLK + lane * N;
      zt[q] = load_raw<ET>(rt, first, limit, fast);
      if (RESID) zd[q] = load_raw<ET>(rd, first, limit, fast);
    }
  }
}

template <typename ET, bool RESID>
__device__ __forceinline__ int cdf_sample(const ET* rt, float ct, float kt, const ET* rd, float cd, float kd, int V, float u,
                          float* chunk_sum /* kMaxChunks */, int* lds_i /* 4 ints */) {
  constexpr int N = Elem<ET>::N;
  constexpr int BLK = 64 * N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool fast = is_aligned16(rt) && (!RESID || is_aligned16(rd));
  const int nblk = (V + BLK - 1) / BLK;
  const int cb = max(kGroup, (((nblk + kMaxChunks - 1) / kMaxChunks) + kGroup - 1) / kGroup * kGroup);
  const int nch = (nblk + cb - 1) / cb;

  // Phase A: chunk sums.  Elements past the chunk's end read as -inf (weight 0).
  for (int ch = wave; ch < nch; ch += kWaves) {
    const int b0 = ch * cb, b1 = min(nblk, b0 + cb);
    const int limit = min(V, b1 * BLK);
    float ls = 0.f;
    for (int g = b0; g < b1; g += kGroup) {
      uint4 zt[kGroup], zd[kGroup];
      load_group<ET, RESID>(rt, rd, fast, g, lane, limit, zt, zd);
#pragma unroll
      for (int q = 0; q < kGroup; ++q) {
        float w[N];
        cdf_weights<ET, RESID>(zt[q], zd[q], ct, kt, cd, kd, w);
#pragma unroll
        for (int j = 0; j < N; ++j) ls += w[j];
      }
    }
    const float tot = wave_sum(ls);
    if (lane == 0) chunk_sum[ch] = tot;
  }
  __syncthreads();

  // Phase B: inclusive prefix of chunk sums (wave 0), then locate the crossing.
  if (wave == 0) {
    float carry = 0.f;
    for (int base = 0; base < nch; base += 64) {
      float v = (base + lane < nch) ? chunk_sum[base + lane] : 0.f;
      v = wave_inclusive_scan(v, lane) + carry;
      if (base + lane < nch) chunk_sum[base + lane] = v;
      carry = __shfl(v, 63, 64);
    }
    if (lane == 0) {
      const float Z = carry;
      int k = -1, fb = 0;
      float t = 0.f;
      if (Z > 0.f) {
        t = u * Z;
        int lo = 0, hi = nch;  // first k with prefix[k] > t
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (chunk_sum[mid] > t) hi = mid; else lo = mid + 1;
        }
        k = lo;
        if (k == nch) {  // rounding: the last chunk with positive mass
          k = nch - 1;
          while (k > 0 && !(chunk_sum[k] > chunk_sum[k - 1])) --k;
          fb = 1;
        }
      }
      lds_i[0] = k;
      lds_i[1] = fb;
      reinterpret_cast<float*>(lds_i)[2] = t;
      reinterpret_cast<float*>(lds_i)[3] = (k > 0) ? chunk_sum[k - 1] : 0.f;
    }
  }
  __syncthreads();
  const int k = lds_i[0];
  if (k < 0) {
    __syncthreads();
    return -1;
  }
  const bool fallback = lds_i[1] != 0;
  const float t = reinterpret_cast<const float*>(lds_i)[2];
  float before = reinterpret_cast<const float*>(lds_i)[3];
  __syncthreads();

  // Phase C: wave 0 rescans chunk k, kGroup blocks at a time.
  if (wave == 0) {
    const int b0 = k * cb, b1 = min(nblk, b0 + cb);
    const int limit = min(V, b1 * BLK);
    int last_pos = -1, result = -1;
    for (int g = b0; g < b1 && result < 0; g += kGroup) {
      uint4 zt[kGroup], zd[kGroup];
      load_group<ET, RESID>(rt, rd, fast, g, lane, limit, zt, zd);
#pragma unroll
      for (int q = 0; q < kGroup; ++q) {
        float w[N];
        cdf_weights<ET, RESID>(zt[q], zd[q], ct, kt, cd, kd, w);
        const int first = (g + q) * BLK + lane * N;
        float run = 0.f, pre[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
          run += w[j];
          pre[j] = run;
          if (w[j] > 0.f) last_pos = max(last_pos, first + j);
        }
        const float incl = wave_inclusive_scan(run, lane);
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0) excl = 0.f;
        const float base = before + excl;
        int mine = -1;
        if (!fallback && result < 0) {
#pragma unroll
          for (int j = N - 1; j >= 0; --j)
            if (w[j] > 0.f && base + pre[j] > t) mine = first + j;
        }
        const unsigned long long hit = __ballot(mine >= 0);
        if (hit && result < 0) {
          const int src = __ffsll(static_cast<long long>(hit)) - 1;
          result = __shfl(mine, src, 64);
        }
        before = before + __shfl(incl, 63, 64);
      }
    }
    if (result < 0) {
      // no crossing inside the chunk (rounding): its last positive-weight element
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) last_pos = max(last_pos, __shfl_xor(last_pos, o, 64));
      result = last_pos;
    }
    if (lane == 0) lds_i[0] = result;
  }
  __syncthreads();
  const int result = lds_i[0];
  __syncthreads();
  return result;
}

// ---------------------------------------------------------------------------
// sampling split over segments
// ---------------------------------------------------------------------------
//
// For the draw, a 32 KiB segment of a row is laid out as kWaves groups of
// kGroup blocks: wave w owns blocks  seg*kSegBlocks + w*kGroup ... +kGroup-1
// (consecutive in vocabulary order).  Every computation of a group's weight
// total uses the same loads and the same order of additions, so the totals
// published by the sampling items and the ones recomputed while searching
// are bit-identical.

constexpr int kSegBlocks = kWaves * kGroup;

template <typename ET, bool RESID>
__device__ __forceinline__ float group_total(const uint4 (&zt)[kGroup], const uint4 (&zd)[kGroup], float ct,
                                             float kt, float cd, float kd) {
  constexpr int N = Elem<ET>::N;
  float ls = 0.f;
#pragma unroll
  for (int q = 0; q < kGroup; ++q) {
    float w[N];
    cdf_weights<ET, RESID>(zt[q], zd[q], ct, kt, cd, kd, w);
#pragma unroll
    for (int j = 0; j < N; ++j) ls += w[j];
  }
  return wave_sum(ls);
}

// Weight total of segment `seg` (valid in thread 0).  lds: kWaves floats.
template <typename ET, bool RESID>
__device__ __forceinline__ float segment_weight(const ET* rt, const ET* rd, bool fast, int seg, int V, float ct,
                                                float kt, float cd, float kd, float* lds) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint4 zt[kGroup], zd[kGroup];
  load_group<ET, RESID>(rt, rd, fast, seg * kSegBlocks + wave * kGroup, lane, V, zt, zd);
  const float g = group_total<ET, RESID>(zt, zd, ct, kt, cd, kd);
  if (lane == 0) lds[wave] = g;
  __syncthreads();
  float W = 0.f;
  if (tid == 0)
    for (int w = 0; w < kWaves; ++w) W += lds[w];
  return W;
}

// First element v of segment `seg` whose running weight sum, starting from
// `before`, exceeds t (the sums of the groups in order, then element by
// element inside the crossing group).  If rounding leaves no crossing
// (`fallback`, or none found), returns the segment's last positive-weight
// element.  Returns the same value in all threads.  lds: kWaves floats,
// ldsi: 2 * kWaves ints.
template <typename ET, bool RESID>
__device__ __forceinline__ int segment_search(const ET* rt, const ET* rd, bool fast, int seg, int V, float ct, float kt,
                                              float cd, float kd, float before, float t, bool fallback, float* lds,
                                              int* ldsi) {
  constexpr int N = Elem<ET>::N;
  constexpr int BLK = 64 * N;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int blk0 = seg * kSegBlocks + wave * kGroup;
  {
    uint4 zt[kGroup], zd[kGroup];
    load_group<ET, RESID>(rt, rd, fast, blk0, lane, V, zt, zd);
    const float g = group_total<ET, RESID>(zt, zd, ct, kt, cd, kd);
    if (lane == 0) lds[wave] = g;
  }
  __syncthreads();

  // the crossing group, and the running sum before it (same order everywhere)
  int cw = -1;
  float base = before;
  if (!fallback) {
    float cum = before;
    for (int w = 0; w < kWaves; ++w) {
      if (cum + lds[w] > t) {
        cw = w;
        base = cum;
        break;
      }
      cum += lds[w];
    }
  }
  int last_pos = -1, found = -1;
  if (cw < 0 || cw == wave) {
    // reload the group (cache-hot) rather than keep it in registers across the barrier
    uint4 zt[kGroup], zd[kGroup];
    load_group<ET, RESID>(rt, rd, fast, blk0, lane, V, zt, zd);
    float run_base = base;
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      float w[N];
      cdf_weights<ET, RESID>(zt[q], zd[q], ct, kt, cd, kd, w);
      const int first = (blk0 + q) * BLK + lane * N;
      float run = 0.f, pre[N];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        run += w[j];
        pre[j] = run;
        if (w[j] > 0.f) last_pos = max(last_pos, first + j);
      }
      const float incl = wave_inclusive_scan(run, lane);
      float excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.f;
      int mine = -1;
      if (cw == wave && found < 0) {
#pragma unroll
        for (int j = N - 1; j >= 0; --j)
          if (w[j] > 0.f && run_base + excl + pre[j] > t) mine = first + j;
      }
      const unsigned long long hit = __ballot(mine >= 0);
      if (hit && found < 0) found = __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1, 64);
      run_base += __shfl(incl, 63, 64);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) last_pos = max(last_pos, __shfl_xor(last_pos, o, 64));
  }
  if (lane == 0) {
    ldsi[wave] = (cw == wave) ? found : -1;  // crossing element of this group, if any
    ldsi[kWaves + wave] = last_pos;           // its last positive-weight element
  }
  __syncthreads();
  int result;
  if (cw >= 0 && ldsi[cw] >= 0) {
    result = ldsi[cw];
  } else if (cw >= 0) {
    // rounding left no crossing inside the crossing group
    result = ldsi[kWaves + cw];
  } else {
    // no group crossed: the last positive-weight element of the segment
    result = -1;
    for (int w = 0; w < kWaves; ++w) result = max(result, ldsi[kWaves + w]);
  }
  __syncthreads();
  return result;
}

}  // namespace sv
