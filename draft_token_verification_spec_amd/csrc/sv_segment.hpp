// Streaming a row segment and reducing it to its statistics: the building
// blocks of the verification's statistics kernel, shared with the filtered
// verification's statistics pass.
//
// A workgroup of kThreads threads reads one 32 KiB segment: thread t holds
// kNV 16-byte vectors, vector k covering elements hb + (k * kThreads + t) * N
// .. + N - 1 (token order: vector, thread, element), so that a wave's load
// covers 1 KiB of contiguous memory.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int kNV = 8;     // 16-byte vectors per thread: 32 KiB per workgroup

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
// its row (token order: vector, thread, element); past the end: -inf.  The
// rows are streamed (non-temporal loads): each is read once per call, apart
// from the few segments the verdict and the draw read again.
// load_vecs loads vectors K0 .. K0 + NV - 1 of the segment at hb.
template <typename ET, int NV, int K0>
__device__ __forceinline__ void load_vecs(const ET* row, int hb0, int V, uint4 (&v)[NV]) {
  constexpr int N = Elem<ET>::N;
  const int tid = fresh_tid();
  const bool al = is_aligned16(row);
  const int hb = hb0 + K0 * kThreads * N;
  if (al && hb + kThreads * NV * N <= V) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load_stream16(row + hb + (k * kThreads + tid) * N);
  } else if (al && V % N == 0) {
    // the tail of an aligned row: each vector is wholly inside or wholly past
    // the end.  Every lane loads (the row's last vector standing in for one
    // past the end), and only then are the vectors past the end set to -inf,
    // so the loads are issued back to back instead of one branch at a time.
    constexpr uint32_t ninf = N == 8 ? (Elem<ET>::kNegInf << 16 | Elem<ET>::kNegInf) : Elem<ET>::kNegInf;
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load_stream16(row + min(hb + (k * kThreads + tid) * N, V - N));
    const int t = fresh_tid(), lim = (V - hb) / N;  // vectors of the tail
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const bool in = k * kThreads + t < lim;
      v[k].x = in ? v[k].x : ninf;
      v[k].y = in ? v[k].y : ninf;
      v[k].z = in ? v[k].z : ninf;
      v[k].w = in ? v[k].w : ninf;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = load_raw<ET>(row, hb + (k * kThreads + tid) * N, V, al);
  }
}

template <typename ET>
__device__ __forceinline__ void load_seg(const ET* row, int hb, int V, uint4 (&v)[kNV], int) {
  load_vecs<ET, kNV, 0>(row, hb, V, v);
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

// Wave reduction of per-lane (max, sum of exp2((z - max) * c)) pairs: the
// wave maximum first, then each lane's sum rescaled to it (one exp2 per
// lane) and added up.  The result in every lane.
__device__ __forceinline__ void wave_ms(float& m, float& s, float c) {
  float M = m;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  s = wave_sum(m > -INFINITY ? s * fast_exp2((m - M) * c) : 0.f);
  m = M;
}

// Workgroup reduction of a per-thread Partial; the result in thread 0.
template <int MODE>
__device__ __forceinline__ Partial block_reduce(Partial p, float c, Partial* lds, int tid) {
  if (MODE == kSumInclusive) {
    wave_ms(p.m, p.s, c);
  } else {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      Partial q;
      q.m = __shfl_xor(p.m, o, 64);
      q.s = __shfl_xor(p.s, o, 64);
      q.cnt = __shfl_xor(p.cnt, o, 64);
      q.idx = __shfl_xor(p.idx, o, 64);
      merge_partial<MODE>(p, q, c);
    }
  }
  if ((tid & 63) == 0) lds[tid >> 6] = p;
  __syncthreads();
  if (tid == 0) {
    p = lds[0];
    for (int w = 1; w < kWaves; ++w) merge_partial<MODE>(p, lds[w], c);
  }
  return p;
}

// One segment of row slot rs: statistics, stored for the verdict.
// Instantiated per statistics mode so that the mode choice is taken before
// the loads.  Args: the kernel's arguments, with the row length V, the
// layout (R, nseg2) and the outputs partials [B][R][nseg2] and zval [B][R].
template <typename ET, int MODE, typename Args>
__device__ __forceinline__ void stats_segment(const Args& a, Partial* red, int b, int rs, int s, bool ztok, float c,
                                              const ET* row, int d, int tid) {
  constexpr int E = kThreads * kNV * Elem<ET>::N;
  const int hb = s * E;
  float z = 0.f;
  if (ztok && tid == 0) z = Elem<ET>::one(row + d);  // in flight with the segment
  uint4 v[kNV];
  load_seg<ET>(row, hb, a.V, v, tid);
  const Partial p = block_reduce<MODE>(thread_stats<ET, MODE>(v, hb, c, tid), c, red, tid);
  if (tid == 0) {
    a.partials[(size_t(b) * a.R + rs) * a.nseg2 + s] = p;
    if (ztok) a.zval[size_t(b) * a.R + rs] = z;
  }
}

}  // namespace sv
