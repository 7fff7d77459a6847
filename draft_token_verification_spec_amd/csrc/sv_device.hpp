// Device building blocks for the verification and scoring kernels (gfx950).
//
// Rows are streamed with 16-byte loads; one thread handles kHalfVecs vectors
// of a 32 KiB segment, strided by the workgroup so that a wave's load covers
// 1 KiB of contiguous memory.  Statistics are kept in fp32 in the base-2
// domain: exp((z - m) / T) = exp2((z - m) * c) with c = log2(e) / T.
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
// row segments
// ---------------------------------------------------------------------------

// What a segment's statistics hold (see Partial): (max, inclusive sum),
// (max, sum without the maximal terms and their count), or (max, lowest
// argmax).
enum SegMode { kSumInclusive = 0, kSumExclusive = 1, kArgmax = 2 };

// Opaque to the optimiser: raw vectors are decoded again after it instead of
// keeping every decoded value alive between two passes over them (for bf16
// that would double the registers held per thread).
__device__ __forceinline__ void keep_raw(uint4& w) { asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w)); }

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


// Loads written before a kernel's first decision go out together when their
// values are pinned there: the compiler otherwise issues each load where its
// value is first needed (a kernel argument pointer, then the value, one round
// trip after another).  pin_all(x...) makes every x available at this point,
// through one word that depends on all of them.
__device__ __forceinline__ uint32_t pin_bits(uint32_t x) { return x; }
__device__ __forceinline__ uint32_t pin_bits(int x) { return uint32_t(x); }
__device__ __forceinline__ uint32_t pin_bits(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t pin_bits(int64_t x) { return uint32_t(x) ^ uint32_t(uint64_t(x) >> 32); }
template <typename... T>
__device__ __forceinline__ void pin_all(const T&... x) {
  const uint32_t w = (pin_bits(x) ^ ...);
  asm volatile("" ::"v"(w));
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

// ---------------------------------------------------------------------------
// the estimator's refit: per-item sums and the damped Newton update
// ---------------------------------------------------------------------------

__device__ __forceinline__ double sigmoid_d(double t) {
  if (t >= 0.0) return 1.0 / (1.0 + exp(-t));
  const double e = exp(t);
  return e / (1.0 + e);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The six sums of one labelled draft (label y in {0, 1}, feature x) at
// parameters (omega, beta_i): n, w, w x, w x^2, r, r x with
// pi = sigmoid(omega x + beta_i), w = pi (1 - pi), r = pi - y; zeros for
// any other label.
__device__ __forceinline__ void fit_item(double omega, double beta_i, float x, int y, double (&v)[6]) {
#pragma unroll
  for (int k = 0; k < 6; ++k) v[k] = 0.0;
  if (y == 0 || y == 1) {
    const double xd = x;
    const double pi = sigmoid_d(omega * xd + beta_i);
    const double w = pi * (1.0 - pi);
    const double r = pi - double(y);
    v[0] = 1.0;
    v[1] = w;
    v[2] = w * xd;
    v[3] = w * xd * xd;
    v[4] = r;
    v[5] = r * xd;
  }
}

// The round's update from its accumulated sums acc[i][k], by the first
// max_k threads of a workgroup (every thread of the workgroup calls it): solve
// the arrowhead system H delta = -g over the slope and the intercepts of
// positions with labels by eliminating the intercepts (Schur complement on
// the slope), damp each step by n / (n + damping_c), scale the whole step so
// that no parameter moves by more than max_step, and add it to params.
// Thread i forms position i's terms; thread 0 adds them in position order.
// A round without labels leaves params unchanged.
struct FitShared {
  double term[SV_MAX_K][5];  // n, the slope's Hessian and gradient terms, Schur and right-hand-side terms
  double step[SV_MAX_K];     // damped intercept steps
  double dw, step_w, shrink;
  int any;
};

__device__ __forceinline__ void fit_update_params(const double (*acc)[6], int max_k, float* params, float damping_c,
                                                  float ridge, float max_step, FitShared& sh, int tid) {
  const double c = damping_c;
  double n = 0.0, D = 1.0, Bi = 0.0, gb = 0.0;
  if (tid < max_k) {
    n = acc[tid][0];
    D = acc[tid][1] + ridge;
    Bi = acc[tid][2];
    gb = acc[tid][4];
    const bool has = n > 0.0;
    sh.term[tid][0] = n;
    sh.term[tid][1] = acc[tid][3];
    sh.term[tid][2] = acc[tid][5];
    sh.term[tid][3] = has ? Bi * Bi / D : 0.0;
    sh.term[tid][4] = has ? Bi * gb / D : 0.0;
  }
  __syncthreads();
  if (tid == 0) {
    double N = 0.0, h = ridge, gw = 0.0, sch = 0.0, r = 0.0;
    for (int i = 0; i < max_k; ++i) {
      N += sh.term[i][0];
      h += sh.term[i][1];
      gw += sh.term[i][2];
      sch += sh.term[i][3];
      r += sh.term[i][4];
    }
    const double schur = h - sch, rhs = r - gw;
    const double dw = (schur > 0.0) ? rhs / schur : 0.0;
    sh.any = N > 0.0;
    sh.dw = dw;
    sh.step_w = dw * (N / (N + c));
  }
  __syncthreads();
  if (!sh.any) return;
  // damped steps, then the whole step scaled so that no parameter moves by
  // more than max_step (far from the optimum, or for a position whose labels
  // all agree, the Newton step on the logistic loss overshoots)
  if (tid < max_k) sh.step[tid] = n > 0.0 ? ((-gb - Bi * sh.dw) / D) * (n / (n + c)) : 0.0;
  __syncthreads();
  if (tid == 0) {
    double largest = fabs(sh.step_w);
    for (int i = 0; i < max_k; ++i) largest = fmax(largest, fabs(sh.step[i]));
    sh.shrink = largest > double(max_step) ? double(max_step) / largest : 1.0;
  }
  __syncthreads();
  if (tid == 0) params[0] = float(double(params[0]) + sh.step_w * sh.shrink);
  if (tid < max_k && n > 0.0) params[1 + tid] = float(double(params[1 + tid]) + sh.step[tid] * sh.shrink);
}

}  // namespace sv
