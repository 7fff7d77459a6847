// The test-time-speculation distillation gradient over the canvas.
//
// Page "ملخص تقني: التخمين في وقت الاختبار (TTS)", section "Algorithm",
// step 3: one gradient step of the draft model on
//   L_t(q) = KL~(p || q) + lambda * KL~(q_t || q)
// with position weights w_k over the canvas.  For canvas position k of
// request b (k < K_b) the kernel writes the gradient with respect to the
// draft logits z, w_k * ((q - p) + lambda * (q - q_t)) / T, and the loss
// w_k * (KL(p || q) + lambda * KL(q_t || q)), every distribution being
// softmax(logits / T) (T = 0 counting as 1).
//
// One workgroup per canvas position: a statistics pass (online max and sum
// of exp2 per row, each thread over its share, then the workgroup; 32
// elements per row and thread in flight per step) and a gradient pass over
// the same rows (16 per row and thread per step).  HBM-bound: the rows are read twice, the gradient row written
// once.
#include "sv_device.hpp"

namespace sv {

namespace {

constexpr int kTT = 256;  // threads
// 16-byte vectors per row and thread per step: 16 elements of either type
// in the gradient pass, 32 in the statistics pass (which holds no gradient)
template <typename ET>
constexpr int kTV = 16 / Elem<ET>::N;
template <typename ET>
constexpr int kTVS = 32 / Elem<ET>::N;
constexpr float kLn2 = 0.6931471805599453f;

// Vectors base/N + k * kTT + t (k < kTV) of a row for thread t: elements
// base + (k * kTT + t) * N .. + N - 1; past V: -inf.
// The rows are streamed (non-temporal loads): the two passes over a row
// are too far apart for the caches to keep it.
template <typename ET, int TV>
__device__ __forceinline__ void load_step(const ET* row, int base, int V, uint4 (&v)[TV], int tid) {
  constexpr int N = Elem<ET>::N;
  const bool al = is_aligned16(row);
  if (al && base + kTT * TV * N <= V) {
#pragma unroll
    for (int k = 0; k < TV; ++k) v[k] = load_stream16(row + base + (k * kTT + tid) * N);
  } else {
#pragma unroll
    for (int k = 0; k < TV; ++k) v[k] = load_raw<ET>(row, base + (k * kTT + tid) * N, V, al);
  }
}

// Online (max, sum of exp2((z - max) * c)) of one thread's elements.
template <typename ET, int TV>
__device__ __forceinline__ void online(const uint4 (&v)[TV], float c, float& m, float& s) {
  constexpr int N = Elem<ET>::N;
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < TV; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) mx = fmaxf(mx, Elem<ET>::get(v[k], j));
  if (mx == -INFINITY) return;
  const float mn = fmaxf(m, mx);
  float acc = (m == -INFINITY) ? 0.f : s * fast_exp2((m - mn) * c);
#pragma unroll
  for (int k = 0; k < TV; ++k)
#pragma unroll
    for (int j = 0; j < N; ++j) acc += fast_exp2(fmaf(Elem<ET>::get(v[k], j), c, -mn * c));
  m = mn;
  s = acc;
}

// log2 normaliser of a row over the workgroup: log2 softmax(z / T)(v) = z c - k.
__device__ __forceinline__ float block_norm(float m, float s, float c, float* red_m, float* red_s, int tid) {
  float cnt = 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64), c2 = 0.f;
    merge_ms(m, s, cnt, m2, s2, c2, c);
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_s[tid >> 6] = s;
  }
  __syncthreads();
  float M = red_m[0], S = red_s[0], C = 0.f;
  for (int w = 1; w < kTT / 64; ++w) merge_ms(M, S, C, red_m[w], red_s[w], 0.f, c);
  __syncthreads();
  return M * c + fast_log2(S);
}

__device__ __forceinline__ float block_total(float x, float* red, int tid) {
  x = wave_sum(x);
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < kTT / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Streaming 16-byte store: a gradient row is written once and not read
// back here, so it is not kept in the caches.
__device__ __forceinline__ void store_stream16(void* p, uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  const u32x4 v = {x, y, z, w};
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
}

// Round to bfloat16 (nearest, ties to even), as bits.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename ET>
__device__ __forceinline__ void store_grad(ET* out, int first, int V, const float (&g)[Elem<ET>::N], bool vec);

template <>
__device__ __forceinline__ void store_grad<uint16_t>(uint16_t* out, int first, int V, const float (&g)[8], bool vec) {
  if (vec && first + 8 <= V) {
    store_stream16(out + first, to_bf16(g[0]) | (to_bf16(g[1]) << 16), to_bf16(g[2]) | (to_bf16(g[3]) << 16),
                   to_bf16(g[4]) | (to_bf16(g[5]) << 16), to_bf16(g[6]) | (to_bf16(g[7]) << 16));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (first + j < V) out[first + j] = uint16_t(to_bf16(g[j]));
  }
}

template <>
__device__ __forceinline__ void store_grad<float>(float* out, int first, int V, const float (&g)[4], bool vec) {
  if (vec && first + 4 <= V) {
    store_stream16(out + first, __float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                   __float_as_uint(g[3]));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (first + j < V) out[first + j] = g[j];
  }
}

struct TtsArgs {
  int B, V, max_k;
  const void* draft;
  const int64_t* draft_start;
  int64_t draft_stride;
  const void* target;
  const int64_t* target_start;
  int64_t target_stride;
  const void* prev;  // null: the draft rows
  const int64_t* prev_start;
  int64_t prev_stride;
  const int32_t* num_draft;
  const float* temperature;
  const float* weights;
  float lambda;
  void* grad;
  float* loss;
  // row statistics of a preceding sv_spec_verify call on the same rows
  // (its workspace's segment partials), or null
  Partial* stats;
  float* loss_parts;  // [B][max_k][nseg2] (segmented kernel)
  uint32_t* tickets;  // arrival counters per request slot (segmented kernel)
  int R, nseg2;
};

// log2 normaliser of a row from its segment partials (in segment order).
__device__ __forceinline__ float stats_norm(const Partial* p, int n, float c, float* red_m, float* red_s, int tid) {
  float m = -INFINITY, s = 0.f, cnt = 0.f;
  for (int q = tid; q < n; q += kTT) {
    const Partial x = p[q];
    merge_ms(m, s, cnt, x.m, x.s + x.cnt, 0.f, c);
  }
  return block_norm(m, s, c, red_m, red_s, tid);
}

template <typename ET, bool PREV, bool REUSE>
__device__ __forceinline__ void tts_position(const TtsArgs& a, const ET* rd, const ET* rt, const ET* rp, float c,
                                             float invT, float w, ET* g, size_t o, int b, int kpos, int tid) {
  constexpr int N = Elem<ET>::N;
  constexpr int TV = kTV<ET>;
  constexpr int STEP = kTT * TV * N;
  __shared__ float red_m[kTT / 64], red_s[kTT / 64];
  const int V = a.V;
  // statistics: a pass over the rows, or (REUSE) the verification's
  // partials of the draft and target rows and a pass over q_t's rows only
  float md = -INFINITY, sd = 0.f, mt = -INFINITY, st = 0.f, mp = -INFINITY, sp = 0.f;
  if (!REUSE || PREV) {
    constexpr int TS = kTVS<ET>;
    for (int base = 0; base < V; base += kTT * TS * N) {
      uint4 vd[TS], vt[TS], vp[TS];
      if (!REUSE) {
        load_step<ET, TS>(rd, base, V, vd, tid);
        load_step<ET, TS>(rt, base, V, vt, tid);
      }
      if (PREV) load_step<ET, TS>(rp, base, V, vp, tid);
      if (!REUSE) {
        online<ET, TS>(vd, c, md, sd);
        online<ET, TS>(vt, c, mt, st);
      }
      if (PREV) online<ET, TS>(vp, c, mp, sp);
    }
  }
  float kd, kt;
  if (REUSE) {
    const Partial* base = a.stats + size_t(b) * a.R * a.nseg2;
    kd = stats_norm(base + size_t(kpos) * a.nseg2, a.nseg2, c, red_m, red_s, tid);
    kt = stats_norm(base + size_t(a.max_k + kpos) * a.nseg2, a.nseg2, c, red_m, red_s, tid);
  } else {
    kd = block_norm(md, sd, c, red_m, red_s, tid);
    kt = block_norm(mt, st, c, red_m, red_s, tid);
  }
  const float kp = PREV ? block_norm(mp, sp, c, red_m, red_s, tid) : kd;
  // gradient and loss (log2 units until the end)
  const float lam = a.lambda;
  const bool vec = is_aligned16(g);
  float loss = 0.f;
  for (int base = 0; base < V; base += STEP) {
    uint4 vd[TV], vt[TV], vp[TV];
    load_step<ET, TV>(rd, base, V, vd, tid);
    load_step<ET, TV>(rt, base, V, vt, tid);
    if (PREV) load_step<ET, TV>(rp, base, V, vp, tid);
#pragma unroll
    for (int k = 0; k < TV; ++k) {
      float gv[N];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float lq = fmaf(Elem<ET>::get(vd[k], j), c, -kd);
        const float lp = fmaf(Elem<ET>::get(vt[k], j), c, -kt);
        const float q = fast_exp2(lq), p = fast_exp2(lp);
        float qt = q, lqt = lq;
        if (PREV) {
          lqt = fmaf(Elem<ET>::get(vp[k], j), c, -kp);
          qt = fast_exp2(lqt);
        }
        gv[j] = w * ((q - p) + lam * (q - qt)) * invT;
        loss += (p > 0.f ? p * (lp - lq) : 0.f) + (PREV && qt > 0.f ? lam * qt * (lqt - lq) : 0.f);
      }
      store_grad<ET>(g, base + (k * kTT + tid) * N, V, gv, vec);
    }
  }
  loss = block_total(loss, red_m, tid);
  if (tid == 0) a.loss[o] = w * kLn2 * loss;
}

template <typename ET, bool PREV, bool REUSE>
__global__ __launch_bounds__(kTT) __attribute__((amdgpu_waves_per_eu(4))) void tts_grad_kernel(TtsArgs a) {
  const int tid = threadIdx.x;
  const int b = int(blockIdx.x / uint32_t(a.max_k)), k = int(blockIdx.x % uint32_t(a.max_k));
  const size_t o = size_t(b) * a.max_k + k;
  const int K = min(max(a.num_draft[b], 0), a.max_k);
  if (k >= K) {
    if (tid == 0) a.loss[o] = NAN;
    return;
  }
  const float T0 = a.temperature[b];
  const float T = T0 > 0.f ? T0 : 1.f;
  const float c = kLog2e / T;
  const float w = a.weights[k];
  const ET* rd = static_cast<const ET*>(a.draft) + (a.draft_start[b] + k) * a.draft_stride;
  const ET* rt = static_cast<const ET*>(a.target) + (a.target_start[b] + k) * a.target_stride;
  ET* g = static_cast<ET*>(a.grad) + o * size_t(a.V);
  const ET* rp = PREV ? static_cast<const ET*>(a.prev) + (a.prev_start[b] + k) * a.prev_stride : rd;
  tts_position<ET, PREV, REUSE>(a, rd, rt, rp, c, 1.f / T, w, g, o, b, k, tid);
}

// The gradient by row segments, with the draft and target rows' statistics
// taken from the verification: workgroup (position, segment s) reads 32 KiB
// of each row (in two 16 KiB halves) and writes its slice of the gradient
// row.  Its loss goes to loss_parts; the last workgroup of a request to
// arrive sums each position's segment losses in segment order, so the loss
// does not depend on the arrival order.
// log2 normaliser of a row from its segment partials, merged by one wave
// (merge_ms is symmetric, so every lane and every wave gets the same value).
__device__ __forceinline__ float wave_stats_norm(const Partial* p, int n, float c, int lane) {
  float m = -INFINITY, s = 0.f, cnt = 0.f;
  for (int q = lane; q < n; q += 64) {
    const Partial x = p[q];
    merge_ms(m, s, cnt, x.m, x.s + x.cnt, 0.f, c);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    merge_ms(m, s, cnt, m2, s2, 0.f, c);
  }
  return m * c + fast_log2(s);
}

template <typename ET>
__global__ __launch_bounds__(kTT) void tts_seg_kernel(TtsArgs a) {
  constexpr int N = Elem<ET>::N;
  constexpr int HALF = 4;                // vectors per row and thread per half
  constexpr int HE = kTT * HALF * N;     // elements per half (16 KiB)
  constexpr int E = 2 * HE;              // elements per segment (32 KiB)
  __shared__ float red[kTT / 64];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int n = a.nseg2;
  const uint32_t pos = blockIdx.x / uint32_t(n);
  const int s = int(blockIdx.x % uint32_t(n));
  const int b = int(pos / uint32_t(a.max_k)), k = int(pos % uint32_t(a.max_k));
  const size_t o = size_t(b) * a.max_k + k;
  const int K = min(max(a.num_draft[b], 0), a.max_k);
  if (k >= K) {
    if (s == 0 && tid == 0) a.loss[o] = NAN;
    return;
  }
  const ET* rd = static_cast<const ET*>(a.draft) + (a.draft_start[b] + k) * a.draft_stride;
  const ET* rt = static_cast<const ET*>(a.target) + (a.target_start[b] + k) * a.target_stride;
  // aligned rows of a whole number of vectors: every vector is wholly inside
  // the row or wholly past its end
  const bool vec_rows = is_aligned16(rd) && is_aligned16(rt) && a.V % N == 0;
  uint4 vd[HALF], vt[HALF];
  // Vectors of a half at hb.  Past the end of the row every lane still loads
  // (the row's last vector standing in) and only then are those vectors set
  // to -inf, so that the loads are issued back to back.
  auto load_half = [&](int hb) {
    if (hb + HE <= a.V) {
#pragma unroll
      for (int q = 0; q < HALF; ++q) {
        vd[q] = load_stream16(rd + hb + (q * kTT + tid) * N);
        vt[q] = load_stream16(rt + hb + (q * kTT + tid) * N);
      }
    } else {
      constexpr uint32_t ninf = N == 8 ? (Elem<ET>::kNegInf << 16 | Elem<ET>::kNegInf) : Elem<ET>::kNegInf;
#pragma unroll
      for (int q = 0; q < HALF; ++q) {
        const int e = hb + (q * kTT + tid) * N;
        vd[q] = load_stream16(rd + min(e, a.V - N));
        vt[q] = load_stream16(rt + min(e, a.V - N));
      }
#pragma unroll
      for (int q = 0; q < HALF; ++q)
        if (hb + (q * kTT + tid) * N >= a.V) vd[q] = vt[q] = make_uint4(ninf, ninf, ninf, ninf);
    }
  };
  // the first half's rows are in flight while the normalisers are merged
  if (vec_rows) load_half(s * E);
  const float T0 = a.temperature[b];
  const float T = T0 > 0.f ? T0 : 1.f;
  const float c = kLog2e / T, invT = 1.f / T;
  const float w = a.weights[k];
  const Partial* base = a.stats + size_t(b) * a.R * n;
  const float kd = wave_stats_norm(base + size_t(k) * n, n, c, tid & 63);
  const float kt = wave_stats_norm(base + size_t(a.max_k + k) * n, n, c, tid & 63);
  ET* g = static_cast<ET*>(a.grad) + o * size_t(a.V);
  const bool vec = is_aligned16(g);
  float loss = 0.f;
  auto grad_vec = [&](const uint4& zd, const uint4& zt, int first) {
    float gv[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const float lq = fmaf(Elem<ET>::get(zd, j), c, -kd);
      const float lp = fmaf(Elem<ET>::get(zt, j), c, -kt);
      const float qv = fast_exp2(lq), pv = fast_exp2(lp);
      gv[j] = w * (qv - pv) * invT;
      loss += pv > 0.f ? pv * (lp - lq) : 0.f;
    }
    // the loss terms are added here: left to the scheduler, they sink past
    // the store's branches and hold every element's terms live (160 VGPRs)
    asm volatile("" : "+v"(loss));
    store_grad<ET>(g, first, a.V, gv, vec);
  };
  if (vec_rows) {
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      const int hb = s * E + h * HE;
      if (h) load_half(hb);
#pragma unroll
      for (int q = 0; q < HALF; ++q) grad_vec(vd[q], vt[q], hb + (q * kTT + tid) * N);
    }
  } else {
    // rows that are not 16-byte aligned, or of a length that is no whole
    // number of vectors: element loads, one vector at a time
    const bool ald = is_aligned16(rd), alt = is_aligned16(rt);
#pragma unroll 1
    for (int q = 0; q < 2 * HALF; ++q) {
      const int first = s * E + (q * kTT + tid) * N;
      grad_vec(load_raw<ET>(rd, first, a.V, ald), load_raw<ET>(rt, first, a.V, alt), first);
    }
  }
  loss = block_total(loss, red, tid);
  if (tid == 0) store_dev(&a.loss_parts[o * n + s], w * kLn2 * loss);
  uint32_t* ticket = &a.tickets[req_slot(b)];
  if (!arrive_last(ticket, uint32_t(n) * uint32_t(K), &last)) return;
  if (tid < K) {
    const float* lp = a.loss_parts + (size_t(b) * a.max_k + tid) * n;
    float total = 0.f;
    for (int q = 0; q < n; ++q) total += load_dev(&lp[q]);
    a.loss[size_t(b) * a.max_k + tid] = total;
  }
  if (tid == 0) store_dev(ticket, 0u);
}

// A greedy request's target rows hold only (maximum, lowest argmax) per
// segment in the verification's statistics; the gradient needs their
// softmax sums (T = 0 counting as 1).  Workgroup (b, k): for a greedy
// request and k < K_b, target row k is summed segment by segment, each
// against the maximum its statistics already hold, and the sums are written
// beside them; the workgroups of other rows leave at once.
template <typename ET>
__global__ __launch_bounds__(kTT) void greedy_target_sums_kernel(TtsArgs a) {
  constexpr int N = Elem<ET>::N;
  constexpr int SV = kHalfVecs;         // vectors per thread and segment
  constexpr int E = kTT * SV * N;       // elements per 32 KiB segment, as the verification's
  static_assert(kTT == kThreads, "the verification's segments");
  __shared__ float red[kTT / 64];
  const int tid = threadIdx.x;
  const int b = int(blockIdx.x / uint32_t(a.max_k)), k = int(blockIdx.x % uint32_t(a.max_k));
  const int K = min(max(a.num_draft[b], 0), a.max_k);
  const float T = a.temperature[b];
  const int64_t ts = a.target_start[b];
  if (T > 0.f || k >= K) return;
  const float c = kLog2e;
  const ET* rt = static_cast<const ET*>(a.target) + (ts + k) * a.target_stride;
  const bool al = is_aligned16(rt);
  Partial* p = a.stats + (size_t(b) * a.R + a.max_k + k) * a.nseg2;
  for (int s = 0; s < a.nseg2; ++s) {
    const float m = p[s].m;
    uint4 v[SV];
#pragma unroll
    for (int q = 0; q < SV; ++q) v[q] = load_raw<ET>(rt, s * E + (q * kTT + tid) * N, a.V, al);
    float sum = 0.f;
    if (m != -INFINITY) {
      const float mc = m * c;
#pragma unroll
      for (int q = 0; q < SV; ++q)
#pragma unroll
        for (int j = 0; j < N; ++j) sum += fast_exp2(fmaf(Elem<ET>::get(v[q], j), c, -mc));
    }
    const float total = block_total(sum, red, tid);
    if (tid == 0) p[s].s = total;
  }
}

template <typename ET, bool PREV>
void launch_tts_kind(const TtsArgs& a, unsigned grid, hipStream_t stream) {
  if (a.stats && !PREV) {
    hipLaunchKernelGGL(tts_seg_kernel<ET>, dim3(grid * unsigned(a.nseg2)), dim3(kTT), 0, stream, a);
  } else if (a.stats) {
    hipLaunchKernelGGL((tts_grad_kernel<ET, PREV, true>), dim3(grid), dim3(kTT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((tts_grad_kernel<ET, PREV, false>), dim3(grid), dim3(kTT), 0, stream, a);
  }
}

}  // namespace

hipError_t launch_tts_grad(int B, int V, int max_k, int dtype, const void* draft, const int64_t* draft_start,
                           int64_t draft_stride, const void* target, const int64_t* target_start,
                           int64_t target_stride, const void* prev, const int64_t* prev_start, int64_t prev_stride,
                           const int32_t* num_draft, const float* temperature, const float* weights, float lambda,
                           void* grad, float* loss, Partial* stats, float* loss_parts, uint32_t* tickets,
                           int R, int nseg2, hipStream_t stream) {
  const TtsArgs a{B,       V,       max_k,     draft,        draft_start, draft_stride, target,
                  target_start, target_stride, prev,   prev_start,  prev_stride,  num_draft, temperature,
                  weights, lambda,  grad,      loss,         stats,       loss_parts,   tickets,  R,
                  nseg2};
  const unsigned grid = unsigned(uint64_t(B) * uint64_t(max_k));
  if (stats) {
    if (dtype == SV_BF16)
      hipLaunchKernelGGL(greedy_target_sums_kernel<uint16_t>, dim3(grid), dim3(kTT), 0, stream, a);
    else
      hipLaunchKernelGGL(greedy_target_sums_kernel<float>, dim3(grid), dim3(kTT), 0, stream, a);
  }
  if (dtype == SV_BF16) {
    if (prev)
      launch_tts_kind<uint16_t, true>(a, grid, stream);
    else
      launch_tts_kind<uint16_t, false>(a, grid, stream);
  } else {
    if (prev)
      launch_tts_kind<float, true>(a, grid, stream);
    else
      launch_tts_kind<float, false>(a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace sv
