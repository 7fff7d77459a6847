// Batched draft-token verification for gfx950.
//
// Method: [CS] "Speculative Decoding: Draft, EAGLE, MTP", sections "One
// speculative step" and "Algorithm loop in code" (accept with
// min(1, pt/pd), first rejection -> normalised residual (pt - pd)+, all
// accepted -> bonus token from the last target row).
//
// One launch of persistent workgroups that claim work items from a device
// counter.  Two kinds of item:
//
//   statistics item (b, r, s): segment s (64 KiB) of row r of request b -
//     draft rows 0..K_b-1, target rows 0..K_b - reduced to a (max, sum-exp)
//     or (max, argmax) partial.  The item completing request b (arrival
//     counter) combines the partials into row statistics, evaluates the
//     accept tests, finds the first rejection, writes the request's outputs
//     and a record of how its last token is drawn.
//   sampling item (b, s): the weight (residual or bonus probabilities) of
//     sampling segment s (32 KiB) of the row(s) the draw needs.  The item completing request b
//     locates the segment where the running weight crosses u * total and
//     searches it for the token.
//
// Requests are split into 16 partitions (b mod 16), each an independent
// schedule with its own claim counter on its own cache line: same-address
// device atomics serialise (~12 ns each), so one counter for every item would
// cap the item rate.  Within a partition, items are claimed in this order:
// the statistics items of request group 0, of group 1, the sampling items of
// group 0, statistics of group 2, sampling of group 1, ...  A sampling item
// waits (bounded) until its request has been decided.  Every item it waits
// for has a smaller claim number in the same partition, and every claimed
// item belongs to a running workgroup that is either processing it or an
// earlier item of the same partition (a workgroup claims one item ahead, and
// only within its current partition), so the smallest unfinished item of a
// partition can always proceed: no deadlock.  Because the workgroups persist, a long item never
// stalls the hardware dispatch of others, and the draw of each request is
// spread over many workgroups.  No host synchronisation; all counters are
// reset by the kernel itself.
#include "sv_device.hpp"

namespace sv {

constexpr int kSleep = 2;  // s_sleep argument inside bounded waits

__device__ __forceinline__ uint32_t claim(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// statistics item
// ---------------------------------------------------------------------------

template <typename ET>
struct Shared {
  Partial part[kWaves];
  Partial rows[2 * SV_MAX_K + 1];
  float chunk_sum[kMaxChunks];
  float g[kWaves];
  int gi[2 * kWaves];
  int lds_i[4];
  int flag;
  int a;
  uint32_t next;
};

template <typename ET>
__device__ __forceinline__ void finish_request(const VerifyArgs& a, Shared<ET>& sh, int b, int K, int nd, bool greedy,
                                               bool want_feat, float c) {
  const int tid = threadIdx.x;
  const int max_k = a.max_k;
  if (tid < a.R) {
    const bool d2 = tid < max_k;
    const int i2 = d2 ? tid : tid - max_k;
    if (d2 ? (i2 < nd) : (i2 <= K))
      sh.rows[tid] = combine_published(&a.partials[(size_t(b) * a.R + tid) * a.nseg2], a.nseg, c, !d2 && greedy);
  }
  __syncthreads();

  if (tid < 64) {
    const int lane = tid;
    bool acc = true;
    float pd = NAN, pt = NAN;
    int d = -1;
    if (lane < K) {
      d = a.tokens[size_t(b) * max_k + lane];
      if (greedy) {
        acc = (d == sh.rows[max_k + lane].idx);
        pt = acc ? 1.f : 0.f;
      } else {
        const Partial D = sh.rows[lane], Tg = sh.rows[max_k + lane];
        const float zd = load_dev(&a.zval[size_t(b) * a.R + lane]);
        const float zt = load_dev(&a.zval[size_t(b) * a.R + max_k + lane]);
        const float l2d = (zd - D.m) * c - fast_log2(D.s + D.cnt);
        const float l2t = (zt - Tg.m) * c - fast_log2(Tg.s + Tg.cnt);
        pd = fast_exp2(l2d);
        pt = fast_exp2(l2t);
        acc = (l2d == -INFINITY) || (a.u_accept[size_t(b) * max_k + lane] < fast_exp2(l2t - l2d));
      }
    }
    const unsigned long long rej = __ballot(lane < K && !acc);
    const int aa = rej ? (__ffsll(static_cast<long long>(rej)) - 1) : K;
    if (lane < max_k) {
      const size_t o = size_t(b) * max_k + lane;
      if (a.labels) a.labels[o] = (lane < aa) ? 1 : ((lane == aa && aa < K) ? 0 : -1);
      if (a.p_draft) a.p_draft[o] = pd;
      if (a.p_target) a.p_target[o] = pt;
      if (want_feat) {
        float x = NAN, sc = NAN;
        if (lane < K && sh.rows[lane].s >= kRecomputeBelow) {
          x = feature_from_other(sh.rows[lane].s - 1.f);
          if (a.av_params) sc = sigmoid_score(a.av_params, lane, x);
        }
        a.av_feature[o] = x;  // rows with s < kRecomputeBelow are written below
        if (a.av_score) a.av_score[o] = sc;
      }
    }
    if (lane <= max_k && lane != aa) a.out_tokens[size_t(b) * (max_k + 1) + lane] = (lane < aa) ? d : -1;
    if (lane == 0) {
      sh.a = aa;
      a.accept_len[b] = aa;
    }
  }
  __syncthreads();

  // confident draft rows: the feature needs the exact sum of the other tokens
  if (want_feat) {
    for (int i = 0; i < K; ++i) {
      if (!(sh.rows[i].s < kRecomputeBelow)) continue;
      const ET* row = static_cast<const ET*>(a.draft) + (a.draft_start[b] + i) * a.draft_stride;
      const float so = exact_other_sum<ET>(row, &a.partials[(size_t(b) * a.R + i) * a.nseg2], a.nseg, a.V,
                                           sh.rows[i].m, c, sh.part);
      if (tid == 0) {
        const float x = feature_from_other(so);
        a.av_feature[size_t(b) * max_k + i] = x;
        if (a.av_score) a.av_score[size_t(b) * max_k + i] = sigmoid_score(a.av_params, i, x);
      }
      __syncthreads();
    }
  }

  if (tid == 0) {
    const int aa = sh.a;
    int mode;
    if (greedy) {
      a.out_tokens[size_t(b) * (max_k + 1) + aa] = sh.rows[max_k + aa].idx;
      mode = kNoDraw;
    } else {
      Record* rec = &a.records[b];
      const Partial Tg = sh.rows[max_k + aa];
      store_dev(&rec->a, aa);
      store_dev(&rec->kt, Tg.m * c + fast_log2(Tg.s + Tg.cnt));
      store_dev(&rec->c, c);
      if (aa < K) {
        const Partial D = sh.rows[aa];
        store_dev(&rec->kd, D.m * c + fast_log2(D.s + D.cnt));
        store_dev(&rec->u, a.u_residual[b]);
        mode = kResidual;
      } else {
        store_dev(&rec->kd, 0.f);
        store_dev(&rec->u, a.u_bonus[b]);
        mode = kBonus;
      }
      store_dev(&rec->mode, mode);
    }
    // publish the decision after the record is complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    store_dev(&a.flags[req_slot(b)], mode);
    store_dev(&a.tickets[req_slot(b)], 0u);
  }
}

template <typename ET>
__device__ __forceinline__ void stats_item(const VerifyArgs& a, Shared<ET>& sh, int b, int r, int s) {
  constexpr int SEG = kSegBytes / int(sizeof(ET));
  const int tid = threadIdx.x;
  const int max_k = a.max_k;
  const int K = min(max(a.num_draft[b], 0), max_k);
  const float T = a.temperature[b];
  const bool greedy = !(T > 0.f);
  const bool want_feat = a.av_feature != nullptr;
  const bool is_draft = r < max_k;
  const int i = is_draft ? r : r - max_k;
  const int nd = (!greedy || want_feat) ? K : 0;  // draft rows read
  if (is_draft ? (i >= nd) : (i > K)) return;
  const uint32_t want = uint32_t(a.nseg) * uint32_t(nd + K + 1);
  const float c = kLog2e / (greedy ? 1.f : T);

  const ET* row = is_draft ? static_cast<const ET*>(a.draft) + (a.draft_start[b] + i) * a.draft_stride
                           : static_cast<const ET*>(a.target) + (a.target_start[b] + i) * a.target_stride;
  const bool aligned = is_aligned16(row);
  const int base = s * SEG;

  Partial p;
  if (is_draft) {
    p = segment_stats<ET, kSumInclusive>(row, base, a.V, aligned, c, sh.part);
  } else if (greedy) {
    p = segment_stats<ET, kArgmax>(row, base, a.V, aligned, c, sh.part);
  } else {
    p = segment_stats<ET, kSumInclusive>(row, base, a.V, aligned, c, sh.part);
  }

  if (tid == 0) {
    publish(&a.partials[(size_t(b) * a.R + r) * a.nseg2 + s], p);
    // logit at the draft token, from the segment that holds it
    if (!greedy && i < K) {
      const int d = a.tokens[size_t(b) * max_k + i];
      if (d >= base && d < base + SEG && d < a.V) store_dev(&a.zval[size_t(b) * a.R + r], Elem<ET>::one(row + d));
    }
  }
  if (arrive_last(&a.tickets[req_slot(b)], want, &sh.flag)) finish_request<ET>(a, sh, b, K, nd, greedy, want_feat, c);
}

// ---------------------------------------------------------------------------
// sampling item
// ---------------------------------------------------------------------------

template <typename ET>
__device__ __forceinline__ void sample_item(const VerifyArgs& a, Shared<ET>& sh, int b, int s) {
  const int tid = threadIdx.x;
  // wait until request b has been decided
  if (tid == 0) {
    int mode = load_dev(&a.flags[req_slot(b)]);
    for (uint32_t n = 0; mode == kUnresolved && n < a.spin_limit; ++n) {
      __builtin_amdgcn_s_sleep(kSleep);
      mode = load_dev(&a.flags[req_slot(b)]);
    }
    if (mode == kUnresolved) store_dev(&a.ctrl[kCtrlError], 1u);
    sh.flag = mode;
  }
  __syncthreads();
  const int mode = sh.flag;
  __syncthreads();
  if (mode == kUnresolved) return;  // wait expired (never expected): leave the token unwritten

  Record rec;
  const ET* rt = nullptr;
  const ET* rd = nullptr;
  bool fast = false;
  if (mode != kNoDraw) {
    const Record* src = &a.records[b];
    rec.a = load_dev(&src->a);
    rec.kt = load_dev(&src->kt);
    rec.kd = load_dev(&src->kd);
    rec.c = load_dev(&src->c);
    rec.u = load_dev(&src->u);
    rt = static_cast<const ET*>(a.target) + (a.target_start[b] + rec.a) * a.target_stride;
    if (mode == kResidual) rd = static_cast<const ET*>(a.draft) + (a.draft_start[b] + rec.a) * a.draft_stride;
    fast = is_aligned16(rt) && (mode != kResidual || is_aligned16(rd));
    const float W = (mode == kResidual)
                        ? segment_weight<ET, true>(rt, rd, fast, s, a.V, rec.c, rec.kt, rec.c, rec.kd, sh.g)
                        : segment_weight<ET, false>(rt, rt, fast, s, a.V, rec.c, rec.kt, rec.c, rec.kt, sh.g);
    if (tid == 0) store_dev(&a.segsum[size_t(b) * a.nseg2 + s], W);
  }
  if (!arrive_last(&a.tickets2[req_slot(b)], uint32_t(a.nseg2), &sh.flag)) return;

  // ---- the last sampling item of request b draws the token ----
  if (mode != kNoDraw) {
    if (tid == 0) {
      float Z = 0.f;
      for (int k = 0; k < a.nseg2; ++k) Z += load_dev(&a.segsum[size_t(b) * a.nseg2 + k]);
      int k = -1, fb = 0;
      float before = 0.f, t = 0.f;
      if (Z > 0.f) {
        t = rec.u * Z;
        float cum = 0.f;
        for (int j = 0; j < a.nseg2; ++j) {
          const float w = load_dev(&a.segsum[size_t(b) * a.nseg2 + j]);
          if (cum + w > t) {
            k = j;
            before = cum;
            break;
          }
          cum += w;
        }
        if (k < 0) {  // rounding: the last segment with positive weight
          fb = 1;
          for (int j = a.nseg2 - 1; j >= 0; --j)
            if (load_dev(&a.segsum[size_t(b) * a.nseg2 + j]) > 0.f) {
              k = j;
              break;
            }
        }
      }
      sh.lds_i[0] = k;
      sh.lds_i[1] = fb;
      reinterpret_cast<float*>(sh.lds_i)[2] = before;
      reinterpret_cast<float*>(sh.lds_i)[3] = t;
    }
    __syncthreads();
    const int k = sh.lds_i[0];
    const bool fb = sh.lds_i[1] != 0;
    const float before = reinterpret_cast<const float*>(sh.lds_i)[2];
    const float t = reinterpret_cast<const float*>(sh.lds_i)[3];
    __syncthreads();
    int tok;
    if (k >= 0) {
      tok = (mode == kResidual)
                ? segment_search<ET, true>(rt, rd, fast, k, a.V, rec.c, rec.kt, rec.c, rec.kd, before, t, fb, sh.g, sh.gi)
                : segment_search<ET, false>(rt, rt, fast, k, a.V, rec.c, rec.kt, rec.c, rec.kt, before, t, fb, sh.g,
                                            sh.gi);
    } else {
      // the residual has no mass (reachable only through rounding): draw from pt itself
      tok = cdf_sample<ET, false>(rt, rec.c, rec.kt, rt, rec.c, rec.kt, a.V, rec.u, sh.chunk_sum, sh.lds_i);
    }
    if (tid == 0) a.out_tokens[size_t(b) * (a.max_k + 1) + rec.a] = tok;
  }
  if (tid == 0) {
    store_dev(&a.flags[req_slot(b)], 0);
    store_dev(&a.tickets2[req_slot(b)], 0u);
  }
}

// ---------------------------------------------------------------------------
// persistent kernel
// ---------------------------------------------------------------------------

// Schedule of one partition: partition p owns requests b = p + j * parts
// (j = 0 .. nreq-1), taken in groups of `group` requests.  Claim numbers run
// over: statistics items of group 0, of group 1, sampling items of group 0,
// statistics of group 2, sampling of group 1, ..., sampling of the last group.
struct Schedule {
  uint32_t A;      // statistics items per group
  uint32_t C;      // sampling items per group
  uint32_t ngroups;
  uint32_t total;  // claim numbers of the partition
  int nreq;
};

__device__ __forceinline__ Schedule schedule(const VerifyArgs& a, int p) {
  Schedule S;
  S.nreq = (a.B - p + a.parts - 1) / a.parts;
  S.A = uint32_t(a.group) * uint32_t(a.R) * uint32_t(a.nseg);
  S.C = uint32_t(a.group) * uint32_t(a.nseg2);
  S.ngroups = (uint32_t(S.nreq) + a.group - 1) / a.group;
  S.total = S.ngroups * (S.A + S.C);
  return S;
}

template <typename ET>
__device__ __forceinline__ void run_item(const VerifyArgs& a, Shared<ET>& sh, const Schedule& S, int p, uint32_t id) {
  bool stats;
  uint32_t group, local;
  if (id < S.A) {
    stats = true;
    group = 0;
    local = id;
  } else {
    const uint32_t q = id - S.A, blk = q / (S.A + S.C), off = q % (S.A + S.C);
    if (blk + 1 < S.ngroups) {
      stats = off < S.A;
      group = stats ? blk + 1 : blk;
      local = stats ? off : off - S.A;
    } else {
      stats = false;
      group = blk;
      local = off;
    }
  }
  const uint32_t per = stats ? uint32_t(a.R) * uint32_t(a.nseg) : uint32_t(a.nseg2);
  const int j = int(group * uint32_t(a.group) + local / per);  // request index within the partition
  if (j >= S.nreq) return;
  const int b = p + j * a.parts;
  const uint32_t rem = local % per;
  if (stats)
    stats_item<ET>(a, sh, b, int(rem / a.nseg), int(rem % a.nseg));
  else
    sample_item<ET>(a, sh, b, int(rem));
}

template <typename ET>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void spec_verify_kernel(VerifyArgs a) {
  __shared__ Shared<ET> sh;
  const int tid = threadIdx.x;
  // Start in partition blockIdx % parts; when it is exhausted, move through
  // the others.  The next item is claimed one ahead within a partition only,
  // so each partition keeps its own ordering argument.
  int p = int(blockIdx.x % uint32_t(a.parts));
  for (int visited = 0; visited < a.parts; ++visited, p = (p + 1) % a.parts) {
    const Schedule S = schedule(a, p);
    uint32_t* counter = &a.ctrl[kCtrlWork + p * kLineWords];
    if (tid == 0) sh.next = claim(counter);
    __syncthreads();
    uint32_t id = sh.next;
    __syncthreads();
    while (id < S.total) {
      uint32_t ahead = 0;
      if (tid == 0) ahead = claim(counter);  // result is needed only at the end of the item
      run_item<ET>(a, sh, S, p, id);
      if (tid == 0) sh.next = ahead;
      __syncthreads();
      id = sh.next;
      __syncthreads();
    }
  }
  // the last workgroup out resets the claim counters for the next launch
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(&a.ctrl[kCtrlExit], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      for (int q = 0; q < a.parts; ++q) store_dev(&a.ctrl[kCtrlWork + q * kLineWords], 0u);
      store_dev(&a.ctrl[kCtrlExit], 0u);
    }
  }
}

// Resident workgroups per CU and CU count, per device and element type.
static int g_capacity[64][2];

static int resident_grid(int dtype) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  const int slot = dtype == SV_BF16 ? 1 : 0;
  int cap = __atomic_load_n(&g_capacity[dev][slot], __ATOMIC_RELAXED);
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    const hipError_t e1 =
        dtype == SV_BF16
            ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, spec_verify_kernel<uint16_t>, kThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, spec_verify_kernel<float>, kThreads, 0);
    const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cap = (e1 == hipSuccess && e2 == hipSuccess && per_cu > 0 && cus > 0) ? per_cu * cus : 1024;
    __atomic_store_n(&g_capacity[dev][slot], cap, __ATOMIC_RELAXED);
  }
  return cap;
}

hipError_t launch_spec_verify(VerifyArgs a, int dtype, hipStream_t stream) {
  const int cap = resident_grid(dtype);
  a.parts = a.B < kParts ? a.B : kParts;
  // groups of requests: about two statistics items per resident workgroup of
  // the partition, so a group's sampling items rarely find their request
  // still undecided
  const int per_request = a.R * a.nseg;
  const int wg_per_part = (cap + a.parts - 1) / a.parts;
  const int nreq_max = (a.B + a.parts - 1) / a.parts;
  a.group = max(1, min(nreq_max, (2 * wg_per_part + per_request - 1) / per_request));
  const uint64_t ngroups = (uint64_t(nreq_max) + a.group - 1) / a.group;
  const uint64_t total = ngroups * uint64_t(a.group) * (uint64_t(a.R) * a.nseg + uint64_t(a.nseg2));
  if (total + uint64_t(cap) >= (uint64_t(1) << 32)) return hipErrorInvalidValue;
  a.spin_limit = 1u << 20;  // ~1-2 s of polling: only reached if the schedule were broken
  const uint64_t all = total * uint64_t(a.parts);
  const unsigned grid = unsigned(all < uint64_t(cap) ? all : uint64_t(cap));
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(spec_verify_kernel<uint16_t>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(spec_verify_kernel<float>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
