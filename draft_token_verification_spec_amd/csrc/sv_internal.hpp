// Internal layout shared by the host dispatch (api.cpp) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/specverify.h"

namespace sv {

// Threads per workgroup (4 wave64s).  Rows are processed in 32 KiB segments:
// kHalfVecs 16-byte vectors per thread of a workgroup, whatever the element
// type.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kHalfVecs = 8;
constexpr int kHalfBytes = kThreads * kHalfVecs * 16;
// The draw's weights are handed off per slice: one 16-byte vector of every
// thread of a 32 KiB draw segment, kDrawSlices slices per segment.
constexpr int kDrawSlices = kHalfVecs;

__host__ __device__ inline int num_sample_segments(int V, int dtype) {
  const int e = kHalfBytes / (dtype == SV_BF16 ? 2 : 4);
  return (V + e - 1) / e;
}

// Rows of one request in the grid: draft rows 0..max_k-1, then target rows
// 0..max_k (slot max_k + j).
__host__ __device__ inline int rows_per_request(int max_k) { return 2 * max_k + 1; }

// Statistics of one segment of one row.
//   m    largest logit of the segment (-inf if none is finite)
//   s    sum of exp((z - m) / T) over the segment; for rows summed
//        "exclusively" the terms with z == m are left out of s and counted
//        in cnt instead (exact 1.0 each), which keeps sum_{v != argmax}
//        accurate when it is tiny
//   cnt  number of z == m terms left out of s (0 for inclusive sums)
//   idx  lowest index with z == m (greedy rows only)
struct Partial {
  float m;
  float s;
  float cnt;
  int idx;
};

// Byte offsets inside the caller's workspace.
//
// The workspace starts with a fixed arena - a control line holding the status
// word, then a per-request-slot array of SV_MAX_B arrival counters (the
// distillation gradient's segmented kernel) - which every call leaves zeroed
// (the status word aside) and no call writes partial data into, whatever its
// shape.  After the arena comes the per-call region, laid out for the call's
// (B, V, max_k).
constexpr int kLineWords = 32;    // 128 bytes: one counter per cache line
constexpr size_t kCtrlBytes = 256;  // the control line, padded so that the arrays after it stay 256-byte aligned
constexpr int kCtrlError = 0;     // status word: set if a bounded wait ever expired
constexpr size_t kArenaBytes = kCtrlBytes + size_t(SV_MAX_B) * 4;

// Slot of request b in the per-request arrays of the arena: consecutive
// requests land 128 bytes apart (for b < SV_MAX_B / 32), so the atomics of
// different requests do not contend for one cache line.  A bijection on
// [0, SV_MAX_B).
__host__ __device__ constexpr int req_slot(int b) {
  return ((b & (SV_MAX_B / kLineWords - 1)) * kLineWords) | (b / (SV_MAX_B / kLineWords));
}
static_assert(SV_MAX_B % kLineWords == 0, "arena slots");

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Filtered verification: after the verification layout, per (row slot,
// 32 KiB segment, search) histograms of kFilterBins bins (fixed-point masses
// and counts), per (row slot, search) threshold-search states, per row slot
// an arrival counter, and the lists of segments still searching (two, used
// by turns) with their counters.
constexpr int kFilterBins = 256;    // key-digit bins
constexpr int kFilterBins0 = 512;  // level-0 bins
constexpr size_t kFilterSearchBytes = 48;
constexpr size_t kFilterRowBytes = 16;   // per row slot: normaliser, threshold, argmax
constexpr size_t kFilterDescBytes = 16;  // per request: accept length, draw kind, uniform
struct FilterLayout {
  size_t hmass, hcount, search, info, desc, slices, tickets, work, wcount, total;
};

// Hand-off slot of the draw kernel: 8 bytes written in one store, the low
// word kSlotReady, the high word the value's bits.  The reader polls until
// the low word is kSlotReady and clears the slot once it has the value.  The
// slots share the per-call region with other arrays when the call shapes
// change; kSlotReady is a signalling-NaN bit pattern that none of them
// holds (no float the kernels store and no index or count equals it), so
// data left there is never taken for a handed-off value.
constexpr uint32_t kSlotReady = 0x7fb5a5a5u;
__host__ __device__ constexpr uint64_t ready_slot(uint32_t bits) { return (uint64_t(bits) << 32) | kSlotReady; }

struct WsLayout {
  size_t ctrl;      // uint32 control line (status word)
  size_t tickets;   // uint32 [SV_MAX_B]  arrivals per request (the distillation gradient)
  size_t partials;  // Partial [B][R][nseg2]
  size_t zval;      // float [B][R]       logit at the draft token, per row
  size_t tagged;    // uint64 [B][nseg2][kDrawSlices]  hand-off slots of the draw's slice weights
  size_t tts_loss;  // float [B][max_k][nseg2]  distillation loss per canvas row segment
  size_t total;
  int nseg2;  // 32 KiB segments per row (partials are strided by this)
  int R;
};

inline WsLayout ws_layout(int B, int V, int max_k, int dtype);
inline FilterLayout filter_layout(int B, int V, int max_k, int dtype) {
  const WsLayout L = ws_layout(B, V, max_k, dtype);
  const size_t segs = size_t(B) * L.R * L.nseg2;
  FilterLayout F;
  F.hmass = L.total;
  F.hcount = F.hmass + align256(segs * 2 * kFilterBins * 8);
  F.search = F.hcount + align256(segs * 2 * kFilterBins0 * 4);
  F.info = F.search + align256(size_t(B) * L.R * 2 * kFilterSearchBytes);
  F.desc = F.info + align256(size_t(B) * L.R * kFilterRowBytes);
  F.slices = F.desc + align256(size_t(B) * kFilterDescBytes);
  F.tickets = F.slices + align256(size_t(B) * L.nseg2 * 2 * kDrawSlices * 4);
  F.work = F.tickets + align256(size_t(B) * L.R * 4);
  F.wcount = F.work + align256(2 * segs * 4);
  F.total = F.wcount + 256;
  return F;
}

inline WsLayout ws_layout(int B, int V, int max_k, int dtype) {
  WsLayout L;
  L.nseg2 = num_sample_segments(V, dtype);
  L.R = rows_per_request(max_k);
  L.ctrl = 0;
  L.tickets = kCtrlBytes;
  L.partials = kArenaBytes;
  L.zval = L.partials + align256(size_t(B) * L.R * L.nseg2 * sizeof(Partial));
  L.tagged = L.zval + align256(size_t(B) * L.R * 4);
  L.tts_loss = L.tagged + align256(size_t(B) * L.nseg2 * kDrawSlices * 8);
  L.total = L.tts_loss + align256(size_t(B) * max_k * L.nseg2 * 4);
  return L;
}

struct VerifyArgs {
  int B, V, max_k, nseg2, R;
  const void* draft;
  const int64_t* draft_start;
  int64_t draft_stride;
  const void* target;
  const int64_t* target_start;
  int64_t target_stride;
  const int32_t* num_draft;
  const int32_t* tokens;
  const float* temperature;
  const float* u_accept;
  const float* u_residual;
  const float* u_bonus;
  int32_t* accept_len;
  int32_t* out_tokens;
  int8_t* labels;
  float* p_draft;
  float* p_target;
  const float* av_params;
  float* av_feature;
  float* av_score;
  // workspace
  uint32_t* ctrl;     // status word at kCtrlError
  Partial* partials;  // [B][R][nseg2]
  float* zval;
  uint64_t* tagged;   // hand-off slots (see WsLayout::tagged)
  uint32_t spin_limit;  // polls of a bounded wait before it gives up
};


// The estimator's scoring pass: statistics of the draft rows into the
// workspace, then feature, score and kept count per request.
hipError_t launch_score(VerifyArgs a, float threshold, int32_t* num_kept, int dtype, hipStream_t stream);
// The two streaming kernels (statistics, then the verdict and the draw).
hipError_t launch_streaming(VerifyArgs a, int dtype, hipStream_t stream);
// Device address of the static scratch of the current device (looked up once
// per device, and zero-filled by a kernel on `stream` until a fill has run
// outside a graph capture).
hipError_t static_scratch(hipStream_t stream, void** out);
// Copy the workspace's status word to *status and, if `clear`, zero it.
hipError_t launch_status(uint32_t* ctrl, int32_t* status, int clear, hipStream_t stream);

// Filtered verification: the statistics kernel, the threshold searches and
// the verdict / draw kernel.
struct FilterIO {
  const int32_t* top_k;
  const float* top_p;
  int32_t* kept;
  uint64_t* hmass;
  uint32_t* hcount;
  void* search;
  void* info;
  void* desc;
  float* slices;
  uint32_t* tickets;
  uint32_t* work;
  uint32_t* wcount;
};
hipError_t launch_filtered(VerifyArgs a, const FilterIO& io, int dtype, hipStream_t stream);
hipError_t launch_av_budget(int B, int max_k, const float* score, const int32_t* num_draft, const float* draft_cost,
                            const float* verify_cost, int32_t* num_kept, int32_t* budget, hipStream_t stream);
hipError_t launch_calib_accumulate(int items, const float* score, const int8_t* labels, double* accum,
                                   hipStream_t stream);
hipError_t launch_calib_metrics(double* accum, double* metrics, int reset, hipStream_t stream);
hipError_t launch_tts_grad(int B, int V, int max_k, int dtype, const void* draft, const int64_t* draft_start,
                           int64_t draft_stride, const void* target, const int64_t* target_start,
                           int64_t target_stride, const void* prev, const int64_t* prev_start, int64_t prev_stride,
                           const int32_t* num_draft, const float* temperature, const float* weights, float lambda,
                           void* grad, float* loss, Partial* stats, float* loss_parts, uint32_t* tickets, int R, int nseg2,
                           hipStream_t stream);
hipError_t launch_av_fit(int B, int max_k, const float* feature, const int8_t* labels,
                         float* params, double* accum, float damping_c, float ridge, float max_step,
                         int do_update, hipStream_t stream);

}  // namespace sv
