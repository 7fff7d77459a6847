// C entry points of libspecverify.so: host-side argument checks, workspace
// layout and kernel launches on the caller's stream.  No call allocates,
// frees or synchronises the host.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "sv_internal.hpp"

using namespace sv;

namespace {

// The kernels number a call's workgroups (row segments) in 32 bits, and a
// 1-D grid holds at most 2^32 - 1 threads.
constexpr uint64_t kMaxItems = uint64_t(1) << 31;
constexpr uint64_t kMaxGrid = (uint64_t(1) << 32) / kThreads - 1;

bool dtype_ok(int dtype) { return dtype == SV_F32 || dtype == SV_BF16; }

int check_sizes(int B, int V, int max_k, int dtype) {
  if (B < 0 || V < 1 || max_k < 0 || !dtype_ok(dtype)) return SV_ERR_INVALID_ARG;
  if (max_k > SV_MAX_K || V > SV_MAX_V || B > SV_MAX_B) return SV_ERR_UNSUPPORTED;
  // a bound on the largest grid: the streaming kernels' statistics, weight and
  // search workgroups (32 KiB segments)
  const uint64_t n2 = uint64_t(num_sample_segments(V, dtype));
  const uint64_t items = uint64_t(B) * (uint64_t(rows_per_request(max_k)) * n2 + n2 + 1);
  if (items > kMaxItems || items > kMaxGrid) return SV_ERR_UNSUPPORTED;
  return SV_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? SV_OK : SV_ERR_HIP; }

// Kernel arguments of a verification call (the estimator outputs unset).
VerifyArgs verify_args(const WsLayout& L, void* workspace, int B, int V, int max_k, const void* draft_logits,
                       const int64_t* draft_row_start, int64_t draft_row_stride, const void* target_logits,
                       const int64_t* target_row_start, int64_t target_row_stride, const int32_t* num_draft,
                       const int32_t* draft_tokens, const float* temperature, const float* u_accept,
                       const float* u_residual, const float* u_bonus, int32_t* accept_len, int32_t* out_tokens,
                       int8_t* labels, float* p_draft_at_token, float* p_target_at_token) {
  char* ws = static_cast<char*>(workspace);
  VerifyArgs a;
  a.B = B;
  a.V = V;
  a.max_k = max_k;
  a.nseg2 = L.nseg2;
  a.R = L.R;
  a.draft = draft_logits;
  a.draft_start = draft_row_start;
  a.draft_stride = draft_row_stride;
  a.target = target_logits;
  a.target_start = target_row_start;
  a.target_stride = target_row_stride;
  a.num_draft = num_draft;
  a.tokens = draft_tokens;
  a.temperature = temperature;
  a.u_accept = u_accept;
  a.u_residual = u_residual;
  a.u_bonus = u_bonus;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.labels = labels;
  a.p_draft = p_draft_at_token;
  a.p_target = p_target_at_token;
  a.av_params = nullptr;
  a.av_feature = nullptr;
  a.av_score = nullptr;
  a.ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  a.partials = reinterpret_cast<Partial*>(ws + L.partials);
  a.zval = reinterpret_cast<float*>(ws + L.zval);
  a.tagged = reinterpret_cast<uint64_t*>(ws + L.tagged);
  a.spin_limit = 0;
  return a;
}

// Host checks of a verification call's arguments (the workspace aside).
int verify_arg_status(int B, int V, int max_k, int dtype, const void* draft_logits, const int64_t* draft_row_start,
                      int64_t draft_row_stride, const void* target_logits, const int64_t* target_row_start,
                      int64_t target_row_stride, const int32_t* num_draft, const int32_t* draft_tokens,
                      const float* temperature, const float* u_accept, const float* u_residual,
                      const float* u_bonus, const int32_t* accept_len, const int32_t* out_tokens,
                      const float* av_params, const float* av_feature, const float* av_score) {
  const int st = check_sizes(B, V, max_k, dtype);
  if (st != SV_OK || B == 0) return st;
  if (!target_logits || !target_row_start || !num_draft || !temperature || !u_residual || !u_bonus ||
      !accept_len || !out_tokens)
    return SV_ERR_INVALID_ARG;
  if (max_k > 0 && (!draft_logits || !draft_row_start || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
  if (target_row_stride < V || (max_k > 0 && draft_row_stride < V)) return SV_ERR_INVALID_ARG;
  if (av_score && (!av_feature || !av_params)) return SV_ERR_INVALID_ARG;
  return SV_OK;
}

// The bytes of a workspace laid out by L that a verification call uses (the
// distillation gradient's region after them is left alone).
size_t verify_scratch_end(const WsLayout& L) { return L.tts_loss; }

// Launch the verification on a checked workspace or scratch of layout L.
int verify_on(void* stream, const WsLayout& L, int dtype, void* workspace, int B, int V, int max_k,
              const void* draft_logits, const int64_t* draft_row_start, int64_t draft_row_stride,
              const void* target_logits, const int64_t* target_row_start, int64_t target_row_stride,
              const int32_t* num_draft, const int32_t* draft_tokens, const float* temperature,
              const float* u_accept, const float* u_residual, const float* u_bonus, int32_t* accept_len,
              int32_t* out_tokens, int8_t* labels, float* p_draft_at_token, float* p_target_at_token,
              const float* av_params, float* av_feature, float* av_score) {
  VerifyArgs a = verify_args(L, workspace, B, V, max_k, draft_logits, draft_row_start, draft_row_stride,
                             target_logits, target_row_start, target_row_stride, num_draft, draft_tokens,
                             temperature, u_accept, u_residual, u_bonus, accept_len, out_tokens, labels,
                             p_draft_at_token, p_target_at_token);
  a.av_params = av_params;
  a.av_feature = av_feature;
  a.av_score = av_score;
  return to_status(launch_streaming(a, dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t sv_workspace_size(int B, int V, int max_k, int dtype) {
  if (check_sizes(B, V, max_k, dtype) != SV_OK) return 0;
  return ws_layout(B, V, max_k, dtype).total;
}

int sv_spec_verify(void* stream, int B, int V, int max_k, int dtype, const void* draft_logits,
                   const int64_t* draft_row_start, int64_t draft_row_stride, const void* target_logits,
                   const int64_t* target_row_start, int64_t target_row_stride, const int32_t* num_draft,
                   const int32_t* draft_tokens, const float* temperature, const float* u_accept,
                   const float* u_residual, const float* u_bonus, int32_t* accept_len, int32_t* out_tokens,
                   int8_t* labels, float* p_draft_at_token, float* p_target_at_token, const float* av_params,
                   float* av_feature, float* av_score, void* workspace, size_t workspace_bytes) {
  const int st = verify_arg_status(B, V, max_k, dtype, draft_logits, draft_row_start, draft_row_stride,
                                   target_logits, target_row_start, target_row_stride, num_draft, draft_tokens,
                                   temperature, u_accept, u_residual, u_bonus, accept_len, out_tokens, av_params,
                                   av_feature, av_score);
  if (st != SV_OK || B == 0) return st;
  const WsLayout L = ws_layout(B, V, max_k, dtype);
  if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;
  return verify_on(stream, L, dtype, workspace, B, V, max_k, draft_logits, draft_row_start, draft_row_stride,
                   target_logits, target_row_start, target_row_stride, num_draft, draft_tokens, temperature,
                   u_accept, u_residual, u_bonus, accept_len, out_tokens, labels, p_draft_at_token,
                   p_target_at_token, av_params, av_feature, av_score);
}

int sv_spec_verify_static(void* stream, int B, int V, int max_k, int dtype, const void* draft_logits,
                          const int64_t* draft_row_start, int64_t draft_row_stride, const void* target_logits,
                          const int64_t* target_row_start, int64_t target_row_stride, const int32_t* num_draft,
                          const int32_t* draft_tokens, const float* temperature, const float* u_accept,
                          const float* u_residual, const float* u_bonus, int32_t* accept_len, int32_t* out_tokens,
                          int8_t* labels, float* p_draft_at_token, float* p_target_at_token,
                          const float* av_params, float* av_feature, float* av_score) {
  const int st = verify_arg_status(B, V, max_k, dtype, draft_logits, draft_row_start, draft_row_stride,
                                   target_logits, target_row_start, target_row_stride, num_draft, draft_tokens,
                                   temperature, u_accept, u_residual, u_bonus, accept_len, out_tokens, av_params,
                                   av_feature, av_score);
  if (st != SV_OK || B == 0) return st;
  const WsLayout L = ws_layout(B, V, max_k, dtype);
  if (verify_scratch_end(L) > size_t(SV_STATIC_SCRATCH_BYTES)) return SV_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (static_scratch(static_cast<hipStream_t>(stream), &scratch) != hipSuccess) return SV_ERR_HIP;
  return verify_on(stream, L, dtype, scratch, B, V, max_k, draft_logits, draft_row_start, draft_row_stride,
                   target_logits, target_row_start, target_row_stride, num_draft, draft_tokens, temperature,
                   u_accept, u_residual, u_bonus, accept_len, out_tokens, labels, p_draft_at_token,
                   p_target_at_token, av_params, av_feature, av_score);
}

size_t sv_filtered_workspace_size(int B, int V, int max_k, int dtype) {
  if (check_sizes(B, V, max_k, dtype) != SV_OK) return 0;
  return filter_layout(B, V, max_k, dtype).total;
}

int sv_spec_verify_filtered(void* stream, int B, int V, int max_k, int dtype, const void* draft_logits,
                            const int64_t* draft_row_start, int64_t draft_row_stride, const void* target_logits,
                            const int64_t* target_row_start, int64_t target_row_stride, const int32_t* num_draft,
                            const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                            const float* top_p, const float* u_accept, const float* u_residual,
                            const float* u_bonus, int32_t* accept_len, int32_t* out_tokens, int8_t* labels,
                            float* p_draft_at_token, float* p_target_at_token, int32_t* kept, void* workspace,
                            size_t workspace_bytes) {
  const int st = check_sizes(B, V, max_k, dtype);
  if (st != SV_OK) return st;
  if (B == 0) return SV_OK;
  if (!target_logits || !target_row_start || !num_draft || !temperature || !top_k || !top_p || !u_residual ||
      !u_bonus || !accept_len || !out_tokens)
    return SV_ERR_INVALID_ARG;
  if (max_k > 0 && (!draft_logits || !draft_row_start || !draft_tokens || !u_accept)) return SV_ERR_INVALID_ARG;
  if (target_row_stride < V || (max_k > 0 && draft_row_stride < V)) return SV_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(B, V, max_k, dtype);
  const FilterLayout F = filter_layout(B, V, max_k, dtype);
  if (!workspace || workspace_bytes < F.total) return SV_ERR_WORKSPACE;
  VerifyArgs a = verify_args(L, workspace, B, V, max_k, draft_logits, draft_row_start, draft_row_stride,
                             target_logits, target_row_start, target_row_stride, num_draft, draft_tokens,
                             temperature, u_accept, u_residual, u_bonus, accept_len, out_tokens, labels,
                             p_draft_at_token, p_target_at_token);
  char* ws = static_cast<char*>(workspace);
  const FilterIO io{top_k,
                    top_p,
                    kept,
                    reinterpret_cast<uint64_t*>(ws + F.hmass),
                    reinterpret_cast<uint32_t*>(ws + F.hcount),
                    ws + F.search,
                    ws + F.info,
                    ws + F.desc,
                    reinterpret_cast<float*>(ws + F.slices),
                    reinterpret_cast<uint32_t*>(ws + F.tickets),
                    reinterpret_cast<uint32_t*>(ws + F.work),
                    reinterpret_cast<uint32_t*>(ws + F.wcount)};
  return to_status(launch_filtered(a, io, dtype, static_cast<hipStream_t>(stream)));
}

int sv_av_score(void* stream, int B, int V, int max_k, int dtype, const void* draft_logits,
                const int64_t* draft_row_start, int64_t draft_row_stride, const int32_t* num_draft,
                const float* temperature, const float* params, float prune_threshold, float* feature,
                float* score, int32_t* num_kept, void* workspace, size_t workspace_bytes) {
  const int st = check_sizes(B, V, max_k, dtype);
  if (st != SV_OK) return st;
  if (B == 0) return SV_OK;
  if (!num_draft || !temperature) return SV_ERR_INVALID_ARG;
  if (max_k == 0) {
    if (!num_kept) return SV_OK;
  } else if (!draft_logits || !draft_row_start || !params || !feature || !score || draft_row_stride < V) {
    return SV_ERR_INVALID_ARG;
  }
  const WsLayout L = ws_layout(B, V, max_k, dtype);
  if (!workspace || workspace_bytes < L.total) return SV_ERR_WORKSPACE;

  // the statistics kernel's layout: draft row i of request b in row slot i
  VerifyArgs a = verify_args(L, workspace, B, V, max_k, draft_logits, draft_row_start, draft_row_stride, nullptr,
                             nullptr, V, num_draft, nullptr, temperature, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, nullptr, nullptr);
  a.av_params = params;
  a.av_feature = feature;
  a.av_score = score;
  return to_status(launch_score(a, prune_threshold, num_kept, dtype, static_cast<hipStream_t>(stream)));
}

int sv_av_fit_step(void* stream, int B, int max_k, const float* feature, const int8_t* labels, float* params,
                   double* accum, float damping_c, float ridge, float max_step, int do_update) {
  if (B < 0 || max_k < 0) return SV_ERR_INVALID_ARG;
  if (max_k > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if (!(damping_c >= 0.f) || !(ridge >= 0.f) || !(max_step > 0.f)) return SV_ERR_INVALID_ARG;
  if (max_k == 0) return SV_OK;
  if (!params || !accum || (B > 0 && (!feature || !labels))) return SV_ERR_INVALID_ARG;
  return to_status(launch_av_fit(B, max_k, feature, labels, params, accum, damping_c, ridge, max_step, do_update,
                                 static_cast<hipStream_t>(stream)));
}

int sv_av_budget(void* stream, int B, int max_k, const float* score, const int32_t* num_draft,
                 const float* draft_cost_ms, const float* verify_cost_ms, int32_t* num_kept, int32_t* budget) {
  if (B < 0 || max_k < 0) return SV_ERR_INVALID_ARG;
  if (max_k > SV_MAX_K || int64_t(B) * max_k > SV_BUDGET_MAX_ITEMS) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!num_draft || !draft_cost_ms || !verify_cost_ms || !num_kept || !budget || (max_k > 0 && !score))
    return SV_ERR_INVALID_ARG;
  return to_status(launch_av_budget(B, max_k, score, num_draft, draft_cost_ms, verify_cost_ms, num_kept, budget,
                                    static_cast<hipStream_t>(stream)));
}

int sv_av_calib_accumulate(void* stream, int B, int max_k, const float* score, const int8_t* labels,
                           double* accum) {
  if (B < 0 || max_k < 0) return SV_ERR_INVALID_ARG;
  if (max_k > SV_MAX_K || B > SV_MAX_B) return SV_ERR_UNSUPPORTED;
  if (!accum) return SV_ERR_INVALID_ARG;
  if (B == 0 || max_k == 0) return SV_OK;
  if (!score || !labels) return SV_ERR_INVALID_ARG;
  return to_status(launch_calib_accumulate(B * max_k, score, labels, accum, static_cast<hipStream_t>(stream)));
}

int sv_av_calib_metrics(void* stream, double* accum, double* metrics, int reset) {
  if (!accum || !metrics) return SV_ERR_INVALID_ARG;
  return to_status(launch_calib_metrics(accum, metrics, reset ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int sv_tts_grad(void* stream, int B, int V, int max_k, int dtype, const void* draft_logits,
                const int64_t* draft_row_start, int64_t draft_row_stride, const void* target_logits,
                const int64_t* target_row_start, int64_t target_row_stride, const void* prev_logits,
                const int64_t* prev_row_start, int64_t prev_row_stride, const int32_t* num_draft,
                const float* temperature, const float* weights, float lambda, void* grad, float* loss,
                void* verify_workspace, size_t workspace_bytes) {
  if (B < 0 || V < 1 || max_k < 0 || !dtype_ok(dtype) || !(lambda >= 0.f)) return SV_ERR_INVALID_ARG;
  if (max_k > SV_MAX_K || V > SV_MAX_V || B > SV_MAX_B) return SV_ERR_UNSUPPORTED;
  if (B == 0 || max_k == 0) return SV_OK;
  if (!draft_logits || !draft_row_start || !target_logits || !target_row_start || !num_draft || !temperature ||
      !weights || !grad || !loss)
    return SV_ERR_INVALID_ARG;
  if (draft_row_stride < V || target_row_stride < V) return SV_ERR_INVALID_ARG;
  if (prev_logits && (!prev_row_start || prev_row_stride < V)) return SV_ERR_INVALID_ARG;
  Partial* stats = nullptr;
  float* loss_parts = nullptr;
  uint32_t* tickets = nullptr;
  int R = 0, nseg2 = 0;
  if (verify_workspace) {
    if (check_sizes(B, V, max_k, dtype) != SV_OK) return SV_ERR_UNSUPPORTED;
    const WsLayout L = ws_layout(B, V, max_k, dtype);
    if (workspace_bytes < L.total) return SV_ERR_WORKSPACE;
    stats = reinterpret_cast<Partial*>(static_cast<char*>(verify_workspace) + L.partials);
    loss_parts = reinterpret_cast<float*>(static_cast<char*>(verify_workspace) + L.tts_loss);
    tickets = reinterpret_cast<uint32_t*>(static_cast<char*>(verify_workspace) + L.tickets);
    R = L.R;
    nseg2 = L.nseg2;
  }
  return to_status(launch_tts_grad(B, V, max_k, dtype, draft_logits, draft_row_start, draft_row_stride,
                                   target_logits, target_row_start, target_row_stride, prev_logits, prev_row_start,
                                   prev_row_stride, num_draft, temperature, weights, lambda, grad, loss, stats,
                                   loss_parts, tickets, R, nseg2, static_cast<hipStream_t>(stream)));
}

int sv_workspace_status(void* stream, void* workspace, size_t workspace_bytes, int32_t* status, int clear) {
  if (!status) return SV_ERR_INVALID_ARG;
  if (!workspace) {  // the static scratch of sv_spec_verify_static on the current device
    if (static_scratch(static_cast<hipStream_t>(stream), &workspace) != hipSuccess) return SV_ERR_HIP;
    workspace_bytes = SV_STATIC_SCRATCH_BYTES;
  }
  if (workspace_bytes < kCtrlBytes) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return to_status(launch_status(reinterpret_cast<uint32_t*>(ws + ws_layout(0, 1, 0, SV_F32).ctrl), status,
                                 clear ? 1 : 0, static_cast<hipStream_t>(stream)));
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported size";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
