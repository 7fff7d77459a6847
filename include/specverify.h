/*
 * specverify.h - C ABI of libspecverify.so: batched draft-token verification
 * and the online acceptance estimator of speculative decoding, for AMD
 * Instinct MI355X (gfx950).
 *
 * Pages this interface follows:
 *   [CS] "Speculative Decoding: Draft, EAGLE, MTP" (cheat sheet, nextadmin.net):
 *        sections "One speculative step", "Algorithm loop in code",
 *        "Functions in the lessons" (spec_step, residual).
 *   [AV] "Adaptive Verification ohne Confidence Head" (spke.com, German; Arabic
 *        mirror "التحقق التكيفي بدون رأس ثقة"): sections "Solution",
 *        "Scoring the distribution", "Fitting the coefficients".
 *
 * Letters: "draft" is the cheap model's distribution pd, "target" the
 * verifier's pt.  Both are softmax(logits / T) of a logit row.
 *
 * Conventions shared by every entry point:
 *   - Every array argument is device memory owned by the caller; the library
 *     never allocates, frees or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising the host.  Outputs are
 *     valid once the stream reaches that point.
 *   - Host-side argument checks run before anything is enqueued; a negative
 *     status means nothing was launched.  SV_ERR_HIP reports a launch error
 *     from the HIP runtime.  Conditions that only the device data can show
 *     (listed per call as "device preconditions") are not checked: checking
 *     them would cost bandwidth; violating them gives unspecified outputs
 *     (never an out-of-bounds access for token ids < 0 or >= V).
 *   - Outputs are a deterministic function of the inputs: the same inputs at
 *     the same addresses give bit-identical outputs.
 *   - Row addressing: request b's draft row i (0 <= i < K_b) starts at element
 *     (draft_row_start[b] + i) * draft_row_stride of draft_logits, and its
 *     target row j (0 <= j <= K_b) at (target_row_start[b] + j) *
 *     target_row_stride of target_logits.  This covers padded [B, max_k, V]
 *     batches, packed ragged batches, and stride-0 broadcasts (all starts 0).
 *     Rows whose start is 16-byte aligned are read with 16-byte vector loads.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest draft length per request, vocabulary, and requests per call. */
#define SV_MAX_K 16
#define SV_MAX_V (1 << 21)
#define SV_MAX_B (1 << 18)

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* null required pointer, negative size, stride < V, ... */
  SV_ERR_UNSUPPORTED = -2, /* size beyond SV_MAX_K / SV_MAX_V / SV_MAX_B / grid  */
  SV_ERR_WORKSPACE = -3,   /* workspace null or smaller than the size query       */
  SV_ERR_HIP = -4          /* the HIP runtime reported an error at launch          */
} sv_status;

/* Element type of the logit rows. */
typedef enum {
  SV_F32 = 0,  /* IEEE binary32                                      */
  SV_BF16 = 1  /* bfloat16 (upper 16 bits of binary32), stored as u16 */
} sv_dtype;

/* Bytes of workspace needed by sv_spec_verify and by sv_av_score for a batch
 * of B requests, vocabulary V, at most max_k drafts each, elements of type
 * `dtype`.  Returns 0 for arguments those calls would reject.
 *
 * The workspace starts with a fixed arena (a status word, one arrival
 * counter per request slot, SV_MAX_B slots), followed by per-row partial
 * statistics, logits at the draft tokens and the draw's hand-off slots.
 * Zero-fill the workspace once after allocation; every call leaves the
 * counters and hand-off slots cleared again, and no call writes anything
 * else into the arena, so one workspace (of the largest size needed) serves
 * any sequence of calls of any shapes on one stream without further
 * clearing, and a call captured in a HIP graph replays without any reset.
 * Calls that can run concurrently (different streams) need different
 * workspaces.  If a call is aborted part way (device fault), or
 * sv_workspace_status reports a nonzero status, zero-fill the workspace
 * again. */
size_t sv_workspace_size(int B, int V, int max_k, int dtype);

/* Batched speculative verification, one step for B requests.
 *
 * [CS] "One speculative step" / "Algorithm loop in code", per request b with
 * K_b = num_draft[b] drafts d_i = draft_tokens[b*max_k + i] and temperature
 * T = temperature[b]:
 *   1. pd_i = softmax(draft row i / T), pt_j = softmax(target row j / T)
 *      (row maximum subtracted: numerically safe).
 *   2. Walk i = 0..K_b-1: accept d_i iff u_accept[b*max_k+i] < min(1,
 *      pt_i(d_i) / pd_i(d_i)), the ratio being +inf when pd_i(d_i) = 0.
 *   3. a_b = the first rejected position (K_b if none): accept_len[b].
 *   4. If a_b < K_b: emit the token drawn from the normalised residual
 *      (pt_a - pd_a)+ (page [CS] function `residual`); if that residual has
 *      no mass (only reachable through rounding) pt_a itself is used.
 *      If a_b = K_b: emit the bonus token drawn from pt_{K_b}.
 *      "Drawn with u" means the inverse CDF in ascending token order: the
 *      first token v whose running sum of weights exceeds u times the total,
 *      with u = u_residual[b] or u_bonus[b] respectively.
 *   T = 0 (greedy): d_i is accepted iff it equals the lowest-index argmax of
 *   target row i; the emitted correction or bonus is that argmax.  Greedy
 *   requests do not read their draft rows unless av_feature is requested.
 *
 * Inputs (device):
 *   draft_logits   elements of type dtype; rows as described above.  May be
 *                  NULL when max_k == 0.
 *   draft_row_start / target_row_start   int64 [B], in rows.
 *   draft_row_stride / target_row_stride   elements between consecutive
 *                  rows, >= V.
 *   num_draft      int32 [B]   K_b.
 *   draft_tokens   int32 [B*max_k]   (entries at i >= K_b are ignored).
 *   temperature    float [B]   T_b >= 0.
 *   u_accept       float [B*max_k] in [0, 1).
 *   u_residual, u_bonus   float [B] in [0, 1).
 * Outputs (device, written for every request):
 *   accept_len     int32 [B]            a_b.
 *   out_tokens     int32 [B*(max_k+1)]  d_0..d_{a-1}, then the residual or
 *                  bonus token, then -1 up to max_k.
 *   labels         int8 [B*max_k]  nullable: 1 before the first rejection,
 *                  0 at it, -1 after it and past K_b ([AV] "Fitting the
 *                  coefficients": only drafts up to the first rejection are
 *                  labelled).
 *   p_draft_at_token, p_target_at_token   float [B*max_k]  nullable:
 *                  pd_i(d_i), pt_i(d_i); NaN past K_b.  For greedy requests
 *                  p_target is 1 if d_i is the target argmax else 0, and
 *                  p_draft is NaN.
 *   av_feature     float [B*max_k]  nullable: the estimator feature
 *                  logit(max_v pd_i(v)) (see sv_av_score), produced from the
 *                  same pass over the draft rows; NaN past K_b.
 *   av_score       float [B*max_k]  nullable, needs av_feature and av_params:
 *                  sigmoid(omega * feature + beta_i).
 *   av_params      float [max_k+1]  nullable: omega, beta_0..beta_{max_k-1}.
 * Device preconditions: 0 <= K_b <= max_k; token ids in [0, V); every row
 * read has at least one finite logit and no NaN or +inf (-inf is allowed and
 * means probability 0); u in [0, 1).
 * Returns SV_OK, or a negative sv_status without launching anything. */
int sv_spec_verify(void* stream, int B, int V, int max_k, int dtype,
                   const void* draft_logits, const int64_t* draft_row_start,
                   int64_t draft_row_stride,
                   const void* target_logits, const int64_t* target_row_start,
                   int64_t target_row_stride,
                   const int32_t* num_draft, const int32_t* draft_tokens,
                   const float* temperature, const float* u_accept,
                   const float* u_residual, const float* u_bonus,
                   int32_t* accept_len, int32_t* out_tokens, int8_t* labels,
                   float* p_draft_at_token, float* p_target_at_token,
                   const float* av_params, float* av_feature, float* av_score,
                   void* workspace, size_t workspace_bytes);

/* The verification without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.
 *
 * Arguments, outputs, device preconditions and results exactly as for
 * sv_spec_verify, with no workspace: the call uses the library's own static
 * scratch instead, SV_STATIC_SCRATCH_BYTES of device memory that each GPU the
 * library runs on holds from the first such call until the process ends (the
 * first call on a device also zero-fills it, with a kernel on `stream`).  It
 * allocates and frees nothing.  Shapes whose scratch would not fit return
 * SV_ERR_UNSUPPORTED without launching (sv_workspace_size(B, V, max_k,
 * dtype) <= SV_STATIC_SCRATCH_BYTES is sufficient; B = 256, K = 4, V = 128256
 * bf16 needs about 1.5 MiB).  Every call on one GPU shares that GPU's
 * scratch, whatever its stream: calls that can overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results;
 * serialise them, or give each its own workspace and use sv_spec_verify.
 * sv_workspace_status(stream, NULL, 0, ...) reads and clears the scratch's
 * status word on the current device. */
#define SV_STATIC_SCRATCH_BYTES (8u << 20)
int sv_spec_verify_static(void* stream, int B, int V, int max_k, int dtype,
                          const void* draft_logits, const int64_t* draft_row_start,
                          int64_t draft_row_stride,
                          const void* target_logits, const int64_t* target_row_start,
                          int64_t target_row_stride,
                          const int32_t* num_draft, const int32_t* draft_tokens,
                          const float* temperature, const float* u_accept,
                          const float* u_residual, const float* u_bonus,
                          int32_t* accept_len, int32_t* out_tokens, int8_t* labels,
                          float* p_draft_at_token, float* p_target_at_token,
                          const float* av_params, float* av_feature, float* av_score);

/* Bytes of workspace needed by sv_spec_verify_filtered (the verification
 * workspace followed by the threshold-search histograms: about
 * B * (2*max_k + 1) * nseg * 6 KiB, nseg = ceil(V * elem_bytes / 32 KiB)).
 * Returns 0 for arguments that call would reject.  Same zero-fill-once
 * contract as sv_workspace_size. */
size_t sv_filtered_workspace_size(int B, int V, int max_k, int dtype);

/* Batched speculative verification on top-k / top-p filtered distributions.
 *
 * [AV] "Adaptive Verification ohne Confidence Head", sections "Other
 * features considered" and "Benchmarks", sample drafts and verify them at
 * temperature 1 with top-p 0.95; the verification of [CS] "One speculative
 * step" then compares the filtered draft and target distributions.  The
 * pages define neither filter; the readings implemented:
 *   top-p   token v of a row is kept when the tokens whose logit is strictly
 *           larger than z_v hold less than top_p of softmax(row / T)
 *           (equal logits are kept or dropped together);
 *   top-k   v is kept when fewer than top_k tokens have a strictly larger
 *           logit (the k largest values, ties included);
 *   both    v must be kept by both, each evaluated on the full row;
 * and every draft row and target row of a stochastic request is replaced by
 * its filtered, renormalised distribution p'(v) = p(v) [v kept] / (sum of p
 * over the kept tokens) before steps 2-4 of sv_spec_verify, which are
 * otherwise unchanged (a draft token outside its draft row's kept set has
 * p' = 0 and is accepted, the ratio being +inf).  Greedy requests (T = 0)
 * are verified as in sv_spec_verify: the argmax is always kept.
 *
 * Arguments as for sv_spec_verify (no estimator outputs), plus:
 *   top_k   int32 [B]   top_k[b] <= 0 or >= V: no top-k filter.
 *   top_p   float [B]   top_p[b] >= 1 (or NaN): no top-p filter; otherwise
 *           0 < top_p[b] < 1 (device precondition).
 *   Device precondition of a filtered row (besides sv_spec_verify's): its
 *   logits z satisfy |z| * 8 * log2(e) / T < 2^21 (fp32 rows' level 0 and
 *   the first key level of bf16 rows whose threshold lies below their key
 *   window bin by cells of 1/8 log2 unit on an absolute grid, formed
 *   exactly in fp32).
 *   kept    int32 [B*(2*max_k+1)]  nullable: per row slot (draft rows
 *           0..max_k-1, then target rows 0..max_k) the number of tokens kept
 *           by the filters, -1 for rows not filtered or not read.
 *   p_draft_at_token, p_target_at_token: the filtered probabilities p'.
 *   workspace: at least sv_filtered_workspace_size(B, V, max_k, dtype)
 *           bytes, zero-filled once.
 * The kept sets are exact to the resolution of the mass sums: fp32 rows'
 * level-0 sums are integers (2^-23 of a bin's lower edge, the binary32
 * weights relative to that edge added exactly); bf16 rows' level 0 counts
 * tokens per key exactly (a key's mass is its count times its weight, in
 * binary64) and takes the row's total from binary32 sums of eight weights
 * added in binary64; key levels sum integers (2^-40 of the row maximum's
 * probability).  Every mass compared, the row's total included, is within
 * 2^-22 of the row's total of the sum of the weights it stands for, and
 * independent of the order of the additions;
 * the top-p comparison is made on them in binary64, the threshold found by a
 * radix select over the logits' order-preserving keys.  Outputs are a
 * deterministic function of the inputs.  Returns SV_OK, or a negative
 * sv_status without launching. */
int sv_spec_verify_filtered(void* stream, int B, int V, int max_k, int dtype,
                            const void* draft_logits, const int64_t* draft_row_start,
                            int64_t draft_row_stride,
                            const void* target_logits, const int64_t* target_row_start,
                            int64_t target_row_stride,
                            const int32_t* num_draft, const int32_t* draft_tokens,
                            const float* temperature, const int32_t* top_k,
                            const float* top_p, const float* u_accept,
                            const float* u_residual, const float* u_bonus,
                            int32_t* accept_len, int32_t* out_tokens, int8_t* labels,
                            float* p_draft_at_token, float* p_target_at_token,
                            int32_t* kept, void* workspace, size_t workspace_bytes);

/* Acceptance-estimator scoring of the draft rows, before verification.
 *
 * [AV] "Solution" / "Scoring the distribution": per draft row i of request b
 *   feature[b*max_k+i] = logit(q_max), q_max the largest probability of
 *       softmax(row / T) (T = 0 is scored at T = 1), computed as
 *       -log(sum over v != argmax of exp((z_v - z_max) / T)), which equals
 *       logit(q_max) exactly and counts tied maxima; clamped to <= 80;
 *   score[b*max_k+i] = sigmoid(omega * feature + beta_i), params = [omega,
 *       beta_0, ..., beta_{max_k-1}] (one shared slope, one intercept per
 *       position: max_k + 1 parameters);
 *   num_kept[b] (nullable) = the number of leading positions whose survival,
 *       the running product of the scores ([AV] "Other features
 *       considered"), is >= prune_threshold; K_b when prune_threshold <= 0.
 *       It can be passed as num_draft of a following sv_spec_verify call.
 * Entries past K_b are NaN.  Uses the same workspace as sv_spec_verify.
 * Device preconditions: as for sv_spec_verify's draft rows. */
int sv_av_score(void* stream, int B, int V, int max_k, int dtype,
                const void* draft_logits, const int64_t* draft_row_start,
                int64_t draft_row_stride, const int32_t* num_draft,
                const float* temperature, const float* params,
                float prune_threshold, float* feature, float* score,
                int32_t* num_kept, void* workspace, size_t workspace_bytes);

/* One step of the estimator's online refit ([AV] "Fitting the coefficients").
 *
 * Over the labelled drafts of the batch (labels 0 or 1; -1 is skipped), at
 * the parameters `params` held fixed for the round, with
 * pi = sigmoid(omega*x + beta_i), w = pi(1-pi), r = pi - y, it adds to
 * accum[i*6 + k], k = 0..5, the sums  n_i, sum w, sum w*x, sum w*x^2,
 * sum r, sum r*x  (fp64).  These are the entries of the gradient g and the
 * Hessian H of the summed negative log-likelihood: H is an arrowhead
 * (slope row/column plus a diagonal over the intercepts).
 * If do_update != 0 (last step of the round) it then solves H * delta = -g
 * over the slope and the intercepts of positions with labels (ridge added to
 * H's diagonal), scales the slope's step by N/(N + damping_c) (N = all
 * labels) and each intercept's by n_i/(n_i + damping_c), then scales the
 * whole step down, if needed, so that no parameter moves by more than
 * max_step, adds it to params (fp32, in place) and zero-fills accum.  The
 * bound is a safeguard the page does not state: far from the optimum (where
 * the sigmoid is flat, so H is small against g) a full Newton step on the
 * logistic loss overshoots, and a position whose labels all agree has no
 * finite optimum; scaling keeps the Newton direction, a descent direction.
 * Typical values: damping_c = 10, ridge = 1e-6, max_step = 1 (logit units);
 * max_step = +inf disables the bound.
 *   feature  float [B*max_k], labels int8 [B*max_k] (e.g. from sv_spec_verify).
 *   params   float [max_k+1] in/out.   accum double [6*max_k] in/out,
 *            zero-filled by the caller before a round's first step.
 * A round with no labels leaves params unchanged. */
int sv_av_fit_step(void* stream, int B, int max_k, const float* feature,
                   const int8_t* labels, float* params, double* accum,
                   float damping_c, float ridge, float max_step, int do_update);

/* The estimator's global draft budget: how many draft tokens of the batch to
 * verify, and which.
 *
 * [AV] "Other features considered" (the budget decision): the survival of
 * request b's draft i is the running product score_0 * ... * score_i (binary32,
 * left to right) over the positions i < K_b = num_draft[b]; the batch's
 * survivals are ranked, highest first (equal ones by flat index
 * b*max_k + i); keeping the j highest is estimated to emit
 * E(j) = B + (sum of those j survivals) tokens, and the budget is the j in
 * 0..N (N = sum K_b) maximising E(j) / (draft_cost_ms[j] + verify_cost_ms[j]),
 * the smallest such j on ties (sums and ratios in binary64).  The kept drafts
 * of a request are always a prefix of its positions.
 *   score          float [B*max_k]   per-position scores in [0, 1] (e.g. the
 *                  `score` output of sv_av_score).
 *   num_draft      int32 [B]         K_b.
 *   draft_cost_ms, verify_cost_ms   float [B*max_k + 1]: the measured cost of
 *                  a step that verifies j draft tokens, by j (only 0..N read).
 * Outputs (device): num_kept int32 [B] (kept prefix length, <= K_b, summing to
 * the budget), budget int32 [1].
 * One workgroup decides the whole batch: B*max_k <= SV_BUDGET_MAX_ITEMS, else
 * SV_ERR_UNSUPPORTED.  B = 0 launches nothing and writes nothing.
 * Device preconditions: 0 <= K_b <= max_k; scores in [0, 1]; every cost sum
 * read is > 0.
 * Returns SV_OK, or a negative sv_status without launching anything. */
#define SV_BUDGET_MAX_ITEMS 4096
int sv_av_budget(void* stream, int B, int max_k, const float* score, const int32_t* num_draft,
                 const float* draft_cost_ms, const float* verify_cost_ms, int32_t* num_kept,
                 int32_t* budget);

/* Calibration metrics of the estimator over its labelled stream.
 *
 * [AV] "Other features considered": AUC = probability that an accepted draft
 * scores above a rejected one (ties count half); log-loss = mean negative
 * log-probability of the observed outcome; ECE = sum over probability bins of
 * (share of the drafts in the bin) * |mean score - observed frequency|.
 * The labels are the refit's ([AV] "Fitting the coefficients"): 1 accepted,
 * 0 the first rejection, anything else (e.g. -1 from sv_spec_verify) no
 * label, skipped.
 *
 * accum: caller-owned binary64 [SV_CALIB_WORDS], zero-filled before a
 * stream's first call: labelled count, accepted count, sum of the log-loss
 * terms (scores clamped to [1e-7, 1 - 1e-7]), per ECE bin (10 equal-width
 * bins; score p in bin min(floor(10 p), 9)) the count, score sum and label
 * sum, then per class (accepted, rejected) a histogram of the score over
 * SV_CALIB_AUC_BINS equal-width bins.  The AUC is that of the binned scores:
 * scores in one bin count as tied.
 *
 * sv_av_calib_accumulate adds B*max_k (score, label) items (row-major, e.g.
 * the score and labels outputs of one verification step).  One workgroup
 * with a fixed summation order: the same calls give bit-identical results.
 * sv_av_calib_metrics writes metrics float64 [3] = AUC, log-loss, ECE (NaN
 * when undefined: no labels, or no accepted or no rejected draft for the
 * AUC) and, if reset != 0, zero-fills accum afterwards (a kernel store: safe
 * inside a captured graph).
 * Device preconditions: scores in [0, 1].  Both return SV_OK, or a negative
 * sv_status without launching anything. */
#define SV_CALIB_AUC_BINS 4096
#define SV_CALIB_WORDS (33 + 2 * SV_CALIB_AUC_BINS)
int sv_av_calib_accumulate(void* stream, int B, int max_k, const float* score, const int8_t* labels,
                           double* accum);
int sv_av_calib_metrics(void* stream, double* accum, double* metrics, int reset);

/* The test-time-speculation distillation gradient over the canvas.
 *
 * Page "ملخص تقني: التخمين في وقت الاختبار (TTS)", section "Algorithm", step 3:
 * one gradient step of the draft model on L_t(q) = KL~(p || q) + lambda *
 * KL~(q_t || q) with position weights w_k.  For each canvas position k < K_b
 * of request b (the draft row k, the target row k as teacher, and the row
 * of the drafter that produced the canvas, q_t):
 *   grad[(b*max_k + k)*V + v] = w_k * ((q(v) - p(v)) + lambda * (q(v) - q_t(v))) / T
 *     (the gradient of the loss with respect to the draft logits z_v),
 *   loss[b*max_k + k] = w_k * (KL(p || q) + lambda * KL(q_t || q))  (nats),
 * with p, q, q_t = softmax(logits / T) at the request's temperature (T = 0
 * counts as 1).  Rows k >= K_b: loss NaN, grad row not written.
 *   draft_logits, target_logits: rows as for sv_spec_verify (dtype).
 *   prev_logits / prev_row_start / prev_row_stride: the rows of q_t; NULL
 *                  means the draft rows themselves (then the lambda terms
 *                  vanish: the gradient step is taken at q = q_t).
 *   num_draft int32 [B], temperature float [B], weights float [max_k] (w_k).
 *   verify_workspace, workspace_bytes: NULL, or the workspace of the
 *                  sv_spec_verify call just made on the same rows, B, V,
 *                  max_k, dtype, temperatures and row starts (no call on that
 *                  workspace in between): the softmax statistics of the draft
 *                  and target rows are then taken from it instead of a pass
 *                  over the rows; without prev_logits the gradient is then
 *                  computed by row segments, whose losses this call writes
 *                  into the workspace's own region and sums in segment order.
 *                  That call must have read every canvas draft row: each
 *                  request stochastic (T > 0), or the call made with
 *                  av_feature.  A greedy request's target rows, of which
 *                  the verification keeps only maxima and argmaxes, are
 *                  summed again by this call (one pass over those rows).
 * Outputs (device): grad, elements of type dtype (bf16 rounded to nearest
 * even), [B*max_k, V] row-major; loss float [B*max_k].
 * Device preconditions as for sv_spec_verify.  Returns SV_OK, or a negative
 * sv_status without launching anything (SV_ERR_WORKSPACE if workspace_bytes
 * is below sv_workspace_size for these sizes). */
int sv_tts_grad(void* stream, int B, int V, int max_k, int dtype,
                const void* draft_logits, const int64_t* draft_row_start, int64_t draft_row_stride,
                const void* target_logits, const int64_t* target_row_start, int64_t target_row_stride,
                const void* prev_logits, const int64_t* prev_row_start, int64_t prev_row_stride,
                const int32_t* num_draft, const float* temperature, const float* weights, float lambda,
                void* grad, float* loss, void* verify_workspace, size_t workspace_bytes);

/* Status of a workspace, for the calls made on it so far.
 *
 * The draw of sv_spec_verify hands each row segment's weight to the
 * request's last workgroup, which waits for it (the hardware dispatches
 * workgroups in order, so the wait ends); the wait is bounded, and if it ever
 * gave up - only possible if that dispatch order were broken - the call's
 * emitted token for the request is not valid and the workspace's status word
 * is set.  This call copies the status word to *status (device int32: 0 =
 * every call so far completed normally) and, if clear != 0, zeroes it.  A
 * nonzero status also means a hand-off slot may have been left filled: zero-
 * fill the whole workspace before reusing it.  Asynchronous on `stream`, like
 * the other calls: read *status once the stream has reached this point.
 * workspace = NULL selects the static scratch of sv_spec_verify_static on
 * the current device (workspace_bytes is then ignored).
 * Returns SV_OK, SV_ERR_WORKSPACE (workspace too small), SV_ERR_INVALID_ARG
 * (status NULL) or SV_ERR_HIP (the static scratch could not be set up). */
int sv_workspace_status(void* stream, void* workspace, size_t workspace_bytes, int32_t* status, int clear);

/* Static description of a status code. */
const char* sv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
