"""Oracle for one verification step - TEST INFRASTRUCTURE ONLY (see package doc).

Follows [CS] "Speculative Decoding: Draft, EAGLE, MTP", sections "One
speculative step" and "Algorithm loop in code":

1. the draft proposes K tokens with per-position distributions pd_0..pd_{K-1};
2. the verifier returns K+1 distributions pt_0..pt_K in one pass;
3. walk left to right; accept token d_i with probability min(1, pt_i(d_i) /
   pd_i(d_i)), the ratio being +inf when pd_i(d_i) = 0;
4. at the first rejection j, sample from the normalised residual
   (pt_j - pd_j)+ and discard the later drafts;
5. if all K are accepted, sample one bonus token from pt_K.

Readings taken where the page leaves a step open (each listed in the design
notes of the repository):

* distributions are the temperature-scaled softmax of the logit rows,
  softmax(z / T), on both draft and target rows;
* one uniform per draft position decides acceptance with a strict ``<``;
  ``u_residual`` and ``u_bonus`` drive the two possible samples;
* "sample" is the inverse CDF in ascending token order: the first v with
  C(v) > u * Z, C the running sum of the (unnormalised) weights and Z their
  total; if rounding leaves no such v, the last positive-weight token;
* if the residual has no mass (Z = 0, unreachable in exact arithmetic after a
  rejection) the target row itself is sampled - parity unpinned;
* T = 0 means greedy verification: a draft is accepted iff it equals the
  lowest-index argmax of its target row, and the emitted correction or bonus
  is that argmax (the T -> 0 limit of steps 3-5);
* labels for the acceptance estimator: 1 for positions before the first
  rejection, 0 at it, -1 after it ([AV] "Fitting the coefficients": only
  drafts up to the first rejection are labelled).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def decode_rows(rows: np.ndarray, dtype: str) -> np.ndarray:
    """Logit rows as float64.  ``dtype`` "bf16" means uint16 bit patterns,
    widened exactly (bf16 is the top half of an IEEE binary32)."""
    if dtype == "bf16":
        bits = np.asarray(rows, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(rows, dtype=np.float32).astype(np.float64)


def log_softmax(z: np.ndarray, T: float) -> np.ndarray:
    """log softmax(z / T) of one row, stabilised by the row maximum.

    [CS] "One speculative step": each position's distribution over the
    vocabulary.  -inf logits give probability 0.
    """
    s = np.asarray(z, dtype=np.float64) / T
    m = np.max(s)
    return s - (m + np.log(np.sum(np.exp(s - m))))


def accept_decision(log_pd_d: float, log_pt_d: float, u: float):
    """[CS] "Algorithm loop in code": ratio = pt(d)/pd(d), +inf when
    pd(d) = 0; accept iff u < min(1, ratio).

    Returns (accept, ratio, margin) with margin = |u - min(1, ratio)|.
    """
    if log_pd_d == -np.inf:
        ratio = np.inf
    else:
        ratio = float(np.exp(log_pt_d - log_pd_d))
    bound = min(1.0, ratio)
    return bool(u < bound), ratio, abs(float(u) - bound)


def inverse_cdf(weights: np.ndarray, u: float):
    """Sample index from unnormalised non-negative ``weights`` with uniform u.

    Returns (token, margin): the first v with C(v) > u*Z in ascending order,
    and the distance of u*Z to the nearer edge of that token's CDF interval,
    divided by Z (0 when the rounding fallback was taken).
    """
    w = np.asarray(weights, dtype=np.float64)
    C = np.cumsum(w)
    Z = C[-1]
    t = float(u) * Z
    tok = int(np.searchsorted(C, t, side="right"))
    if tok >= len(w):
        return int(np.nonzero(w > 0)[0][-1]), 0.0
    lo = C[tok - 1] if tok > 0 else 0.0
    return tok, float(min(t - lo, C[tok] - t) / Z)


@dataclass
class VerifyResult:
    accept_len: int  # a: number of accepted drafts
    tokens: np.ndarray  # emitted tokens, length a + 1
    labels: np.ndarray  # int8 [K]
    p_draft: np.ndarray  # pd_i(d_i), [K] (NaN for greedy requests)
    p_target: np.ndarray  # pt_i(d_i), [K] (one-hot limit for greedy requests)
    accept_margin: np.ndarray  # |u_i - min(1, ratio_i)|, [K]; inf where not decided by a float
    cdf_margin: float  # margin of the residual / bonus sample; inf for greedy


def verify_request(zd: np.ndarray, zt: np.ndarray, d, T: float, u_accept, u_residual: float,
                   u_bonus: float) -> VerifyResult:
    """One request: ``zd`` [K, V] draft logits, ``zt`` [K+1, V] target logits
    (float64), ``d`` [K] draft tokens, temperature ``T``."""
    K = zd.shape[0]
    d = [int(x) for x in d]
    labels = np.full(K, -1, dtype=np.int8)
    margins = np.full(K, np.inf)
    p_draft = np.full(K, np.nan)
    p_target = np.full(K, np.nan)

    if T == 0.0:
        # greedy: accept iff the draft equals the target's lowest-index argmax
        top = [int(np.argmax(zt[j])) for j in range(K + 1)]
        a = K
        for i in range(K):
            p_target[i] = 1.0 if d[i] == top[i] else 0.0
            if d[i] != top[i]:
                a = i
                break
        for i in range(a + 1, K):
            p_target[i] = 1.0 if d[i] == top[i] else 0.0
        tokens = np.array(d[:a] + [top[a]], dtype=np.int64)
        labels[:a] = 1
        if a < K:
            labels[a] = 0
        return VerifyResult(a, tokens, labels, p_draft, p_target, margins, np.inf)

    log_pd = [log_softmax(zd[i], T) for i in range(K)]
    log_pt = [log_softmax(zt[j], T) for j in range(K + 1)]
    return verify_logprobs(log_pd, log_pt, d, u_accept, u_residual, u_bonus)


def verify_logprobs(log_pd, log_pt, d, u_accept, u_residual: float, u_bonus: float) -> VerifyResult:
    """Steps 3-5 of [CS] "One speculative step" on given distributions:
    ``log_pd`` K rows and ``log_pt`` K+1 rows of log-probabilities (-inf for
    probability 0), draft tokens ``d``."""
    K = len(log_pd)
    d = [int(x) for x in d]
    labels = np.full(K, -1, dtype=np.int8)
    margins = np.full(K, np.inf)
    p_draft = np.full(K, np.nan)
    p_target = np.full(K, np.nan)
    a = K
    for i in range(K):
        p_draft[i] = np.exp(log_pd[i][d[i]])
        p_target[i] = np.exp(log_pt[i][d[i]])
    for i in range(K):
        ok, _, margins[i] = accept_decision(log_pd[i][d[i]], log_pt[i][d[i]], u_accept[i])
        if not ok:
            a = i
            break
    margins[a + 1:] = np.inf  # later positions are discarded, never compared
    if a < K:
        pt, pd = np.exp(log_pt[a]), np.exp(log_pd[a])
        resid = np.maximum(0.0, pt - pd)
        if not np.cumsum(resid)[-1] > 0.0:
            resid = pt
        tok, cdf_margin = inverse_cdf(resid, u_residual)
    else:
        tok, cdf_margin = inverse_cdf(np.exp(log_pt[K]), u_bonus)
    tokens = np.array(d[:a] + [tok], dtype=np.int64)
    labels[:a] = 1
    if a < K:
        labels[a] = 0
    return VerifyResult(a, tokens, labels, p_draft, p_target, margins, cdf_margin)


def verify_batch(batch, requests=None) -> dict:
    """Run ``verify_request`` over (a subset of) a ``synth.Batch``.

    Returns arrays shaped like the library's outputs for the selected
    requests: accept_len [n], out_tokens [n, max_k+1] (-1 past the emitted
    tokens), labels [n, max_k], p_draft/p_target [n, max_k], plus the
    margins used by the parity rules.
    """
    idx = np.arange(batch.B) if requests is None else np.asarray(requests)
    n, mk = len(idx), batch.max_k
    out = {
        "requests": idx,
        "accept_len": np.zeros(n, np.int32),
        "out_tokens": np.full((n, mk + 1), -1, np.int32),
        "labels": np.full((n, mk), -1, np.int8),
        "p_draft": np.full((n, mk), np.nan),
        "p_target": np.full((n, mk), np.nan),
        "accept_margin": np.full((n, mk), np.inf),
        "cdf_margin": np.full(n, np.inf),
    }
    for r, b in enumerate(idx):
        k = int(batch.num_draft[b])
        ds, ts = int(batch.draft_row_start[b]), int(batch.target_row_start[b])
        zd = decode_rows(batch.draft[ds:ds + k], batch.dtype) if k else np.zeros((0, batch.V))
        zt = decode_rows(batch.target[ts:ts + k + 1], batch.dtype)
        res = verify_request(zd, zt, batch.draft_tokens[b, :k], float(batch.temperature[b]),
                             batch.u_accept[b, :k], float(batch.u_residual[b]), float(batch.u_bonus[b]))
        out["accept_len"][r] = res.accept_len
        out["out_tokens"][r, :res.accept_len + 1] = res.tokens
        out["labels"][r, :k] = res.labels
        out["p_draft"][r, :k] = res.p_draft
        out["p_target"][r, :k] = res.p_target
        out["accept_margin"][r, :k] = res.accept_margin
        out["cdf_margin"][r] = res.cdf_margin
    return out
