"""Oracle of verification with top-k / top-p filtered distributions - TEST
INFRASTRUCTURE ONLY.

The acceptance-estimator page ([AV] "Adaptive Verification ohne Confidence
Head", sections "Other features considered" and "Benchmarks") collects its
labelled drafts and runs its benchmarks while sampling at temperature 1 with
top-p 0.95: the draft and target distributions that speculative sampling
([CS] "Speculative Decoding: Draft, EAGLE, MTP", "One speculative step")
verifies are then the filtered ones.  The pages define neither filter; the
readings below are the plainest ones the rest supports.

* F1 (top-p, nucleus).  Token v of a row is kept when the tokens whose logit
  is strictly larger than z_v hold less than ``top_p`` of the row's
  probability: sum_{w: z_w > z_v} p(w) < top_p.  Equal logits are kept or
  dropped together, so the kept set is a function of the values alone (the
  smallest set of most probable tokens reaching ``top_p``, ties at its
  boundary included).  ``top_p`` >= 1 disables the filter.
* F2 (top-k).  Token v is kept when fewer than ``top_k`` tokens have a
  strictly larger logit (the k largest values, ties included).
  ``top_k`` <= 0 or >= V disables it.
* F3 (both).  A token is kept when both filters keep it, each evaluated on the
  row's full temperature-scaled distribution.
* F4.  Every draft row and every target row of a stochastic request is
  filtered with the request's parameters; the filtered distribution is
  p'(v) = p(v) [v kept] / sum of p over the kept tokens, and steps 3-5 of the
  verification (accept test, residual, bonus) run on p' unchanged.  A draft
  token outside its draft row's kept set has p'_draft = 0: ratio +inf
  (accepted, as for an unfiltered zero-probability draft).
* F5.  Greedy requests (T = 0) are not filtered: the argmax is always kept,
  and greedy verification reads nothing else.

Comparisons of logits treat -0 and +0 as equal.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import verify as ov


@dataclass
class RowFilter:
    keep: np.ndarray  # bool [V]
    kept: int  # number of kept tokens
    margin: float  # top-p decision margin (inf without top-p): distance of the boundary masses to top_p


def keep_mask(z: np.ndarray, T: float, top_k: int, top_p: float) -> RowFilter:
    """F1-F3 on one logit row ``z`` (float64) at temperature ``T`` > 0.

    For each token the mass and the count of the tokens with a strictly
    larger logit are found by walking the distinct values in descending
    order (ties share one value).  The top-p margin is the smaller of
    top_p - F at the smallest kept value and F - top_p at the largest dropped
    value, F being the mass strictly above the value."""
    z = np.asarray(z, dtype=np.float64)
    V = z.shape[0]
    keep = np.ones(V, dtype=bool)
    margin = np.inf
    use_k = 0 < top_k < V
    use_p = top_p < 1.0
    if not (use_k or use_p):
        return RowFilter(keep, V, margin)
    p = np.exp(ov.log_softmax(z, T))
    zz = np.where(z == 0.0, 0.0, z)  # -0 counts as +0
    order = np.argsort(-zz, kind="stable")
    vals = zz[order]
    # first sorted index of each value's group: the count strictly above it
    new = np.ones(V, dtype=bool)
    new[1:] = vals[1:] != vals[:-1]
    group_start = np.maximum.accumulate(np.where(new, np.arange(V), 0))
    mass_before = np.concatenate([[0.0], np.cumsum(p[order])[:-1]])
    above_count = group_start  # per sorted position
    above_mass = mass_before[group_start]
    ks = np.ones(V, dtype=bool)
    if use_k:
        ks &= above_count < top_k
    if use_p:
        kp = above_mass < top_p
        ks &= kp
        starts = np.nonzero(new)[0]
        F = mass_before[starts]
        kept_groups = F < top_p
        last_kept = F[kept_groups][-1]
        margin = top_p - last_kept
        if not kept_groups.all():
            margin = min(margin, F[~kept_groups][0] - top_p)
    keep[order] = ks
    return RowFilter(keep, int(keep.sum()), float(margin))


def filtered_log_probs(z: np.ndarray, T: float, f: RowFilter) -> np.ndarray:
    """log p' of F4: log softmax(z / T) renormalised over the kept tokens,
    -inf elsewhere."""
    lp = ov.log_softmax(z, T)
    p = np.exp(lp)
    total = float(np.sum(p[f.keep]))
    return np.where(f.keep, lp - np.log(total), -np.inf)


@dataclass
class FilteredResult:
    result: ov.VerifyResult
    kept: np.ndarray  # int [2K + 1]: draft rows 0..K-1, then target rows 0..K; -1 when not filtered
    filter_margin: np.ndarray  # float [2K + 1]; inf when not filtered


def verify_request_filtered(zd: np.ndarray, zt: np.ndarray, d, T: float, top_k: int, top_p: float, u_accept,
                            u_residual: float, u_bonus: float) -> FilteredResult:
    """One request on filtered distributions (F4); ``zd`` [K, V], ``zt``
    [K+1, V] float64 logits."""
    K = zd.shape[0]
    kept = np.full(2 * K + 1, -1, dtype=np.int64)
    fm = np.full(2 * K + 1, np.inf)
    active = (0 < top_k < zt.shape[1]) or top_p < 1.0
    if T == 0.0 or not active:
        return FilteredResult(ov.verify_request(zd, zt, d, T, u_accept, u_residual, u_bonus), kept, fm)
    log_pd, log_pt = [], []
    for i in range(K):
        f = keep_mask(zd[i], T, top_k, top_p)
        kept[i], fm[i] = f.kept, f.margin
        log_pd.append(filtered_log_probs(zd[i], T, f))
    for j in range(K + 1):
        f = keep_mask(zt[j], T, top_k, top_p)
        kept[K + j], fm[K + j] = f.kept, f.margin
        log_pt.append(filtered_log_probs(zt[j], T, f))
    res = ov.verify_logprobs(log_pd, log_pt, d, u_accept, u_residual, u_bonus)
    return FilteredResult(res, kept, fm)


def verify_batch_filtered(batch, top_k, top_p, requests=None) -> dict:
    """``ov.verify_batch`` with per-request filter parameters ``top_k`` [B]
    and ``top_p`` [B]; adds per-row kept counts and top-p margins, laid out
    [n, 2*max_k + 1] (draft rows 0..max_k-1, then target rows 0..max_k)."""
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
        "kept": np.full((n, 2 * mk + 1), -1, np.int64),
        "filter_margin": np.full((n, 2 * mk + 1), np.inf),
    }
    for r, b in enumerate(idx):
        k = int(batch.num_draft[b])
        ds, ts = int(batch.draft_row_start[b]), int(batch.target_row_start[b])
        zd = ov.decode_rows(batch.draft[ds:ds + k], batch.dtype) if k else np.zeros((0, batch.V))
        zt = ov.decode_rows(batch.target[ts:ts + k + 1], batch.dtype)
        fr = verify_request_filtered(zd, zt, batch.draft_tokens[b, :k], float(batch.temperature[b]),
                                     int(top_k[b]), float(top_p[b]), batch.u_accept[b, :k],
                                     float(batch.u_residual[b]), float(batch.u_bonus[b]))
        res = fr.result
        out["accept_len"][r] = res.accept_len
        out["out_tokens"][r, :res.accept_len + 1] = res.tokens
        out["labels"][r, :k] = res.labels
        out["p_draft"][r, :k] = res.p_draft
        out["p_target"][r, :k] = res.p_target
        out["accept_margin"][r, :k] = res.accept_margin
        out["cdf_margin"][r] = res.cdf_margin
        out["kept"][r, :k] = fr.kept[:k]
        out["kept"][r, mk:mk + k + 1] = fr.kept[k:]
        out["filter_margin"][r, :k] = fr.filter_margin[:k]
        out["filter_margin"][r, mk:mk + k + 1] = fr.filter_margin[k:]
    return out
