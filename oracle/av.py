"""Oracle for the online acceptance estimator - TEST INFRASTRUCTURE ONLY.

Follows [AV] "Adaptive Verification ohne Confidence Head" (and its Arabic
mirror):

* "Solution" / "Scoring the distribution": the acceptance probability of
  the draft at position i is a logistic regression on one scalar, the
  log-odds of the draft's most likely token, x = logit(q_max), with one
  slope shared by all positions and one intercept per position:
  score_i = sigmoid(omega * x + beta_i)  (K + 1 parameters).  The displayed
  formula is lost from the extracted page; the surrounding prose fixes it.
* "Other features considered": survival probabilities are the running
  product of the scores over positions.
* "Fitting the coefficients": only drafts up to and including the first
  rejection carry labels; IRLS minimises the log-likelihood loss by a
  second-order Taylor step, solving H * dtheta = -g with H the (K+1)x(K+1)
  Hessian and g the gradient; H and g are accumulated over a round of decode
  steps and the system is solved on its last step; each coefficient's step
  is scaled by n / (n + constant), n the number of scored drafts behind it.

Readings (parity unpinned where marked):

* the feature uses the request's temperature, T = 0 counting as T = 1
  (unpinned); x = -log(sum_{v != v*} exp(s_v - s_max)), which equals
  logit(q_max) exactly and counts tied maxima; x is clamped at 80 (unpinned);
* the survival prune keeps the leading positions whose survival is >= the
  threshold; a threshold <= 0 keeps every position;
* H and g are evaluated at the round's fixed parameters; positions with no
  labels in the round drop out of the solve; a ridge ``ridge`` is added to
  H's diagonal and ``damping_c`` is the damping constant (both unpinned);
  the slope's n is the total label count, each intercept's n its own count;
* a step bound: far from the optimum a full Newton step on the logistic loss
  overshoots (where the sigmoid is flat, H is tiny against g), and a position
  whose labels all agree has no finite optimum at all, so the damped step is
  scaled as a whole, when needed, until no parameter moves by more than
  ``max_step`` in one refit.  Scaling keeps the Newton direction, a descent
  direction of the convex loss; near the optimum the steps are small and the
  page's damped step is taken unchanged (the bound's value is unpinned).
"""
from __future__ import annotations

import numpy as np

from .verify import decode_rows

FEATURE_CLAMP = 80.0


def feature(z: np.ndarray, T: float) -> float:
    """x = logit(q_max) of softmax(z / T) for one draft row."""
    T = 1.0 if T == 0.0 else T
    s = np.asarray(z, dtype=np.float64) / T
    top = int(np.argmax(s))
    others = np.exp(s - s[top])
    others[top] = 0.0
    s_other = float(np.sum(others))
    if s_other <= 0.0:
        return FEATURE_CLAMP
    return min(-np.log(s_other), FEATURE_CLAMP)


def _sigmoid(t: float) -> float:
    if t >= 0:
        return 1.0 / (1.0 + np.exp(-t))
    e = np.exp(t)
    return e / (1.0 + e)


def score(x: float, params, i: int) -> float:
    """sigmoid(omega * x + beta_i); params = [omega, beta_0, ...]."""
    return _sigmoid(float(params[0]) * x + float(params[1 + i]))


def survival_and_kept(scores, threshold: float):
    """Running product of the scores and the count of leading positions
    whose survival is >= threshold (all of them when threshold <= 0)."""
    surv = np.cumprod(np.asarray(scores, dtype=np.float64))
    if threshold <= 0.0:
        return surv, len(surv)
    kept = 0
    for s in surv:
        if s >= threshold:
            kept += 1
        else:
            break
    return surv, kept


def av_score_batch(batch, params=None, threshold=None, requests=None) -> dict:
    """Feature, score, survival and kept count for (a subset of) a batch."""
    params = batch.av_params if params is None else params
    threshold = batch.prune_threshold if threshold is None else threshold
    idx = np.arange(batch.B) if requests is None else np.asarray(requests)
    n, mk = len(idx), batch.max_k
    out = {"requests": idx, "feature": np.full((n, mk), np.nan), "score": np.full((n, mk), np.nan),
           "survival": np.full((n, mk), np.nan), "num_kept": np.zeros(n, np.int32)}
    for r, b in enumerate(idx):
        k = int(batch.num_draft[b])
        ds = int(batch.draft_row_start[b])
        T = float(batch.temperature[b])
        for i in range(k):
            z = decode_rows(batch.draft[ds + i], batch.dtype)
            out["feature"][r, i] = feature(z, T)
            out["score"][r, i] = score(out["feature"][r, i], params, i)
        surv, kept = survival_and_kept(out["score"][r, :k], threshold)
        out["survival"][r, :k] = surv
        out["num_kept"][r] = kept
    return out


# ----------------------------------------------------------------------------
# fitting
# ----------------------------------------------------------------------------

SUM_NAMES = ("n", "A", "B", "C", "gb", "gw")


def fit_sums(feature_arr, labels, params) -> np.ndarray:
    """Per-position sums over the labelled drafts, at fixed parameters.

    For each labelled draft (label 0 or 1) at position i with feature x:
    pi = sigmoid(omega*x + beta_i), w = pi(1-pi), r = pi - y, and
    n_i += 1, A_i += w, B_i += w*x, C_i += w*x^2, gb_i += r, gw_i += r*x.
    Returns float64 [max_k, 6] in the order of ``SUM_NAMES``.
    """
    feature_arr = np.asarray(feature_arr, dtype=np.float32).astype(np.float64)
    labels = np.asarray(labels)
    p = np.asarray(params, dtype=np.float32).astype(np.float64)
    mk = feature_arr.shape[1]
    sums = np.zeros((mk, 6))
    for b in range(feature_arr.shape[0]):
        for i in range(mk):
            y = int(labels[b, i])
            if y not in (0, 1):
                continue
            x = feature_arr[b, i]
            pi = _sigmoid(p[0] * x + p[1 + i])
            w = pi * (1.0 - pi)
            r = pi - y
            sums[i] += (1.0, w, w * x, w * x * x, r, r * x)
    return sums


def hessian_gradient(sums: np.ndarray, ridge: float = 0.0):
    """Dense (K+1)x(K+1) Hessian and gradient of the summed negative
    log-likelihood in the parameter order [omega, beta_0..beta_{K-1}]."""
    mk = sums.shape[0]
    H = np.zeros((mk + 1, mk + 1))
    g = np.zeros(mk + 1)
    H[0, 0] = sums[:, 3].sum() + ridge
    g[0] = sums[:, 5].sum()
    for i in range(mk):
        H[0, 1 + i] = H[1 + i, 0] = sums[i, 2]
        H[1 + i, 1 + i] = sums[i, 1] + ridge
        g[1 + i] = sums[i, 4]
    return H, g


def newton_step(sums: np.ndarray, params, damping_c: float, ridge: float, max_step: float = 1.0) -> np.ndarray:
    """Damped Newton update of the parameters from accumulated sums.

    Solves H * delta = -g over the slope and the intercepts of positions that
    have labels, scales the slope's step by N/(N+c) (N = all labels) and each
    intercept's by n_i/(n_i+c), then scales the whole damped step down so that
    its largest component is at most ``max_step`` (infinity: no bound), and
    returns params + delta in float64.
    """
    p = np.asarray(params, dtype=np.float32).astype(np.float64)
    n = sums[:, 0]
    N = n.sum()
    if N == 0:
        return p.copy()
    H, g = hessian_gradient(sums, ridge)
    keep = np.concatenate([[True], n > 0])
    delta = np.zeros_like(p)
    delta[keep] = np.linalg.solve(H[np.ix_(keep, keep)], -g[keep])
    scale = np.concatenate([[N / (N + damping_c)], n / (n + damping_c)])
    step = delta * scale
    largest = np.max(np.abs(step))
    if largest > max_step:
        step = step * (max_step / largest)
    return p + step


def fit_step(feature_arr, labels, params, accum, damping_c=10.0, ridge=1e-6, do_update=False, max_step=1.0):
    """One call of the batched refit: add this step's sums to ``accum``
    ([max_k, 6] float64); on the round's last step solve, update and clear.
    Returns (params float32, accum float64)."""
    accum = np.asarray(accum, dtype=np.float64) + fit_sums(feature_arr, labels, params)
    params = np.asarray(params, dtype=np.float32)
    if do_update:
        params = newton_step(accum, params, damping_c, ridge, max_step).astype(np.float32)
        accum = np.zeros_like(accum)
    return params, accum


def nll(feature_arr, labels, params) -> float:
    """Summed negative log-likelihood of the labelled drafts."""
    feature_arr = np.asarray(feature_arr, dtype=np.float64)
    p = np.asarray(params, dtype=np.float64)
    total = 0.0
    for b in range(feature_arr.shape[0]):
        for i in range(feature_arr.shape[1]):
            y = int(labels[b, i])
            if y not in (0, 1):
                continue
            t = p[0] * feature_arr[b, i] + p[1 + i]
            total += np.logaddexp(0.0, -t) if y == 1 else np.logaddexp(0.0, t)
    return float(total)
