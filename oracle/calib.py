"""Oracle for the estimator's calibration metrics - TEST INFRASTRUCTURE ONLY.

Follows [AV] "Adaptive Verification ohne Confidence Head" (and its Arabic
mirror), section "Other features considered", which judges a feature by:

* AUC: the probability that a randomly chosen accepted draft scores higher
  than a randomly chosen rejected one (ties count one half);
* log-loss: the mean negative log of the probability the score assigns to the
  observed outcome;
* ECE: the drafts are put into bins by predicted acceptance probability; the
  error between the mean prediction and the observed frequency of each bin is
  weighted by the bin's share of the drafts and summed.

The metrics run over the labelled stream of the refit ([AV] "Fitting the
coefficients": a draft is labelled 1 if accepted, 0 at the first rejection,
and carries no label after it).

The AUC is computed as the page defines it: over every (accepted,
rejected) pair of labelled drafts, the share in which the accepted one has
the higher score, an equal score counting one half (binary64 from the
binary32 scores).

Readings (the page gives no sizes or constants):

* ECE uses 10 equal-width bins of [0, 1]; a score p falls into bin
  min(floor(10 p), 9);
* log-loss clamps p to [1e-7, 1 - 1e-7] (parity unpinned: the constant).
"""
from __future__ import annotations

import numpy as np

ECE_BINS = 10
EPS = 1e-7


def _items(scores, labels):
    p = np.asarray(scores, dtype=np.float32).reshape(-1)
    y = np.asarray(labels).reshape(-1)
    keep = (y == 0) | (y == 1)
    return p[keep].astype(np.float64), y[keep].astype(np.int64), p[keep]


def ece_bin(p32):
    return np.minimum(np.floor(np.asarray(p32, np.float32) * np.float32(ECE_BINS)).astype(np.int64), ECE_BINS - 1)


def auc(p, y) -> float:
    """P(score of an accepted draft > score of a rejected one), ties one half,
    over all pairs; NaN without both classes.  Each accepted draft's wins are
    counted against the sorted rejected scores (a library sort and search)."""
    p = np.asarray(p, np.float64)
    y = np.asarray(y)
    pos, neg = p[y == 1], np.sort(p[y == 0])
    if len(pos) == 0 or len(neg) == 0:
        return float("nan")
    below = np.searchsorted(neg, pos, side="left")  # rejected drafts scoring lower
    upto = np.searchsorted(neg, pos, side="right")  # ... lower or equal
    wins = below.sum() + 0.5 * (upto - below).sum()
    return float(wins) / (float(len(pos)) * float(len(neg)))


def metrics(scores, labels) -> dict:
    """AUC, log-loss and ECE of the labelled items (labels 0/1; others skipped).

    ECE bin indices are taken on the binary32 scores, as the kernels see them."""
    p, y, p32 = _items(scores, labels)
    n = len(y)
    out = {"n": n, "n_pos": int(y.sum())}
    if n == 0:
        return {**out, "auc": float("nan"), "log_loss": float("nan"), "ece": float("nan")}
    # log-loss: mean of -log of the probability given to the observed outcome
    pc = np.clip(p, EPS, 1 - EPS)
    out["log_loss"] = float(np.mean(-(y * np.log(pc) + (1 - y) * np.log(1 - pc))))
    # ECE: sum over bins of (share of drafts) * |mean prediction - observed frequency|
    eb = ece_bin(p32)
    ece = 0.0
    for k in range(ECE_BINS):
        sel = eb == k
        if sel.any():
            ece += sel.sum() / n * abs(p[sel].mean() - y[sel].mean())
    out["ece"] = float(ece)
    out["auc"] = auc(p, y)
    return out
