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

Readings (the page gives no sizes or constants):

* ECE uses 10 equal-width bins of [0, 1]; a score p falls into bin
  min(floor(10 p), 9);
* the stream keeps, per class, a histogram of 4096 equal-width score bins
  (bin min(floor(4096 p), 4095)); the AUC is that of the binned scores, so
  two scores in one bin count as a tie - it equals the exact AUC when no
  accepted and rejected draft share a bin, and differs from it by at most
  half the share of accepted/rejected pairs that do;
* log-loss clamps p to [1e-7, 1 - 1e-7] (parity unpinned: the constant).
"""
from __future__ import annotations

import numpy as np

ECE_BINS = 10
AUC_BINS = 4096
EPS = 1e-7


def _items(scores, labels):
    p = np.asarray(scores, dtype=np.float32).reshape(-1)
    y = np.asarray(labels).reshape(-1)
    keep = (y == 0) | (y == 1)
    return p[keep].astype(np.float64), y[keep].astype(np.int64), p[keep]


def ece_bin(p32):
    return np.minimum(np.floor(np.asarray(p32, np.float32) * np.float32(ECE_BINS)).astype(np.int64), ECE_BINS - 1)


def auc_bin(p32):
    return np.minimum(np.floor(np.asarray(p32, np.float32) * np.float32(AUC_BINS)).astype(np.int64), AUC_BINS - 1)


def metrics(scores, labels) -> dict:
    """AUC, log-loss and ECE of the labelled items (labels 0/1; others skipped).

    Bin indices are taken on the binary32 scores, as the kernels see them."""
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
    # AUC over the binned scores: P(pos > neg) + 1/2 P(pos == neg)
    ab = auc_bin(p32)
    pos = np.bincount(ab[y == 1], minlength=AUC_BINS).astype(np.float64)
    neg = np.bincount(ab[y == 0], minlength=AUC_BINS).astype(np.float64)
    npos, nneg = pos.sum(), neg.sum()
    if npos == 0 or nneg == 0:
        out["auc"] = float("nan")
    else:
        below = np.cumsum(neg) - neg  # rejected drafts in lower bins
        out["auc"] = float((pos * below).sum() + 0.5 * (pos * neg).sum()) / (npos * nneg)
    return out
