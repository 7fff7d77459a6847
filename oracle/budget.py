"""Oracle for the estimator's global draft budget - TEST INFRASTRUCTURE ONLY.

Follows [AV] "Adaptive Verification ohne Confidence Head" (its Arabic mirror
prints the code of the decision), section "Other features considered":

* survival probabilities are the running product of the scores along each
  request's draft positions;
* the survivals of the whole batch are flattened and ranked, and the
  `draft_budget` highest are the drafts kept (the top-k of the flat tensor);
* the estimated number of accepted tokens after keeping the j highest is the
  number of sampling requests plus the sum of those j survivals (j = 0 keeps
  no draft: every request still emits one token);
* a measured cost table gives the time of a step with j draft tokens (draft
  cost plus verify cost); the budget is the j that maximises estimated
  tokens per unit of cost.

Readings (the page elides the indices and sizes):

* only positions i < K_b take part; N = sum_b K_b entries, j = 0..N;
* the number of sampling requests is B (every request emits at least one
  token);
* both cost tables are indexed by j, the number of draft tokens verified in
  the step, and hold at least N + 1 entries;
* the survivals are running products in binary32, left to right: the page
  forms them with ``cumprod`` over the per-position probabilities held in a
  floating-point tensor, whose default element type is binary32, and ranks
  those values; the running sums of the survivals and the ratios are
  binary64, as the page's ``np.cumsum`` and division over them;
* equal survivals are ranked by their flat index b * max_k + i (lower
  first): the page's ``topk`` leaves the order of equal values open, and
  this order makes the decision deterministic and keeps each request's kept
  drafts a prefix of its positions (a later position's survival never
  exceeds an earlier one's); equal ratios give the smallest j, the first
  maximum, as ``np.argmax`` returns.

Parity unpinned: the reading of the cost tables' index (no cost table is
printed on the page; the tables are synthetic inputs here).
"""
from __future__ import annotations

import numpy as np


def survivals(scores, num_draft) -> np.ndarray:
    """fp32 running products of the scores over positions i < K_b; 0 past
    K_b (such positions take no part)."""
    scores = np.asarray(scores, dtype=np.float32)
    B, max_k = scores.shape
    surv = np.zeros((B, max_k), dtype=np.float32)
    for b in range(B):
        run = np.float32(1.0)
        for i in range(int(np.clip(num_draft[b], 0, max_k))):
            run = np.float32(run * scores[b, i])
            surv[b, i] = run
    return surv


def global_budget(scores, num_draft, draft_cost, verify_cost):
    """The budget decision over one batch.

    Returns (budget, kept, ratios): the number of draft tokens to verify,
    the kept prefix length of every request (int32 [B], summing to budget)
    and the estimated-tokens-per-cost curve over j = 0..N (fp64).
    """
    scores = np.asarray(scores, dtype=np.float32)
    B, max_k = scores.shape
    surv = survivals(scores, num_draft)
    # the flat tensor of survivals, ranked: highest first, ties by flat index
    entries = [(b * max_k + i, float(surv[b, i]))
               for b in range(B) for i in range(int(np.clip(num_draft[b], 0, max_k)))]
    ranked = sorted(entries, key=lambda e: (-e[1], e[0]))
    n = len(ranked)
    # estimated accepted tokens for j = 0..N kept drafts
    est = np.concatenate(([float(B)], float(B) + np.cumsum([v for _, v in ranked], dtype=np.float64)))
    costs = (np.asarray(draft_cost, dtype=np.float64)[:n + 1] +
             np.asarray(verify_cost, dtype=np.float64)[:n + 1])
    ratios = est / costs
    budget = int(np.argmax(ratios))
    kept = np.zeros(B, dtype=np.int32)
    for idx, _ in ranked[:budget]:
        kept[idx // max_k] += 1
    return budget, kept, ratios
