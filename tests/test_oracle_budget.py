"""Pins of the global-budget oracle ([AV] "Other features considered": the
survival ranking and the argmax of estimated tokens per cost), against
closed forms, a worked example and brute force - nothing here re-runs the
oracle's own formula."""
import itertools

import numpy as np
import pytest

from oracle import av as oav
from oracle import budget as ob


def _linear_costs(n, c0, c1):
    draft = np.array([c1 * j for j in range(n + 1)], dtype=np.float32)
    verify = np.full(n + 1, c0, dtype=np.float32)
    return draft, verify


@pytest.mark.parametrize("s,c0,c1,expect_all", [(0.9, 10.0, 0.5, True), (0.02, 10.0, 0.5, False),
                                                 (0.7, 1.0, 2.0, False), (0.6, 100.0, 1.0, True)])
def test_equal_survivals_with_linear_cost_keep_all_or_nothing(s, c0, c1, expect_all):
    # one draft per request, all scores s: (B + j s) / (c0 + c1 j) is monotone in j,
    # increasing exactly when s * c0 > B * c1
    B = 8
    scores = np.full((B, 1), s, dtype=np.float32)
    draft, verify = _linear_costs(B, c0, c1)
    budget, kept, _ = ob.global_budget(scores, np.ones(B, np.int32), draft, verify)
    assert (float(np.float32(s)) * c0 > B * c1) == expect_all
    assert budget == (B if expect_all else 0)
    assert kept.tolist() == ([1] * B if expect_all else [0] * B)


def test_worked_example():
    # survivals [[0.9, 0.45], [0.8, 0.72]]; ranked 0.9, 0.8, 0.72, 0.45;
    # estimated tokens 2, 2.9, 3.7, 4.42, 4.87 over costs 10, 11.5, 13, 14.5, 16:
    # ratios 0.2, 0.2522, 0.2846, 0.3048, 0.3044 -> three drafts, request 0 keeps
    # its first, request 1 both
    scores = np.array([[0.9, 0.5], [0.8, 0.9]], dtype=np.float32)
    draft = np.array([0, 1, 2, 3, 4], dtype=np.float32)
    verify = np.array([10, 10.5, 11, 11.5, 12], dtype=np.float32)
    budget, kept, ratios = ob.global_budget(scores, np.array([2, 2], np.int32), draft, verify)
    np.testing.assert_allclose(ratios, [0.2, 2.9 / 11.5, 3.7 / 13, 4.42 / 14.5, 4.87 / 16], rtol=1e-6)
    assert budget == 3
    assert kept.tolist() == [1, 2]


def _brute(scores, num_draft, draft, verify):
    """Every j, with the j kept drafts chosen as the j largest survivals by
    exhaustive comparison of prefix-closed choices."""
    B, max_k = scores.shape
    k = [int(np.clip(num_draft[b], 0, max_k)) for b in range(B)]
    surv = [[float(np.prod(scores[b, :i + 1].astype(np.float64))) for i in range(k[b])] for b in range(B)]
    best = None
    for choice in itertools.product(*[range(kb + 1) for kb in k]):  # kept prefix per request
        j = sum(choice)
        total = B + sum(sum(surv[b][:choice[b]]) for b in range(B))
        r = total / (float(draft[j]) + float(verify[j]))
        if best is None or r > best[0] + 1e-12:
            best = (r, j, choice)
    return best


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_over_prefix_choices(seed):
    # any prefix-closed choice of j drafts estimates at most the sum of the j
    # largest survivals, so the best choice overall is the oracle's
    g = np.random.default_rng(seed)
    B, max_k = int(g.integers(1, 4)), int(g.integers(1, 4))
    scores = g.uniform(0.05, 1.0, (B, max_k)).astype(np.float32)
    num_draft = g.integers(0, max_k + 1, B).astype(np.int32)
    n = int(num_draft.sum())
    draft = np.sort(g.uniform(0, 3, n + 1)).astype(np.float32)
    verify = (5 + np.sort(g.uniform(0, 3, n + 1))).astype(np.float32)
    budget, kept, ratios = ob.global_budget(scores, num_draft, draft, verify)
    r, j, choice = _brute(scores, num_draft, draft, verify)
    assert ratios[budget] == pytest.approx(r, rel=1e-6)
    if abs(np.sort(ratios)[-1] - np.sort(ratios)[-2] if len(ratios) > 1 else 1.0) > 1e-6:
        assert budget == j
        assert kept.tolist() == list(choice)


@pytest.mark.parametrize("seed", range(6))
def test_kept_drafts_are_the_top_survivals(seed):
    g = np.random.default_rng(100 + seed)
    B, max_k = 40, 6
    scores = g.uniform(0.2, 1.0, (B, max_k)).astype(np.float32)
    num_draft = g.integers(0, max_k + 1, B).astype(np.int32)
    n = int(num_draft.sum())
    draft = np.linspace(0, 0.2 * n, n + 1).astype(np.float32)
    verify = (20 + np.linspace(0, 0.05 * n, n + 1)).astype(np.float32)
    budget, kept, _ = ob.global_budget(scores, num_draft, draft, verify)
    surv = ob.survivals(scores, num_draft)
    assert int(kept.sum()) == budget
    assert np.all(kept <= np.clip(num_draft, 0, max_k))
    win = np.concatenate([surv[b, :kept[b]] for b in range(B)])
    lose = np.concatenate([surv[b, kept[b]:num_draft[b]] for b in range(B)])
    if len(win) and len(lose):
        assert win.min() >= lose.max()


def test_survivals_match_the_threshold_prune():
    # the same running product as the survival prune of [AV] "Other features considered"
    g = np.random.default_rng(5)
    scores = g.uniform(0.3, 1.0, (7, 5)).astype(np.float32)
    num_draft = np.array([5, 4, 0, 5, 2, 3, 1], np.int32)
    surv = ob.survivals(scores, num_draft)
    for b in range(7):
        ref, _ = oav.survival_and_kept(scores[b, :num_draft[b]], 0.0)
        np.testing.assert_allclose(surv[b, :num_draft[b]], ref, rtol=1e-6)
        assert np.all(surv[b, num_draft[b]:] == 0)


def test_ties_rank_by_flat_index_and_keep_prefixes():
    # score 1.0 everywhere: every survival is 1, the ranking is the flat order
    B, max_k = 3, 3
    scores = np.ones((B, max_k), np.float32)
    num_draft = np.array([3, 2, 3], np.int32)
    # cost rises by 0.3 per draft from 10: (3 + j) / (10 + 0.3 j) peaks at j = n
    n = 8
    draft = (0.3 * np.arange(n + 1)).astype(np.float32)
    verify = np.full(n + 1, 10.0, np.float32)
    budget, kept, _ = ob.global_budget(scores, num_draft, draft, verify)
    assert budget == 8 and kept.tolist() == [3, 2, 3]
    # a cost table that makes j = 4 best: the first four in flat order
    verify = np.array([10, 10, 10, 10, 10, 40, 40, 40, 40], np.float32)
    budget, kept, _ = ob.global_budget(scores, num_draft, draft, verify)
    assert budget == 4 and kept.tolist() == [3, 1, 0]


def test_cost_scale_invariance_and_no_drafts():
    g = np.random.default_rng(9)
    scores = g.uniform(0.1, 1.0, (10, 4)).astype(np.float32)
    num_draft = g.integers(0, 5, 10).astype(np.int32)
    n = int(num_draft.sum())
    draft = np.linspace(0, 4, n + 1).astype(np.float32)
    verify = np.linspace(8, 12, n + 1).astype(np.float32)
    b1, k1, _ = ob.global_budget(scores, num_draft, draft, verify)
    b2, k2, _ = ob.global_budget(scores, num_draft, 4 * draft, 4 * verify)
    assert b1 == b2 and k1.tolist() == k2.tolist()
    b0, k0, r0 = ob.global_budget(scores[:, :0], np.zeros(10, np.int32), draft[:1], verify[:1])
    assert b0 == 0 and k0.tolist() == [0] * 10 and len(r0) == 1


def test_equal_ratios_take_the_smallest_budget():
    # estimated tokens 2, 2.5, 3 over costs 4, 10, 6: j = 0 and j = 2 tie at exactly 0.5
    scores = np.array([[0.5], [0.5]], np.float32)
    budget, kept, ratios = ob.global_budget(scores, np.array([1, 1], np.int32), np.zeros(3, np.float32),
                                            np.array([4, 10, 6], np.float32))
    assert ratios[0] == ratios[2] == 0.5
    assert budget == 0 and kept.tolist() == [0, 0]
