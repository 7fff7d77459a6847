"""Pins of the filtered-verification oracle (top-k / top-p, readings F1-F5 of
``oracle.filtered``): the filter against a brute-force pairwise count, hand-
worked nuclei, the reductions to the unfiltered and the greedy oracle, and
exact enumeration of the emitted-token distribution at tiny vocabularies
(losslessness with respect to the filtered target rows)."""
import itertools
from collections import defaultdict

import numpy as np
import pytest
import scipy.special as sp

from oracle import filtered as of
from oracle import verify as ov


def brute_keep(z, T, top_k, top_p):
    """F1-F3 token by token: pairwise comparisons, scipy softmax."""
    z = np.asarray(z, dtype=np.float64)
    p = sp.softmax(z / T)
    V = len(z)
    keep = np.ones(V, dtype=bool)
    for v in range(V):
        bigger = [w for w in range(V) if z[w] > z[v]]
        if 0 < top_k < V and not len(bigger) < top_k:
            keep[v] = False
        if top_p < 1.0 and not sum(p[w] for w in bigger) < top_p:
            keep[v] = False
    return keep


@pytest.mark.parametrize("seed", range(12))
def test_keep_mask_matches_pairwise_definition(seed):
    g = np.random.default_rng(seed)
    V = int(g.integers(2, 40))
    z = np.round(g.normal(0, 1.5, V) * 2) / 2  # a coarse grid: many ties
    if seed % 3 == 0:
        z[g.integers(0, V)] = -np.inf
    if seed % 4 == 1:
        z[z == 0.0] = -0.0  # -0 and +0 are one value
    T = [1.0, 0.7, 1.6][seed % 3]
    for top_k, top_p in [(0, 1.0), (1, 1.0), (3, 1.0), (V, 0.5), (0, 0.3), (0, 0.9), (5, 0.8), (2, 0.05)]:
        f = of.keep_mask(z, T, top_k, top_p)
        want = brute_keep(z, T, top_k, top_p)
        np.testing.assert_array_equal(f.keep, want, err_msg=f"k={top_k} p={top_p}")
        assert f.kept == int(want.sum())


def test_hand_worked_nuclei():
    # p = (0.5, 0.3, 0.2): above 0.3 lies 0.5, above 0.2 lies 0.8
    z = np.log([0.5, 0.3, 0.2])
    assert of.keep_mask(z, 1.0, 0, 0.6).keep.tolist() == [True, True, False]
    assert of.keep_mask(z, 1.0, 0, 0.5).keep.tolist() == [True, False, False]  # 0.5 is not < 0.5
    assert of.keep_mask(z, 1.0, 0, 0.81).keep.tolist() == [True, True, True]
    assert of.keep_mask(z, 1.0, 0, 0.6).margin == pytest.approx(0.1)  # 0.6 - 0.5 vs 0.8 - 0.6
    # ties at the boundary are kept together: p = (0.4, 0.3, 0.3)
    z = np.log([0.4, 0.3, 0.3])
    assert of.keep_mask(z, 1.0, 0, 0.45).keep.tolist() == [True, True, True]
    assert of.keep_mask(z, 1.0, 2, 1.0).keep.tolist() == [True, True, True]  # top-2 keeps the tie
    assert of.keep_mask(z, 1.0, 1, 1.0).keep.tolist() == [True, False, False]
    # a uniform row keeps everything for any top_p > 0
    assert of.keep_mask(np.zeros(7), 1.0, 0, 0.01).kept == 7
    # both filters: the intersection
    z = np.log([0.35, 0.25, 0.2, 0.2])
    assert of.keep_mask(z, 1.0, 3, 0.7).keep.tolist() == [True, True, True, True]  # the tie at 0.2 stays
    assert of.keep_mask(z, 1.0, 2, 0.7).keep.tolist() == [True, True, False, False]
    assert of.keep_mask(z, 1.0, 3, 0.5).keep.tolist() == [True, True, False, False]


def test_filtered_log_probs_renormalise():
    g = np.random.default_rng(3)
    z = g.normal(0, 2, 50)
    f = of.keep_mask(z, 0.8, 0, 0.9)
    lp = of.filtered_log_probs(z, 0.8, f)
    p = sp.softmax(z / 0.8)
    np.testing.assert_allclose(np.exp(lp), np.where(f.keep, p / p[f.keep].sum(), 0.0), rtol=1e-12, atol=0)
    assert np.exp(lp).sum() == pytest.approx(1.0, abs=1e-12)


def test_disabled_filters_are_the_unfiltered_oracle():
    g = np.random.default_rng(5)
    K, V = 3, 40
    zd, zt = g.normal(0, 2, (K, V)), g.normal(0, 2, (K + 1, V))
    d = g.integers(0, V, K)
    u = g.random(K)
    for top_k, top_p in [(0, 1.0), (V, 1.0), (-3, 2.0)]:
        a = of.verify_request_filtered(zd, zt, d, 1.0, top_k, top_p, u, 0.3, 0.6).result
        b = ov.verify_request(zd, zt, d, 1.0, u, 0.3, 0.6)
        assert a.accept_len == b.accept_len and a.tokens.tolist() == b.tokens.tolist()
        np.testing.assert_array_equal(a.p_target, b.p_target)


@pytest.mark.parametrize("seed", range(6))
def test_top1_verification_is_greedy_verification(seed):
    """With top_k = 1 both distributions are one-hot at the rows' argmax, so
    speculative sampling on drafts taken at the draft argmax reduces to the
    greedy rule (accept iff the draft is the target argmax; emit that argmax)."""
    g = np.random.default_rng(20 + seed)
    K, V = 4, 30
    zd, zt = g.normal(0, 2, (K, V)), g.normal(0, 2, (K + 1, V))
    zt[:K, np.argmax(zd, axis=1)[: K]] += g.choice([0.0, 9.0], K)  # some positions agree
    d = np.argmax(zd, axis=1)
    u = g.random(K)
    a = of.verify_request_filtered(zd, zt, d, 1.0, 1, 1.0, u, float(g.random()), float(g.random())).result
    b = ov.verify_request(zd, zt, d, 0.0, u, 0.5, 0.5)
    assert a.accept_len == b.accept_len and a.tokens.tolist() == b.tokens.tolist()


def enumerate_filtered(zd, zt, T, top_k, top_p):
    """Exact distribution of the emitted sequences of the filtered oracle:
    one call per (draft tuple, accept/reject interval of each uniform, CDF
    interval of the drawn token) at the interval's midpoint, weighted by its
    length.  Interval edges come from the brute-force filter and scipy."""
    K, V = zd.shape
    def filt(z):
        keep = brute_keep(z, T, top_k, top_p)
        p = np.where(keep, sp.softmax(z / T), 0.0)
        return p / p.sum()
    pd = [filt(zd[i]) for i in range(K)]
    pt = [filt(zt[j]) for j in range(K + 1)]
    dist = defaultdict(float)
    for d in itertools.product(range(V), repeat=K):
        w_d = float(np.prod([pd[i][d[i]] for i in range(K)]))
        if w_d == 0.0:
            continue
        bound = [min(1.0, pt[i][d[i]] / pd[i][d[i]]) for i in range(K)]
        for j in range(K + 1):
            w = w_d
            u = np.full(K, 0.5)
            for i in range(j):
                w *= bound[i]
                u[i] = bound[i] / 2
            if w == 0.0:
                continue
            if j < K:
                if bound[j] >= 1.0:
                    continue
                w *= 1.0 - bound[j]
                u[j] = (bound[j] + 1.0) / 2
                r = np.maximum(0.0, pt[j] - pd[j])
                cand = r / r.sum()
            else:
                cand = pt[K]
            C = np.cumsum(cand)
            for v in range(V):
                if cand[v] <= 0.0:
                    continue
                mid = ((C[v - 1] if v else 0.0) + C[v]) / 2
                res = of.verify_request_filtered(zd, zt, d, T, top_k, top_p, u, mid if j < K else 0.5,
                                                 mid if j == K else 0.5).result
                dist[tuple(int(t) for t in res.tokens)] += w * cand[v]
    return dist, pd, pt


@pytest.mark.parametrize("V,K,T,top_k,top_p,seed", [(6, 2, 1.0, 0, 0.8, 0), (7, 2, 0.8, 4, 1.0, 1),
                                                   (6, 3, 1.2, 3, 0.9, 2), (5, 1, 1.0, 0, 0.5, 3)])
def test_bruteforce_lossless_on_filtered_rows(V, K, T, top_k, top_p, seed):
    """Slot j's token, given the slot is reached with prefix y_0..y_{j-1},
    is distributed as the filtered target row p'_j: P(prefix) =
    prod_{i<j} min(pd'_i, pt'_i)(y_i) * pt'_j(y_j)."""
    g = np.random.default_rng(seed)
    zd = g.normal(0, 1.5, (K, V))
    zt = g.normal(0, 1.5, (K + 1, V))
    dist, pd, pt = enumerate_filtered(zd, zt, T, top_k, top_p)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    assert any((p == 0).any() for p in pd + pt)  # the filters bite
    for j in range(K + 1):
        for prefix in itertools.product(range(V), repeat=j + 1):
            want = float(np.prod([min(pd[i][prefix[i]], pt[i][prefix[i]]) for i in range(j)])) * pt[j][prefix[j]]
            got = sum(p for s, p in dist.items() if len(s) > j and s[:j + 1] == prefix)
            assert abs(got - want) < 1e-12, (j, prefix)


def test_filtered_rows_change_the_verdict_and_report_counts():
    # the draft token lies outside the target's nucleus: rejected, and the
    # residual draws from the target's kept set
    zd = np.log(np.array([[0.1, 0.6, 0.3]]))
    zt = np.log(np.array([[0.7, 0.05, 0.25], [0.5, 0.25, 0.25]]))
    fr = of.verify_request_filtered(zd, zt, [1], 1.0, 0, 0.85, [0.01], 0.5, 0.5)
    # pt' = (0.7, 0, 0.25) / 0.95 and pd' = (0, 0.6, 0.3) / 0.9: residual mass on token 0 only
    assert fr.result.accept_len == 0 and fr.result.tokens.tolist() == [0]
    assert fr.result.p_target[0] == 0.0
    assert fr.kept.tolist() == [2, 2, 3]
    # unfiltered the same uniform accepts (0.01 < 0.05 / 0.6)
    assert ov.verify_request(zd, zt, [1], 1.0, [0.01], 0.5, 0.5).accept_len == 1
