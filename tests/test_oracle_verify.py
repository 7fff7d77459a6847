"""Pins of the verification oracle against what the pages and the mathematics
fix: library routines, the footnote's worked example, exact enumeration of the
output distribution at tiny vocabularies, the tokens-per-verify closed form,
chi-square tests at the demo's sizes, and degenerate cases."""
import itertools
from collections import defaultdict

import numpy as np
import pytest
import scipy.special as sp
import scipy.stats as st

from oracle import verify as ov
from synth import gen


# ---------------------------------------------------------------------------
# helpers (independent of the oracle: scipy softmax for interval edges)
# ---------------------------------------------------------------------------

def enumerate_outputs(zd, zt, T=1.0):
    """Exact distribution of emitted sequences, obtained by calling the
    oracle once per (draft tuple, accept/reject interval of each uniform,
    CDF interval of the sampled token) at the interval's midpoint and
    weighting by the interval's length.  Interval edges come from scipy."""
    K, V = zd.shape
    pd = [sp.softmax(zd[i] / T) for i in range(K)]
    pt = [sp.softmax(zt[j] / T) for j in range(K + 1)]
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
                res = ov.verify_request(zd, zt, d, T, u, mid if j < K else 0.5, mid if j == K else 0.5)
                dist[tuple(int(t) for t in res.tokens)] += w * cand[v]
    return dist, pd, pt


def prefix_prob(dist, prefix):
    n = len(prefix)
    return sum(p for seq, p in dist.items() if len(seq) >= n and seq[:n] == tuple(prefix))


# ---------------------------------------------------------------------------
# a1: softmax against a library routine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_log_softmax_matches_logsumexp(T):
    rng = np.random.default_rng(0)
    z = rng.normal(0, 3, 1000)
    z[[3, 77]] = -np.inf
    got = ov.log_softmax(z, T)
    want = z / T - sp.logsumexp(z / T)
    fin = np.isfinite(z)
    assert np.allclose(got[fin], want[fin], rtol=0, atol=1e-12)
    assert np.all(got[~fin] == -np.inf)
    assert abs(np.exp(got).sum() - 1.0) < 1e-12


def test_decode_bf16_bits():
    bits = np.array([0x3F80, 0xC000, 0xFF80, 0x3F81, 0x0000, 0x7F7F], dtype=np.uint16)
    got = ov.decode_rows(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == -np.inf
    assert got[3] == 1.0 + 2.0 ** -7 and got[4] == 0.0
    assert got[5] == float(np.float32(3.3895313892515355e38))


# ---------------------------------------------------------------------------
# sampler
# ---------------------------------------------------------------------------

def test_inverse_cdf_edges():
    w = np.array([0.0, 1.0, 0.0, 3.0])
    assert ov.inverse_cdf(w, 0.0)[0] == 1  # never a zero-mass token
    assert ov.inverse_cdf(w, 0.2499)[0] == 1
    assert ov.inverse_cdf(w, 0.25)[0] == 3  # C(v) > u*Z is strict
    assert ov.inverse_cdf(w, 0.999999)[0] == 3
    tok, margin = ov.inverse_cdf(w, 0.125)
    assert tok == 1 and abs(margin - 0.125) < 1e-15
    # against a library routine on random weights
    rng = np.random.default_rng(1)
    for _ in range(200):
        w = rng.exponential(size=50) * (rng.random(50) < 0.7)
        if w.sum() == 0:
            continue
        u = rng.random()
        want = int(np.searchsorted(np.cumsum(w) / np.cumsum(w)[-1], u, side="right"))
        assert ov.inverse_cdf(w, u)[0] == want


def test_accept_decision_rule():
    # strict '<', ratio +inf when the draft probability is 0
    ok, ratio, m = ov.accept_decision(np.log(0.8), np.log(0.5), 0.625 - 1e-9)
    assert ok and abs(ratio - 0.625) < 1e-15 and m < 2e-9
    assert not ov.accept_decision(np.log(0.8), np.log(0.5), 0.625 + 1e-9)[0]
    ok, ratio, _ = ov.accept_decision(-np.inf, np.log(0.3), 0.99)
    assert ok and ratio == np.inf
    assert ov.accept_decision(np.log(0.1), np.log(0.4), 0.999999)[0]  # ratio >= 1 always accepts


# ---------------------------------------------------------------------------
# footnote 1 worked example (golden)
# ---------------------------------------------------------------------------

def test_footnote_two_token_example(golden):
    g = golden("footnote_two_token.txt")
    pd_, pt_ = np.array(g["draft"]), np.array(g["target"])
    zd, zt = np.log(pd_)[None, :], np.log(np.vstack([pt_, pt_]))
    # acceptance probability of token b: the oracle's ratio
    res = ov.verify_request(zd, zt, [1], 1.0, [0.0], 0.5, 0.5)
    ratio = res.p_target[0] / res.p_draft[0]
    assert abs(ratio - g["accept_prob_b"]) < 1e-12
    assert ov.verify_request(zd, zt, [1], 1.0, [g["accept_prob_b"] - 1e-9], 0.5, 0.5).accept_len == 1
    assert ov.verify_request(zd, zt, [1], 1.0, [g["accept_prob_b"] + 1e-9], 0.5, 0.5).accept_len == 0
    # the residual is [1, 0]: every rejected b resamples a
    for u in np.linspace(0, 0.999, 17):
        assert list(ov.verify_request(zd, zt, [1], 1.0, [0.9], u, 0.5).tokens) == [0]
    # lossless: untrimmed slot-0 output equals the target
    dist, _, _ = enumerate_outputs(zd, zt)
    out = np.array([prefix_prob(dist, [0]), prefix_prob(dist, [1])])
    assert np.allclose(out, g["lossless_output"], atol=1e-12)
    # trimmed variant: a draft whose own probability is below trim_below skips verification
    # and the target samples its own distribution; otherwise the oracle verifies it.  The
    # uniform grid integrates the oracle's decision exactly for the page's probabilities.
    grid = (np.arange(1000) + 0.5) / 1000
    trimmed = np.zeros(2)
    for d in (0, 1):
        if pd_[d] < g["trim_below"]:
            trimmed += pd_[d] * pt_
            continue
        for u in grid:
            tok = ov.verify_request(zd, zt, [d], 1.0, [u], 0.5, 0.5).tokens[0]
            trimmed[tok] += pd_[d] / len(grid)
    assert np.allclose(trimmed, g["trimmed_output"], atol=1e-12)


# ---------------------------------------------------------------------------
# brute force: losslessness identity at V <= 8
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,K,T,seed", [(6, 3, 1.0, 0), (8, 2, 0.7, 1), (5, 3, 1.3, 2), (4, 1, 1.0, 3)])
def test_bruteforce_lossless(V, K, T, seed):
    rng = np.random.default_rng(seed)
    zd = rng.normal(0, 1.5, (K, V))
    zt = rng.normal(0, 1.5, (K + 1, V))
    zd[0, 1] = -np.inf  # a zero-probability draft token
    zt[min(1, K), 2] = -np.inf  # a zero-probability target token
    dist, pd, pt = enumerate_outputs(zd, zt, T)
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    for j in range(K + 1):
        for prefix in itertools.product(range(V), repeat=j + 1):
            want = float(np.prod([min(pd[i][prefix[i]], pt[i][prefix[i]]) for i in range(j)])) * pt[j][prefix[j]]
            assert abs(prefix_prob(dist, prefix) - want) < 1e-12, (j, prefix)


def test_bruteforce_catches_a_swapped_residual():
    """The identity above has power: the same enumeration over a deliberately
    wrong sampler (residual (pd - pt)+) breaks it."""
    V, K = 5, 1
    rng = np.random.default_rng(4)
    zd, zt = rng.normal(0, 1.5, (K, V)), rng.normal(0, 1.5, (K + 1, V))
    pd, pt = sp.softmax(zd[0]), sp.softmax(zt[0])
    out = np.zeros(V)
    for d in range(V):
        acc = min(1.0, pt[d] / pd[d])
        out[d] += pd[d] * acc
        wrong = np.maximum(0, pd - pt)
        out += pd[d] * (1 - acc) * wrong / wrong.sum()
    assert np.abs(out - pt).max() > 1e-3


# ---------------------------------------------------------------------------
# closed form: tokens per verify on a constant-alpha source (golden 3.36)
# ---------------------------------------------------------------------------

def test_tokens_per_verify_closed_form_exact(golden):
    g = golden("tokens_per_verify.txt")
    alpha, K = g["alpha"], int(g["K"])
    pd, pt = gen.constant_alpha_rows(alpha, V=4, K=K, seed=7)
    dist, _, _ = enumerate_outputs(np.log(pd), np.log(pt))
    mean_len = sum(len(s) * p for s, p in dist.items())
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    assert abs(mean_len - closed) < 1e-12
    assert round(mean_len, int(g["printed_decimals"])) == g["tokens_per_verify"]
    for j in range(K + 1):
        pj = sum(p for s, p in dist.items() if len(s) == j + 1)
        want = alpha ** j * (1 - alpha) if j < K else alpha ** K
        assert abs(pj - want) < 1e-12


@pytest.mark.parametrize("alpha_key", ["alpha", "golden08"])
def test_tokens_per_verify_monte_carlo(golden, alpha_key):
    """Monte Carlo at the demo's default sizes (vocab, k, samples, seed)."""
    d = golden("script_defaults.txt")
    alpha = d["alpha"] if alpha_key == "alpha" else golden("tokens_per_verify.txt")["alpha"]
    V, K, M = int(d["vocab"]), int(d["k"]), int(d["samples"])
    pd, pt = gen.constant_alpha_rows(alpha, V=V, K=K, seed=int(d["seed"]))
    b = gen.broadcast_batch(np.log(pd).astype(np.float32), np.log(pt).astype(np.float32), M,
                            seed=int(d["seed"]), draft_probs=pd)
    zd, zt = np.log(pd), np.log(pt)
    lens = np.empty(M)
    for t in range(M):
        r = ov.verify_request(zd, zt, b.draft_tokens[t], 1.0, b.u_accept[t], b.u_residual[t], b.u_bonus[t])
        lens[t] = r.accept_len + 1
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    se = lens.std(ddof=1) / np.sqrt(M)
    assert abs(lens.mean() - closed) < 4 * se


# ---------------------------------------------------------------------------
# chi-square of emitted tokens against the target (functions table: chi_square)
# ---------------------------------------------------------------------------

def chi_square_p(observed, expected_probs, min_expected=5.0):
    """Pearson chi-square p-value, merging cells with expected count < 5."""
    observed = np.asarray(observed, dtype=np.float64)
    n = observed.sum()
    exp = np.asarray(expected_probs) * n
    order = np.argsort(exp)
    o_m, e_m, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += observed[i]
        acc_e += exp[i]
        if acc_e >= min_expected:
            o_m.append(acc_o)
            e_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        o_m[-1] += acc_o
        e_m[-1] += acc_e
    return st.chisquare(o_m, e_m).pvalue


def test_chi_square_slots_match_target(golden):
    d = golden("script_defaults.txt")
    V, K, M, seed = int(d["vocab"]), int(d["k"]), int(d["samples"]), int(d["seed"])
    rng = np.random.default_rng(seed)
    zd = (3.0 * rng.standard_normal((K, V))).astype(np.float32)
    zt = (np.vstack([zd, 3.0 * rng.standard_normal((1, V))]) + rng.standard_normal((K + 1, V))).astype(np.float32)
    b = gen.broadcast_batch(zd, zt, M, seed=seed)
    counts = np.zeros((K + 1, V))
    for t in range(M):
        r = ov.verify_request(zd.astype(np.float64), zt.astype(np.float64), b.draft_tokens[t], 1.0,
                              b.u_accept[t], b.u_residual[t], b.u_bonus[t])
        for j, tok in enumerate(r.tokens):
            counts[j, tok] += 1
    for j in range(K + 1):
        if counts[j].sum() < 200:
            continue
        p = chi_square_p(counts[j], sp.softmax(zt[j].astype(np.float64)))
        assert p > 1e-4, (j, p)


def test_chi_square_rejects_trimmed_variant(golden):
    """Negative control from footnote 1: trimming on the sampled draft's own
    probability biases the output, and the chi-square check detects it."""
    g = golden("footnote_two_token.txt")
    pd_, pt_ = np.array(g["draft"]), np.array(g["target"])
    zd, zt = np.log(pd_)[None, :], np.log(np.vstack([pt_, pt_]))
    rng = np.random.default_rng(0)
    counts = np.zeros(2)
    for _ in range(20000):
        dtok = int(rng.random() < pd_[1])
        if pd_[dtok] < g["trim_below"]:
            counts[int(rng.random() < pt_[1])] += 1
        else:
            r = ov.verify_request(zd, zt, [dtok], 1.0, [rng.random()], rng.random(), rng.random())
            counts[r.tokens[0]] += 1
    assert chi_square_p(counts, pt_) < 1e-4
    assert np.allclose(counts / counts.sum(), g["trimmed_output"], atol=0.015)


# ---------------------------------------------------------------------------
# degenerate cases
# ---------------------------------------------------------------------------

def test_identical_rows_accept_everything():
    rng = np.random.default_rng(5)
    K, V = 4, 50
    z = rng.normal(0, 2, (K + 1, V))
    for t in range(50):
        d = rng.integers(0, V, K)
        r = ov.verify_request(z[:K], z, d, 1.0, rng.random(K), rng.random(), rng.random())
        assert r.accept_len == K and list(r.labels) == [1] * K
        assert list(r.tokens[:K]) == list(d)


def test_disjoint_supports_reject_first_and_sample_target():
    rng = np.random.default_rng(6)
    K, V = 3, 40
    zd = rng.normal(0, 1, (K, V))
    zd[:, V // 2:] = -np.inf
    zt = rng.normal(0, 1, (K + 1, V))
    zt[:, :V // 2] = -np.inf
    for t in range(50):
        d = rng.integers(0, V // 2, K)
        u_res = rng.random()
        r = ov.verify_request(zd, zt, d, 1.0, rng.random(K), u_res, rng.random())
        assert r.accept_len == 0 and list(r.labels) == [0, -1, -1]
        want = int(np.searchsorted(np.cumsum(sp.softmax(zt[0])), u_res, side="right"))
        assert r.tokens[0] == want and r.tokens[0] >= V // 2


def test_greedy_is_the_zero_temperature_limit():
    rng = np.random.default_rng(8)
    K, V = 3, 16
    for t in range(100):
        zd = np.vstack([rng.permutation(V) * 0.5 for _ in range(K)])
        zt = np.vstack([rng.permutation(V) * 0.5 for _ in range(K + 1)])
        if t % 3 == 0:
            zt[0] = zd[0]  # force some acceptances
        d = [int(np.argmax(zd[i])) for i in range(K)]
        u = rng.uniform(1e-3, 1 - 1e-3, K)
        g = ov.verify_request(zd, zt, d, 0.0, u, 0.5, 0.5)
        s = ov.verify_request(zd, zt, d, 1e-3, u, rng.uniform(1e-3, 1 - 1e-3), rng.uniform(1e-3, 1 - 1e-3))
        assert g.accept_len == s.accept_len and list(g.tokens) == list(s.tokens)
        assert list(g.labels) == list(s.labels)


def test_zero_drafts_draws_the_bonus_from_row_zero():
    rng = np.random.default_rng(9)
    zt = rng.normal(0, 1, (1, 30))
    u = 0.37
    r = ov.verify_request(np.zeros((0, 30)), zt, [], 1.0, [], 0.9, u)
    want = int(np.searchsorted(np.cumsum(sp.softmax(zt[0])), u, side="right"))
    assert r.accept_len == 0 and list(r.tokens) == [want]


def test_batch_driver_matches_single_requests():
    b = gen.make_batch("tiny_fp32_b4_k4_v1024")
    out = ov.verify_batch(b)
    for r in range(b.B):
        k = b.num_draft[r]
        zd = b.draft[b.draft_row_start[r]:b.draft_row_start[r] + k].astype(np.float64)
        zt = b.target[b.target_row_start[r]:b.target_row_start[r] + k + 1].astype(np.float64)
        res = ov.verify_request(zd, zt, b.draft_tokens[r, :k], 1.0, b.u_accept[r], b.u_residual[r], b.u_bonus[r])
        assert out["accept_len"][r] == res.accept_len
        assert list(out["out_tokens"][r, :res.accept_len + 1]) == list(res.tokens)
        assert np.all(out["out_tokens"][r, res.accept_len + 1:] == -1)
