"""Pins of the acceptance-estimator oracle: the feature against scipy's
softmax/logit, closed forms, the "no fit" identity (omega=1, beta=0 gives
q_max), finite differences of the log-likelihood, the textbook IRLS step,
convergence to the maximum-likelihood estimate and planted-parameter
recovery."""
import numpy as np
import pytest
import scipy.optimize as so
import scipy.special as sp

from oracle import av
from synth import gen


# ---------------------------------------------------------------------------
# feature and score
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 0.7])
def test_feature_is_logit_of_qmax(T):
    rng = np.random.default_rng(0)
    for _ in range(20):
        z = rng.normal(0, 3, 1000)
        want = sp.logit(sp.softmax(z / T).max())
        assert abs(av.feature(z, T) - want) < 1e-9 * max(1.0, abs(want))


def test_feature_closed_forms():
    # two tokens with the footnote's draft [0.2, 0.8]: logit(0.8) = ln 4
    assert abs(av.feature(np.log([0.2, 0.8]), 1.0) - np.log(4.0)) < 1e-14
    # uniform row: q_max = 1/V, logit = -ln(V - 1)
    V = 128256
    assert abs(av.feature(np.zeros(V), 1.0) + np.log(V - 1)) < 1e-12
    # tied maxima: q_max is the same whichever index wins
    z = np.array([1.0, 3.0, 3.0, 0.0])
    want = sp.logit(sp.softmax(z).max())
    assert abs(av.feature(z, 1.0) - want) < 1e-14
    # all other tokens impossible: clamped
    assert av.feature(np.array([-np.inf, 2.0, -np.inf]), 1.0) == av.FEATURE_CLAMP


def test_score_and_no_fit_identity():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 3, 500)
    x = av.feature(z, 1.0)
    # omega = 1, beta = 0: the score is the draft's top-token probability itself
    assert abs(av.score(x, [1.0, 0.0], 0) - sp.softmax(z).max()) < 1e-12
    for omega, beta in [(1.2, 0.5), (0.5, -3.0), (-2.0, 40.0), (3.0, -800.0)]:
        assert abs(av.score(x, [omega, 0.0, beta], 1) - sp.expit(omega * x + beta)) < 1e-15


def test_survival_and_prune():
    surv, kept = av.survival_and_kept([0.9, 0.5, 0.8], 0.3)
    assert np.allclose(surv, [0.9, 0.45, 0.36]) and kept == 3
    assert av.survival_and_kept([0.9, 0.5, 0.8], 0.4)[1] == 2
    assert av.survival_and_kept([0.2, 0.9], 0.3)[1] == 0
    assert av.survival_and_kept([0.2, 0.9], 0.0)[1] == 2


def test_av_score_batch_config_identity():
    b = gen.make_batch("tiny_fp32_b4_k4_v1024")
    out = av.av_score_batch(b)
    for r in range(b.B):
        for i in range(b.max_k):
            z = b.draft[b.draft_row_start[r] + i].astype(np.float64)
            assert abs(out["score"][r, i] - sp.softmax(z).max()) < 1e-12


# ---------------------------------------------------------------------------
# fitting
# ---------------------------------------------------------------------------

def _synthetic_labels(rng, B, K, omega, beta, censor=True):
    x = rng.normal(1.0, 1.5, (B, K)).astype(np.float32)
    p = sp.expit(omega * x.astype(np.float64) + np.asarray(beta)[None, :])
    y = (rng.random((B, K)) < p).astype(np.int8)
    if censor:  # only drafts up to the first rejection carry labels
        lab = np.full((B, K), -1, np.int8)
        for b in range(B):
            for i in range(K):
                lab[b, i] = y[b, i]
                if y[b, i] == 0:
                    break
        return x, lab
    return x, y


def test_sums_match_finite_differences():
    rng = np.random.default_rng(2)
    K = 4
    x, lab = _synthetic_labels(rng, 300, K, 0.8, [0.5, 0.2, -0.1, -0.4])
    theta = np.array([0.7, 0.4, 0.1, 0.0, -0.3], dtype=np.float32).astype(np.float64)
    H, g = av.hessian_gradient(av.fit_sums(x, lab, theta))
    f = lambda t: av.nll(x, lab, t)
    h = 1e-5
    E = np.eye(K + 1)
    g_fd = np.array([(f(theta + h * E[k]) - f(theta - h * E[k])) / (2 * h) for k in range(K + 1)])
    assert np.allclose(g, g_fd, rtol=1e-6, atol=1e-6)
    h = 1e-3
    H_fd = np.array([[(f(theta + h * (E[k] + E[l])) - f(theta + h * (E[k] - E[l]))
                       - f(theta - h * (E[k] - E[l])) + f(theta - h * (E[k] + E[l]))) / (4 * h * h)
                      for l in range(K + 1)] for k in range(K + 1)])
    assert np.allclose(H, H_fd, rtol=1e-4, atol=1e-3)
    # the Hessian is an arrowhead: intercepts do not couple with each other
    assert np.all(H[1:, 1:][~np.eye(K, dtype=bool)] == 0.0)


def test_undamped_step_is_the_textbook_irls_step():
    rng = np.random.default_rng(3)
    K = 3
    x, lab = _synthetic_labels(rng, 400, K, 1.1, [0.3, -0.2, -0.6])
    theta = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float32)
    new = av.newton_step(av.fit_sums(x, lab, theta), theta, damping_c=0.0, ridge=0.0, max_step=np.inf)
    # design matrix [x, onehot(position)] over labelled drafts
    rows, ys = [], []
    for b in range(x.shape[0]):
        for i in range(K):
            if lab[b, i] in (0, 1):
                rows.append([float(x[b, i])] + [1.0 if j == i else 0.0 for j in range(K)])
                ys.append(float(lab[b, i]))
    X, y = np.array(rows), np.array(ys)
    pi = sp.expit(X @ theta.astype(np.float64))
    W = pi * (1 - pi)
    step = np.linalg.solve(X.T @ (W[:, None] * X), X.T @ (y - pi))
    assert np.allclose(new - theta, step, rtol=1e-10, atol=1e-12)


def test_iterated_steps_reach_the_mle():
    rng = np.random.default_rng(4)
    K = 4
    x, lab = _synthetic_labels(rng, 600, K, 0.55, [0.6, 0.2, -0.2, -0.5])
    params = np.array([1.0, 0, 0, 0, 0], dtype=np.float32)
    accum = np.zeros((K, 6))
    for _ in range(30):
        params, accum = av.fit_step(x, lab, params, accum, damping_c=0.0, ridge=0.0, do_update=True)
    ref = so.minimize(lambda t: av.nll(x, lab, t), np.zeros(K + 1), method="BFGS",
                      options={"gtol": 1e-9}).x
    assert np.allclose(params, ref, rtol=1e-4, atol=1e-4)
    # at the MLE the damped step barely moves: damping does not shift the fixed point
    again = av.newton_step(av.fit_sums(x, lab, params), params, damping_c=10.0, ridge=1e-6)
    assert np.abs(again - params).max() < 1e-5


def test_planted_parameters_are_recovered():
    """Config-2 planted values omega = 1.2, beta_i = 0.5 - 0.3 i."""
    rng = np.random.default_rng(5)
    K = 5
    omega, beta = 1.2, [0.5 - 0.3 * i for i in range(K)]
    x, lab = _synthetic_labels(rng, 8000, K, omega, beta)
    params = np.array([1.0] + [0.0] * K, dtype=np.float32)
    accum = np.zeros((K, 6))
    for _ in range(25):
        params, accum = av.fit_step(x, lab, params, accum, damping_c=10.0, ridge=1e-6, do_update=True)
    H, _ = av.hessian_gradient(av.fit_sums(x, lab, params))
    sd = np.sqrt(np.diag(np.linalg.inv(H)))
    assert np.all(np.abs(params - np.array([omega] + beta)) < 4 * sd), (params, sd)


def test_round_accumulation_equals_one_big_batch():
    rng = np.random.default_rng(6)
    K = 3
    parts = [_synthetic_labels(rng, 100, K, 0.9, [0.4, 0.0, -0.4]) for _ in range(3)]
    params = np.array([1.0, 0.1, 0.0, -0.1], dtype=np.float32)
    accum = np.zeros((K, 6))
    for j, (x, lab) in enumerate(parts):
        params_out, accum = av.fit_step(x, lab, params, accum, do_update=(j == 2))
        if j < 2:
            assert np.all(params_out == params)
    X = np.vstack([p[0] for p in parts])
    L = np.vstack([p[1] for p in parts])
    big, acc2 = av.fit_step(X, L, params, np.zeros((K, 6)), do_update=True)
    assert np.allclose(params_out, big, rtol=1e-6, atol=1e-7)
    assert np.all(accum == 0) and np.all(acc2 == 0)


def test_positions_without_labels_keep_their_intercept():
    rng = np.random.default_rng(7)
    K = 4
    x, lab = _synthetic_labels(rng, 200, K, 0.9, [0.4, 0.0, -0.4, -0.8])
    lab[:, 2] = -1
    params = np.array([1.0, 0.1, 0.2, 0.3, 0.4], dtype=np.float32)
    new = av.newton_step(av.fit_sums(x, lab, params), params, 10.0, 1e-6)
    assert new[3] == np.float64(np.float32(0.3))
    assert np.all(new[[0, 1, 2, 4]] != params[[0, 1, 2, 4]])
    # no labels at all: nothing moves
    none = np.full_like(lab, -1)
    assert np.all(av.newton_step(av.fit_sums(x, none, params), params, 10.0, 1e-6) == params.astype(np.float64))


def test_damping_scales_each_coefficient_by_its_evidence():
    rng = np.random.default_rng(8)
    K = 3
    x, lab = _synthetic_labels(rng, 300, K, 0.9, [0.4, 0.0, -0.4])
    params = np.array([0.5, 0.0, 0.0, 0.0], dtype=np.float32)
    sums = av.fit_sums(x, lab, params)
    raw = av.newton_step(sums, params, 0.0, 1e-6, max_step=np.inf) - params
    c = 25.0
    damped = av.newton_step(sums, params, c, 1e-6, max_step=np.inf) - params
    n = sums[:, 0]
    scale = np.concatenate([[n.sum() / (n.sum() + c)], n / (n + c)])
    assert np.allclose(damped, raw * scale, rtol=1e-12, atol=1e-15)


def test_step_bound_keeps_the_newton_direction():
    """A damped step larger than the bound is scaled as a whole: same
    direction, largest component equal to the bound; smaller steps pass."""
    rng = np.random.default_rng(9)
    K = 3
    x, lab = _synthetic_labels(rng, 300, K, 0.9, [2.0, 1.0, -1.0])
    params = np.array([-1.0, -3.0, 2.0, 1.0], dtype=np.float32)  # far from the optimum
    sums = av.fit_sums(x, lab, params)
    free = av.newton_step(sums, params, 10.0, 1e-6, max_step=np.inf) - params
    assert np.abs(free).max() > 0.5
    for bound in (0.5 * np.abs(free).max(), 0.1):
        got = av.newton_step(sums, params, 10.0, 1e-6, max_step=bound) - params
        assert np.abs(got).max() == pytest.approx(bound, rel=1e-12)
        ratio = got / free
        assert np.allclose(ratio, ratio[0], rtol=1e-12)
    wide = av.newton_step(sums, params, 10.0, 1e-6, max_step=2.0 * np.abs(free).max()) - params
    assert np.array_equal(wide, free)


def test_separable_position_moves_by_the_bound():
    """Every draft at position 0 rejected, features all 0: the log-likelihood
    has no finite optimum in beta_0.  At beta_0 = 0, pi = 1/2, so g = n/2 and
    H = n/4 (+ ridge): the Newton step is -2 before damping, -2 n/(n+c)
    after it, and the bound cuts it to exactly -max_step."""
    n, c = 100, 10.0
    x = np.zeros((n, 1), np.float32)
    lab = np.zeros((n, 1), np.int8)
    params = np.array([0.5, 0.0], dtype=np.float32)
    sums = av.fit_sums(x, lab, params)
    free = av.newton_step(sums, params, c, 1e-6, max_step=np.inf)
    assert free[1] == pytest.approx(-2.0 * n / (n + c), rel=1e-6)
    assert free[0] == pytest.approx(0.5, abs=1e-12)  # the slope sees no spread in x
    bounded = av.newton_step(sums, params, c, 1e-6, max_step=1.0)
    assert bounded[1] == pytest.approx(-1.0, rel=1e-12)


def test_refit_on_the_benchmark_workload_stays_bounded():
    """The benchmark's loop: the peaked B=256, K=4, V=128256 batch, features
    and first-rejection labels from the oracle, a refit on every step from
    omega = 1, beta = 0.  The page's undamped-by-distance Newton step runs
    away there (features bunch near -4.8, where the sigmoid is flat, and the
    deepest positions see labels of one class only); with the step bound the
    parameters stay bounded and the log-loss falls."""
    from oracle import verify as ov
    from synth import gen

    b = gen.make_batch("bf16_b256_k4_v128256_peaked")
    x = av.av_score_batch(b)["feature"].astype(np.float32)
    lab = ov.verify_batch(b)["labels"]
    start = b.av_params.astype(np.float32)
    n = int(((lab == 0) | (lab == 1)).sum())

    def loop(max_step, steps):
        p, acc = start.copy(), np.zeros((b.max_k, 6))
        for _ in range(steps):
            p, acc = av.fit_step(x, lab, p, acc, damping_c=10.0, ridge=1e-6, do_update=True, max_step=max_step)
        return p

    free = loop(np.inf, 3)
    assert np.abs(free).max() > 1e3
    bounded = loop(1.0, 30)
    assert np.all(np.isfinite(bounded)) and np.abs(bounded).max() < 10.0
    assert av.nll(x, lab, bounded) / n < 0.75 * av.nll(x, lab, start) / n
