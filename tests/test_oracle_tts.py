"""Pins of the TTS distillation oracle (page "ملخص تقني: التخمين في وقت
الاختبار (TTS)", section "Algorithm", step 3): finite differences of the loss,
library KL, closed forms and invariants."""
import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy

from oracle import tts as ot


@pytest.mark.parametrize("seed,T,lam,prev", [(0, 1.0, 0.0, False), (1, 0.7, 0.3, True), (2, 1.3, 1.0, True),
                                               (3, 1.0, 0.5, False)])
def test_gradient_is_the_derivative_of_the_loss(seed, T, lam, prev):
    g = np.random.default_rng(seed)
    V = 12
    zd, zt = g.normal(0, 2, V), g.normal(0, 2, V)
    zp = g.normal(0, 2, V) if prev else None
    w = 0.8
    grad, _ = ot.position(zd, zt, zp, T, w, lam)
    h = 1e-6
    for v in range(V):
        e = np.zeros(V)
        e[v] = h
        # the loss as a function of the trained draft logits; q_t stays the
        # canvas drafter's distribution (the draft rows themselves when no
        # separate rows are given)
        zp_fixed = zd if zp is None else zp
        lp = ot.position(zd + e, zt, zp_fixed, T, w, lam)[1]
        lm = ot.position(zd - e, zt, zp_fixed, T, w, lam)[1]
        assert grad[v] == pytest.approx((lp - lm) / (2 * h), abs=1e-7)


@pytest.mark.parametrize("seed", range(3))
def test_loss_is_the_library_kl(seed):
    g = np.random.default_rng(10 + seed)
    zd, zt, zp = g.normal(0, 3, (3, 50))
    T, lam, w = 0.9, 0.4, 1.7
    p, q, qt = softmax(zt / T), softmax(zd / T), softmax(zp / T)
    _, loss = ot.position(zd, zt, zp, T, w, lam)
    assert loss == pytest.approx(w * (entropy(p, q) + lam * entropy(qt, q)), rel=1e-10)


def test_identical_rows_give_nothing_and_gradients_sum_to_zero():
    g = np.random.default_rng(4)
    z = g.normal(0, 2, 30)
    grad, loss = ot.position(z, z, None, 1.0, 1.0, 0.7)
    assert loss == pytest.approx(0.0, abs=1e-15) and np.abs(grad).max() < 1e-15
    zt, zp = g.normal(0, 2, (2, 30))
    grad, _ = ot.position(z, zt, zp, 0.8, 0.6, 0.9)
    assert abs(grad.sum()) < 1e-14
    # the regulariser vanishes at the canvas drafter's own distribution
    g1, l1 = ot.position(z, zt, None, 0.8, 0.6, 0.9)
    g0, l0 = ot.position(z, zt, None, 0.8, 0.6, 0.0)
    np.testing.assert_allclose(g1, g0, atol=1e-15)
    assert l1 == pytest.approx(l0, abs=1e-15)


def test_closed_form_two_tokens_and_greedy_temperature():
    # q = (1/2, 1/2), p = (1, 0) in the limit: gradient (q - p) = (-1/2, 1/2), w = 2, T = 1
    grad, loss = ot.position(np.zeros(2), np.array([0.0, -np.inf]), None, 1.0, 2.0, 0.0)
    np.testing.assert_allclose(grad, [-1.0, 1.0])
    assert loss == pytest.approx(2 * np.log(2))
    # T = 0 counts as T = 1
    g0, l0 = ot.position(np.array([1.0, 0.0]), np.array([0.0, 1.0]), None, 0.0, 1.0, 0.0)
    g1, l1 = ot.position(np.array([1.0, 0.0]), np.array([0.0, 1.0]), None, 1.0, 1.0, 0.0)
    np.testing.assert_array_equal(g0, g1)
    assert l0 == l1
