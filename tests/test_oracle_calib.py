"""Pins of the calibration-metric oracle ([AV] "Other features considered":
AUC, log-loss, ECE) against library routines for the same definitions,
closed forms and a direct pair count."""
import numpy as np
import pytest
from sklearn.metrics import log_loss, roc_auc_score

from oracle import calib as oc


@pytest.mark.parametrize("seed", range(5))
def test_auc_equals_the_library_on_arbitrary_scores(seed):
    g = np.random.default_rng(seed)
    p = g.random(3000).astype(np.float32)
    p[:300] = np.round(p[:300] * 20) / 20  # and some exact ties
    y = (g.random(3000) < p).astype(np.int8)
    assert oc.metrics(p, y)["auc"] == pytest.approx(roc_auc_score(y, p.astype(np.float64)), abs=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_auc_equals_a_direct_pair_count(seed):
    # P(pos > neg) + 1/2 P(pos == neg), counting every pair by brute force
    g = np.random.default_rng(10 + seed)
    p = (np.round(g.random(400) * 50) / 50).astype(np.float32)  # many ties
    y = (g.random(400) < 0.6).astype(np.int8)
    pp, pn = p[y == 1], p[y == 0]
    wins = (pp[:, None] > pn[None, :]).sum() + 0.5 * (pp[:, None] == pn[None, :]).sum()
    assert oc.metrics(p, y)["auc"] == pytest.approx(wins / (len(pp) * len(pn)), abs=1e-12)


def test_auc_tells_scores_one_float_step_apart():
    # scores that any binning of [0, 1] would merge still order the pair
    lo = np.float32(0.5)
    hi = np.nextafter(lo, np.float32(1.0))
    assert oc.metrics(np.array([hi, lo], np.float32), [1, 0])["auc"] == 1.0
    assert oc.metrics(np.array([lo, lo], np.float32), [1, 0])["auc"] == 0.5


def test_auc_separated_and_reversed():
    p = np.array([0.1, 0.2, 0.3, 0.7, 0.8, 0.9], np.float32)
    assert oc.metrics(p, [0, 0, 0, 1, 1, 1])["auc"] == 1.0
    assert oc.metrics(p, [1, 1, 1, 0, 0, 0])["auc"] == 0.0
    assert np.isnan(oc.metrics(p, [1] * 6)["auc"])


@pytest.mark.parametrize("seed", range(3))
def test_log_loss_equals_the_library(seed):
    g = np.random.default_rng(20 + seed)
    p = g.random(2000).astype(np.float32)
    p[:5] = [0.0, 1.0, 1e-9, 1 - 1e-9, 0.5]
    y = (g.random(2000) < 0.5).astype(np.int8)
    ref = log_loss(y, np.clip(p.astype(np.float64), oc.EPS, 1 - oc.EPS), labels=[0, 1])
    assert oc.metrics(p, y)["log_loss"] == pytest.approx(ref, rel=1e-12)


def test_ece_closed_forms():
    # one bin, mean prediction 0.75, frequency 0.5: ECE 0.25
    assert oc.metrics(np.full(8, 0.75, np.float32), [1, 0] * 4)["ece"] == pytest.approx(0.25, abs=1e-7)
    # two bins, each perfectly calibrated: ECE 0
    p = np.array([0.25] * 4 + [0.75] * 4, np.float32)
    y = [1, 0, 0, 0, 1, 1, 1, 0]
    assert oc.metrics(p, y)["ece"] == pytest.approx(0.0, abs=1e-7)
    # two bins with errors 0.25 (weight 1/2) and 0.45 (weight 1/2): 0.35
    p = np.array([0.25] * 4 + [0.95] * 4, np.float32)
    y = [1, 1, 0, 0, 1, 0, 1, 0.0]
    assert oc.metrics(p, np.array(y, np.int8))["ece"] == pytest.approx(0.5 * 0.25 + 0.5 * 0.45, abs=1e-7)


def test_ece_of_calibrated_draws_vanishes_with_n():
    g = np.random.default_rng(3)
    p = g.random(200_000).astype(np.float32)
    y = (g.random(200_000) < p).astype(np.int8)
    assert oc.metrics(p, y)["ece"] < 0.01
    # a miscalibrated estimator (predicting p^2 for frequency p) is far off
    assert oc.metrics(p ** 2, y)["ece"] > 0.1


def test_unlabelled_items_are_skipped_and_bins_edges():
    p = np.array([0.0, 0.1, 0.99999994, 1.0, 0.5, 0.5], np.float32)
    y = np.array([0, 1, 1, 1, -1, -1], np.int8)
    m = oc.metrics(p, y)
    assert m["n"] == 4 and m["n_pos"] == 3
    assert oc.ece_bin(np.float32(1.0)) == 9 and oc.ece_bin(np.float32(0.1)) == 1
    empty = oc.metrics(p, np.full(6, -1, np.int8))
    assert empty["n"] == 0 and np.isnan(empty["ece"])
