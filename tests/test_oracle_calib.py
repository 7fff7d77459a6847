"""Pins of the calibration-metric oracle ([AV] "Other features considered":
AUC, log-loss, ECE) against library routines for the same definitions,
closed forms and a direct pair count."""
import numpy as np
import pytest
from sklearn.metrics import log_loss, roc_auc_score

from oracle import calib as oc


def _grid(g, n):
    """Scores on the AUC grid (bin centres), where the binned AUC is exact."""
    return ((g.integers(0, oc.AUC_BINS, n) + 0.5) / oc.AUC_BINS).astype(np.float32)


@pytest.mark.parametrize("seed", range(5))
def test_auc_on_grid_scores_equals_the_library(seed):
    g = np.random.default_rng(seed)
    p = _grid(g, 3000)
    y = (g.random(3000) < p).astype(np.int8)
    assert oc.metrics(p, y)["auc"] == pytest.approx(roc_auc_score(y, p), abs=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_auc_equals_a_direct_pair_count(seed):
    # P(pos > neg) + 1/2 P(tie) over the binned scores, by counting pairs
    g = np.random.default_rng(10 + seed)
    p = g.random(400).astype(np.float32)
    y = (g.random(400) < 0.6).astype(np.int8)
    b = oc.auc_bin(p)
    bp, bn = b[y == 1], b[y == 0]
    wins = (bp[:, None] > bn[None, :]).sum() + 0.5 * (bp[:, None] == bn[None, :]).sum()
    assert oc.metrics(p, y)["auc"] == pytest.approx(wins / (len(bp) * len(bn)), abs=1e-12)
    # and the binned AUC is within half the tied-pair share of the exact one
    ties = (bp[:, None] == bn[None, :]).mean()
    assert abs(oc.metrics(p, y)["auc"] - roc_auc_score(y, p)) <= 0.5 * ties + 1e-12


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
    assert oc.auc_bin(np.float32(1.0)) == oc.AUC_BINS - 1
    empty = oc.metrics(p, np.full(6, -1, np.int8))
    assert empty["n"] == 0 and np.isnan(empty["ece"])
