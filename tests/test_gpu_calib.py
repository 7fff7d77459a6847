"""GPU parity of the calibration metrics (sv_av_calib_*) against the oracle
([AV] "Other features considered": AUC, log-loss, ECE) over a stream of
several steps.

The kernel keeps per class a histogram of SV_CALIB_AUC_BINS equal-width score
bins and reports the AUC of the binned scores; the oracle computes the AUC as
the page defines it, over every pair.  The two differ only for accepted and
rejected drafts in one bin (the binned AUC counts such a pair as a tie), so
the kernel's AUC is checked against the oracle's within half the share of
such pairs, and its histograms and binned AUC exactly against a binned
reference kept here (the kernel's own design, not the page's).  Log-loss and
ECE within 1e-12 / 1e-9 relative (binary64 sums in another order); repeats
bit-identical."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import to_device
from oracle import calib as oc
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]

DEV = torch.device("cuda")
BINS = sv.SV_CALIB_AUC_BINS


def auc_bin(p32):
    """The kernel's AUC bin of a binary32 score: min(floor(BINS * p), BINS - 1)."""
    return np.minimum(np.floor(np.asarray(p32, np.float32) * np.float32(BINS)).astype(np.int64), BINS - 1)


def binned_auc(p, y):
    """AUC of the binned scores and the share of (accepted, rejected) pairs in
    one bin."""
    b = auc_bin(p)
    pos = np.bincount(b[y == 1], minlength=BINS).astype(np.float64)
    neg = np.bincount(b[y == 0], minlength=BINS).astype(np.float64)
    pairs = pos.sum() * neg.sum()
    below = np.cumsum(neg) - neg
    return float((pos * below).sum() + 0.5 * (pos * neg).sum()) / pairs, float((pos * neg).sum()) / pairs


def stream(seed, steps, B, max_k, grid=False):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(steps):
        if grid:
            p = ((g.integers(0, BINS, (B, max_k)) + 0.5) / BINS).astype(np.float32)
        else:
            p = g.random((B, max_k)).astype(np.float32)
        y = (g.random((B, max_k)) < p ** 1.3).astype(np.int8)
        y[g.random((B, max_k)) < 0.3] = -1  # unlabelled positions
        out.append((p, y))
    return out


def run(items, reset=True):
    acc = torch.zeros(sv.SV_CALIB_WORDS, dtype=torch.float64, device=DEV)
    for p, y in items:
        sv.sv_av_calib_accumulate(torch.from_numpy(p).to(DEV), torch.from_numpy(y).to(DEV), acc)
    snap = acc.clone()
    m = sv.sv_av_calib_metrics(acc, reset=reset)
    torch.cuda.synchronize()
    return m.cpu().numpy(), snap.cpu().numpy(), acc.cpu().numpy()


@pytest.mark.parametrize("seed,steps,B,max_k,grid", [(0, 1, 4, 4, False), (1, 5, 256, 4, False),
                                                      (2, 3, 1024, 8, True), (3, 2, 4096, 16, False),
                                                      (4, 20, 64, 5, False)])
def test_stream_metrics_match_the_oracle(seed, steps, B, max_k, grid):
    items = stream(seed, steps, B, max_k, grid)
    print(f"case calib seed={seed} steps={steps} B={B} max_k={max_k}", flush=True)
    m, acc, after = run(items)
    p = np.concatenate([a.reshape(-1) for a, _ in items])
    y = np.concatenate([b.reshape(-1) for _, b in items])
    ref = oc.metrics(p, y)
    assert acc[0] == ref["n"] and acc[1] == ref["n_pos"]
    lab = (y == 0) | (y == 1)
    np.testing.assert_array_equal(acc[33:33 + BINS], np.bincount(auc_bin(p[lab & (y == 1)]), minlength=BINS))
    np.testing.assert_array_equal(acc[33 + BINS:], np.bincount(auc_bin(p[lab & (y == 0)]), minlength=BINS))
    np.testing.assert_array_equal(acc[3:13], np.bincount(oc.ece_bin(p[lab]), minlength=10))
    # the page's AUC (oracle) within half the tied-pair share; the binned AUC exactly
    auc_b, tied = binned_auc(p[lab], y[lab])
    assert abs(m[0] - ref["auc"]) <= 0.5 * tied + 1e-12, (m[0], ref["auc"], tied)
    assert m[0] == pytest.approx(auc_b, rel=1e-12)
    if grid:
        assert m[0] == pytest.approx(ref["auc"], rel=1e-12)  # one score value per bin: no merged pairs
    assert m[1] == pytest.approx(ref["log_loss"], rel=1e-12)
    assert m[2] == pytest.approx(ref["ece"], rel=1e-9, abs=1e-15)
    assert np.all(after == 0)  # reset
    m2, acc2, _ = run(items)
    np.testing.assert_array_equal(m, m2)
    np.testing.assert_array_equal(acc, acc2)


def test_undefined_metrics_are_nan():
    p = np.full((8, 2), 0.4, np.float32)
    m, _, _ = run([(p, np.full((8, 2), -1, np.int8))])
    assert np.all(np.isnan(m))
    m, _, _ = run([(p, np.ones((8, 2), np.int8))])
    assert np.isnan(m[0]) and m[1] == pytest.approx(-np.log(0.4), rel=1e-7) and m[2] == pytest.approx(0.6, rel=1e-6)


def test_verification_labels_and_scores_on_device():
    """Scores from sv_av_score and labels from sv_spec_verify, accumulated
    over steps without host round trips."""
    acc = torch.zeros(sv.SV_CALIB_WORDS, dtype=torch.float64, device=DEV)
    ps, ys = [], []
    for trial in range(3):
        b = gen.make_batch("bf16_b64_k5_v32000", trial=10 + trial)
        d = to_device(b)
        sc = sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], d["av_params"],
                            b.max_k, 0.0)
        out = sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                d["num_draft"], d["draft_tokens"], d["temperature"], d["u_accept"],
                                d["u_residual"], d["u_bonus"], max_k=b.max_k)
        sv.sv_av_calib_accumulate(sc["score"], out["labels"], acc)
        ps.append(sc["score"].cpu().numpy())
        ys.append(out["labels"].cpu().numpy())
    print("case calib pipeline bf16_b64_k5_v32000", flush=True)
    m = sv.sv_av_calib_metrics(acc).cpu().numpy()
    P, Y = np.concatenate(ps).reshape(-1), np.concatenate(ys).reshape(-1)
    ref = oc.metrics(P, Y)
    for k, name in enumerate(["log_loss", "ece"], start=1):
        assert m[k] == pytest.approx(ref[name], rel=1e-9, abs=1e-15)
    lab = (Y == 0) | (Y == 1)
    auc_b, tied = binned_auc(P[lab], Y[lab])
    assert abs(m[0] - ref["auc"]) <= 0.5 * tied + 1e-12, (m[0], ref["auc"], tied)
    assert m[0] == pytest.approx(auc_b, rel=1e-12)
