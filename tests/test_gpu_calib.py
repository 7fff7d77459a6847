"""GPU parity of the calibration metrics (sv_av_calib_*) against the oracle
([AV] "Other features considered": AUC, log-loss, ECE) over a stream of
several steps: counts exactly, sums and metrics within 1e-12 relative
(binary64 sums in another order), and bit-identical results on repeats."""
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


def stream(seed, steps, B, max_k, grid=False):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(steps):
        if grid:
            p = ((g.integers(0, oc.AUC_BINS, (B, max_k)) + 0.5) / oc.AUC_BINS).astype(np.float32)
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
    np.testing.assert_array_equal(acc[33:33 + oc.AUC_BINS],
                                  np.bincount(oc.auc_bin(p[lab & (y == 1)]), minlength=oc.AUC_BINS))
    np.testing.assert_array_equal(acc[33 + oc.AUC_BINS:],
                                  np.bincount(oc.auc_bin(p[lab & (y == 0)]), minlength=oc.AUC_BINS))
    np.testing.assert_array_equal(acc[3:13], np.bincount(oc.ece_bin(p[lab]), minlength=10))
    assert m[0] == pytest.approx(ref["auc"], rel=1e-12)
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
    ref = oc.metrics(np.concatenate(ps), np.concatenate(ys))
    for k, name in enumerate(["auc", "log_loss", "ece"]):
        assert m[k] == pytest.approx(ref[name], rel=1e-9, abs=1e-15)
