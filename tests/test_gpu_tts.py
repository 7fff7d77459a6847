"""GPU parity of the TTS distillation gradient (sv_tts_grad) against the
oracle (page "ملخص تقني: التخمين في وقت الاختبار (TTS)", "Algorithm" step 3):
every gradient element within a tolerance derived from the arithmetic, the
loss within 1e-4 relative, rows past K_b untouched and their loss NaN."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import dev_rows
from oracle import tts as ot
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]

DEV = torch.device("cuda")
# fp32 arithmetic from exactly widened inputs: q and p carry ~1e-6 relative
# error, so an element's error is ~1e-6 of the row's largest probability
# (times w / T); a bf16 output adds its rounding (2^-9 of the value)
REL = {"f32": 1e-5, "bf16": 4e-3}
ABS = {"f32": 2e-6, "bf16": 2e-5}


def row_scale(zd, zt, T, w):
    """w / T times the row pair's largest probability: the size of the
    gradient's rounding errors."""
    T = T if T > 0 else 1.0
    q, _ = ot._softmax(zd, T)
    p, _ = ot._softmax(zt, T)
    return w / T * max(q.max(), p.max())


def rows_f32(bits_or_f32, dtype):
    return gen.bf16_bits_to_f32(bits_or_f32) if dtype == "bf16" else np.asarray(bits_or_f32, np.float32)


def make(seed, B, max_k, V, dtype, prev, stride_pad=0, ragged=True):
    g = np.random.default_rng(seed)
    K = g.integers(0 if ragged else max_k, max_k + 1, B).astype(np.int32)
    n = B * max_k
    zd = g.normal(0, 2.5, (n, V)).astype(np.float32)
    zt = (zd + g.normal(0, 1.0, (n, V))).astype(np.float32)
    zp = (zd + g.normal(0, 0.5, (n, V))).astype(np.float32) if prev else None
    if dtype == "bf16":
        zd, zt = gen.f32_to_bf16_bits(zd), gen.f32_to_bf16_bits(zt)
        zp = gen.f32_to_bf16_bits(zp) if prev else None
    T = g.choice(np.array([0.0, 0.7, 1.0, 1.3], np.float32), B)
    w = (1.0 / (1.0 + np.arange(max_k))).astype(np.float32)
    return K, zd, zt, zp, T, w


def to_dev(rows, dtype, pad):
    if pad:
        rows = np.concatenate([rows, np.zeros((rows.shape[0], pad), rows.dtype)], axis=1)
    t = dev_rows(rows, dtype, DEV)
    return t[:, :rows.shape[1] - pad] if pad else t


@pytest.mark.parametrize("dtype,prev,lam,V,pad", [("f32", False, 0.0, 1000, 0), ("f32", True, 0.5, 1003, 0),
                                                  ("bf16", False, 0.3, 4096, 0), ("bf16", True, 1.0, 2500, 3),
                                                  ("f32", True, 0.2, 70000, 5)])
def test_gradient_and_loss_match_the_oracle(dtype, prev, lam, V, pad):
    B, max_k = 5, 4
    K, zd, zt, zp, T, w = make(7, B, max_k, V, dtype, prev)
    print(f"case tts {dtype} prev={prev} lam={lam} V={V} pad={pad}", flush=True)
    starts = torch.arange(B, dtype=torch.int64, device=DEV) * max_k
    d, t = to_dev(zd, dtype, pad), to_dev(zt, dtype, pad)
    p = to_dev(zp, dtype, pad) if prev else None
    sentinel = torch.full((B * max_k, V), 7.0, device=DEV).to(d.dtype)
    out = sv.sv_tts_grad(d, starts, t, starts, torch.from_numpy(K).to(DEV), torch.from_numpy(T).to(DEV),
                         torch.from_numpy(w).to(DEV), max_k, lam, prev_logits=p,
                         prev_row_start=starts if prev else None, out={"grad": sentinel})
    torch.cuda.synchronize()
    grad = out["grad"].float().cpu().numpy()
    loss = out["loss"].cpu().numpy()
    fd, ft = rows_f32(zd, dtype), rows_f32(zt, dtype)
    fp = rows_f32(zp, dtype) if prev else None
    for b in range(B):
        for k in range(max_k):
            r = b * max_k + k
            if k >= K[b]:
                assert np.isnan(loss[b, k])
                assert np.all(grad[r] == 7.0)
                continue
            gref, lref = ot.position(fd[r], ft[r], fp[r] if prev else None, float(T[b]), float(w[k]), lam)
            scale = row_scale(fd[r], ft[r], float(T[b]), float(w[k]))
            err = np.abs(grad[r] - gref)
            assert np.all(err <= REL[dtype] * np.abs(gref) + ABS[dtype] * scale), (b, k, err.max(), scale)
            assert loss[b, k] == pytest.approx(lref, rel=1e-4, abs=1e-6)


def test_identical_rows_and_benchmark_shape():
    # the benchmark's rows (B=256, K=4, V=128256 bf16): the canvas of a sample
    # of requests checked in full against the oracle
    b = gen.make_batch("bf16_b256_k4_v128256_peaked", trial=0)
    d = dev_rows(b.draft, b.dtype, DEV)
    t = dev_rows(b.target, b.dtype, DEV)
    print("case tts benchmark shape", flush=True)
    w = torch.ones(b.max_k, dtype=torch.float32, device=DEV)
    out = sv.sv_tts_grad(d, torch.from_numpy(b.draft_row_start).to(DEV), t,
                         torch.from_numpy(b.target_row_start).to(DEV), torch.from_numpy(b.num_draft).to(DEV),
                         torch.from_numpy(b.temperature).to(DEV), w, b.max_k, 0.0)
    torch.cuda.synchronize()
    loss = out["loss"].cpu().numpy()
    for r in range(0, b.B, 37):
        for k in range(int(b.num_draft[r])):
            zd = gen.bf16_bits_to_f32(b.draft[int(b.draft_row_start[r]) + k])
            zt = gen.bf16_bits_to_f32(b.target[int(b.target_row_start[r]) + k])
            gref, lref = ot.position(zd, zt, None, float(b.temperature[r]), 1.0, 0.0)
            g = out["grad"][r * b.max_k + k].float().cpu().numpy()
            scale = row_scale(zd, zt, float(b.temperature[r]), 1.0)
            assert np.all(np.abs(g - gref) <= REL["bf16"] * np.abs(gref) + ABS["bf16"] * scale)
            assert loss[r, k] == pytest.approx(lref, rel=1e-4, abs=1e-6)
    # identical draft and target rows: zero gradient and loss
    same = sv.sv_tts_grad(d, torch.from_numpy(b.draft_row_start).to(DEV), d,
                          torch.from_numpy(b.draft_row_start).to(DEV), torch.from_numpy(b.num_draft).to(DEV),
                          torch.from_numpy(b.temperature).to(DEV), w, b.max_k, 0.5)
    torch.cuda.synchronize()
    assert float(same["grad"].float().abs().max()) == 0.0
    assert np.nanmax(np.abs(same["loss"].cpu().numpy())) == 0.0


@pytest.mark.parametrize("prev", [False, True])
def test_statistics_reused_from_the_verification(prev):
    """The gradient taken with the row statistics of the sv_spec_verify call
    just made on the same rows equals the oracle's like the two-pass one."""
    b = gen.make_batch("bf16_b64_k5_v32000", trial=3)
    from gpu_harness import to_device
    d = to_device(b)
    print(f"case tts reuse prev={prev}", flush=True)
    ws = sv.Workspace()
    sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                      d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                      max_k=b.max_k, want_feature=True, workspace=ws)
    w = torch.linspace(1.0, 0.5, b.max_k, device=DEV)
    prev_rows = (d["draft"].float() + 0.25).to(d["draft"].dtype) if prev else None
    kw = dict(prev_logits=prev_rows, prev_row_start=d["draft_row_start"] if prev else None)
    out = sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                         d["temperature"], w, b.max_k, 0.4, verify_workspace=ws, **kw)
    torch.cuda.synchronize()
    loss = out["loss"].cpu().numpy()
    wh = w.cpu().numpy()
    pr = prev_rows.float().cpu().numpy() if prev else None
    for r in range(0, b.B, 7):
        for k in range(int(b.num_draft[r])):
            zd = gen.bf16_bits_to_f32(b.draft[int(b.draft_row_start[r]) + k])
            zt = gen.bf16_bits_to_f32(b.target[int(b.target_row_start[r]) + k])
            zp = pr[int(b.draft_row_start[r]) + k] if prev else None
            gref, lref = ot.position(zd, zt, zp, float(b.temperature[r]), float(wh[k]), 0.4)
            g = out["grad"][r * b.max_k + k].float().cpu().numpy()
            scale = row_scale(zd, zt, float(b.temperature[r]), float(wh[k]))
            assert np.all(np.abs(g - gref) <= REL["bf16"] * np.abs(gref) + ABS["bf16"] * scale)
            assert loss[r, k] == pytest.approx(lref, rel=1e-4, abs=1e-6)


@pytest.mark.parametrize("prev", [False, True])
def test_statistics_reused_with_greedy_requests(prev):
    """Greedy requests (T = 0) in the verification, whose target rows'
    statistics hold only maxima and argmaxes: the gradient reusing the
    statistics equals the oracle's at T = 1 (the verification made with the
    estimator feature, so that every canvas draft row was read)."""
    b = gen.make_batch("fp32_b1024_k1to3_v129280_greedy_mix", B=24)
    from gpu_harness import to_device
    d = to_device(b)
    print(f"case tts reuse with greedy requests prev={prev}", flush=True)
    ws = sv.Workspace()
    sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                      d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                      max_k=b.max_k, want_feature=True, workspace=ws)
    w = torch.linspace(1.0, 0.5, b.max_k, device=DEV)
    lam = 0.3 if prev else 0.0
    prev_rows = d["draft"] + 0.25 if prev else None
    kw = dict(prev_logits=prev_rows, prev_row_start=d["draft_row_start"] if prev else None)
    out = sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                         d["temperature"], w, b.max_k, lam, verify_workspace=ws, **kw)
    torch.cuda.synchronize()
    loss = out["loss"].cpu().numpy()
    wh = w.cpu().numpy()
    pr = prev_rows.cpu().numpy() if prev else None
    greedy = 0
    for r in range(b.B):
        greedy += int(b.temperature[r] == 0.0)
        for k in range(int(b.num_draft[r])):
            zd = b.draft[int(b.draft_row_start[r]) + k]
            zt = b.target[int(b.target_row_start[r]) + k]
            zp = pr[int(b.draft_row_start[r]) + k] if prev else None
            gref, lref = ot.position(zd, zt, zp, float(b.temperature[r]), float(wh[k]), lam)
            g = out["grad"][r * b.max_k + k].float().cpu().numpy()
            scale = row_scale(zd, zt, float(b.temperature[r]) or 1.0, float(wh[k]))
            assert np.all(np.abs(g - gref) <= REL["f32"] * np.abs(gref) + ABS["f32"] * scale), (r, k)
            assert loss[r, k] == pytest.approx(lref, rel=1e-4, abs=1e-6), (r, k)
    assert greedy > 0


def test_reused_statistics_calls_repeat_bit_identically():
    """The segmented gradient hands each position's loss to the request's
    last workgroup through an arrival counter in the workspace arena; every
    call leaves the counters at zero, so the next call gives the same
    gradient and loss bit for bit (other work in between on the stream)."""
    b = gen.make_batch("bf16_b64_k5_v32000", trial=4)
    from gpu_harness import to_device
    d = to_device(b)
    print("case tts reuse repeated", flush=True)
    ws = sv.Workspace()
    sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                      d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                      max_k=b.max_k, want_feature=True, workspace=ws)
    w = torch.linspace(1.0, 0.25, b.max_k, device=DEV)
    call = lambda: sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                  d["num_draft"], d["temperature"], w, b.max_k, 0.0, verify_workspace=ws)
    first = call()
    torch.cuda.synchronize()
    g0, l0 = first["grad"].clone(), first["loss"].cpu().numpy()
    params = torch.tensor(b.av_params, device=DEV)
    sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], params, b.max_k,
                   workspace=sv.Workspace())
    second = call()
    torch.cuda.synchronize()
    assert torch.equal(second["grad"], g0)
    l1 = second["loss"].cpu().numpy()
    np.testing.assert_array_equal(np.isnan(l1), np.isnan(l0))
    np.testing.assert_array_equal(l1[~np.isnan(l1)], l0[~np.isnan(l0)])
    K = b.num_draft
    assert all(np.isnan(l1[r, k]) == (k >= K[r]) for r in range(b.B) for k in range(b.max_k))
