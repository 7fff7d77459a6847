"""GPU parity of sv_av_score, the fused estimator outputs of sv_spec_verify,
and sv_av_fit_step, against the oracle through the C ABI."""
import numpy as np
import pytest
import scipy.special as sp
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import TOL, compare_scores, compare_verify, flip_budget, gpu_score, gpu_verify, rel_close, to_device
from oracle import av as oav
from oracle import verify as ov
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


@pytest.mark.parametrize("name,B", [("tiny_fp32_b4_k4_v1024", 64), ("bf16_b64_k5_v32000", 64),
                                    ("bf16_b512_k8_v151936_t0.7", 16),
                                    ("fp32_b1024_k1to3_v129280_greedy_mix", 24)])
def test_av_score_parity(name, B):
    b = gen.make_batch(name, B=B)
    print(f"case {name} B={B}", flush=True)
    g = gpu_score(b)
    o = oav.av_score_batch(b)
    compare_scores(b, g["feature"], g["score"], o)
    # kept counts: exact unless a survival value sits within tolerance of the threshold
    for r in range(b.B):
        if g["num_kept"][r] != o["num_kept"][r]:
            k = int(b.num_draft[r])
            near = np.abs(o["survival"][r, :k] - b.prune_threshold) <= TOL[b.dtype] * b.prune_threshold
            assert near.any(), (r, g["num_kept"][r], o["num_kept"][r])


def test_no_fit_identity_on_gpu():
    """omega = 1, beta = 0: the score is the draft's top-token probability."""
    b = gen.make_batch("tiny_fp32_b4_k4_v1024", B=32)
    g = gpu_score(b)
    for r in range(b.B):
        for i in range(b.max_k):
            z = b.draft[b.draft_row_start[r] + i].astype(np.float64)
            assert abs(g["score"][r, i] - sp.softmax(z).max()) <= 1e-5 * sp.softmax(z).max()


def test_fused_feature_equals_av_score():
    """The feature and score sv_spec_verify produces from its own pass over the
    draft rows agree with sv_av_score's (64 KiB segments there, 32 KiB halves
    here: equal up to fp32 summation order) and with the oracle."""
    for name, B in [("bf16_b256_k4_v128256_peaked", 32), ("fp32_b1024_k1to3_v129280_greedy_mix", 32)]:
        b = gen.make_batch(name, B=B)
        v = gpu_verify(b, want_feature=True)
        s = gpu_score(b, threshold=0.0)
        assert np.all(rel_close(v["av_feature"], s["feature"], 1e-5, scale_floor=1.0))
        assert np.all(rel_close(v["av_score"], s["score"], 1e-5))
        compare_scores(b, v["av_feature"], v["av_score"], oav.av_score_batch(b))


def test_fused_feature_of_confident_and_tied_rows():
    """The exact re-summation of confident draft rows inside sv_spec_verify:
    tied maxima across segments, q_max ~ 1 - 1e-9, a single finite logit."""
    g = np.random.default_rng(2)
    B, K, V = 16, 4, 50000
    z = np.round(g.standard_normal((B * K, V)) * 2).astype(np.float32)
    z[0::4, 5] = 9.0
    z[0::4, 40000] = 9.0
    z[1::4, 123] = 30.0
    z[2::4, :] = -np.inf
    z[2::4, 7] = 1.0
    d = gen.f32_to_bf16_bits(z)
    zt = gen.f32_to_bf16_bits(np.round(g.standard_normal((B * (K + 1), V)) * 2).astype(np.float32))
    toks = np.tile(np.array([5, 123, 7, 11], np.int32), (B, 1))
    b = gen.Batch("ties_fused", B, V, K, "bf16", d, np.arange(B, dtype=np.int64) * K, zt,
                  np.arange(B, dtype=np.int64) * (K + 1), np.full(B, K, np.int32), toks,
                  np.ones(B, np.float32), np.full((B, K), 0.5, np.float32), np.full(B, 0.5, np.float32),
                  np.full(B, 0.5, np.float32), np.array([0.6, 0.5, 0.2, -0.1, -0.4], np.float32))
    v = gpu_verify(b, want_feature=True)
    compare_scores(b, v["av_feature"], v["av_score"], oav.av_score_batch(b, threshold=0.0), tol=1e-5)
    assert np.all(v["av_feature"][:, 2] == 80.0)


def test_feature_ties_and_peaked_rows():
    """Tied maxima (bf16) and very confident rows, where sum_{v != argmax} is tiny."""
    g = np.random.default_rng(1)
    B, K, V = 16, 4, 50000
    z = np.round(g.standard_normal((B * K, V)) * 2).astype(np.float32)
    z[0::4, 5] = 9.0
    z[0::4, 40000] = 9.0        # tie at the maximum in two segments
    z[1::4, 123] = 30.0         # q_max ~ 1 - 1e-9: the feature is large
    z[2::4, :] = -np.inf
    z[2::4, 7] = 1.0            # single finite logit: clamped feature
    d = gen.f32_to_bf16_bits(z)
    b = gen.Batch("ties", B, V, K, "bf16", d, np.arange(B, dtype=np.int64) * K, d,
                  np.arange(B, dtype=np.int64) * K, np.full(B, K, np.int32), np.zeros((B, K), np.int32),
                  np.ones(B, np.float32), np.zeros((B, K), np.float32), np.zeros(B, np.float32),
                  np.zeros(B, np.float32), np.array([0.6, 0.5, 0.2, -0.1, -0.4], np.float32))
    g_ = gpu_score(b, threshold=0.0)
    compare_scores(b, g_["feature"], g_["score"], oav.av_score_batch(b, threshold=0.0), tol=1e-5)
    assert np.all(g_["feature"][:, 2] == 80.0)


def _fit_inputs(seed, B, K, omega, beta):
    g = np.random.default_rng(seed)
    x = g.normal(1.0, 1.5, (B, K)).astype(np.float32)
    p = sp.expit(omega * x.astype(np.float64) + np.asarray(beta)[None, :])
    y = (g.random((B, K)) < p).astype(np.int8)
    lab = np.full((B, K), -1, np.int8)
    for r in range(B):
        for i in range(K):
            lab[r, i] = y[r, i]
            if y[r, i] == 0:
                break
    return x, lab


def test_fit_step_parity_one_round():
    K = 5
    params0 = np.array([1.0] + [0.0] * K, np.float32)
    dev_p = torch.tensor(params0, device="cuda")
    dev_acc = torch.zeros(K, 6, dtype=torch.float64, device="cuda")
    o_p, o_acc = params0.copy(), np.zeros((K, 6))
    for step in range(3):
        x, lab = _fit_inputs(step, 700, K, 1.2, [0.5 - 0.3 * i for i in range(K)])
        last = step == 2
        sv.sv_av_fit_step(torch.tensor(x, device="cuda"), torch.tensor(lab, device="cuda"), dev_p, dev_acc,
                          damping_c=10.0, ridge=1e-6, do_update=last)
        if not last:
            torch.cuda.synchronize()
            o_acc_next = o_acc + oav.fit_sums(x, lab, o_p)
            assert np.allclose(dev_acc.cpu().numpy(), o_acc_next, rtol=1e-12, atol=1e-12)
        o_p, o_acc = oav.fit_step(x, lab, o_p, o_acc, damping_c=10.0, ridge=1e-6, do_update=last)
    torch.cuda.synchronize()
    assert np.all(dev_acc.cpu().numpy() == 0)
    assert rel_close(dev_p.cpu().numpy(), o_p, 1e-5).all(), (dev_p.cpu().numpy(), o_p)


def test_fit_converges_to_planted_parameters_on_gpu():
    K = 5
    omega, beta = 1.2, [0.5 - 0.3 * i for i in range(K)]
    x, lab = _fit_inputs(42, 8000, K, omega, beta)
    xd, ld = torch.tensor(x, device="cuda"), torch.tensor(lab, device="cuda")
    p = torch.tensor([1.0] + [0.0] * K, device="cuda")
    acc = torch.zeros(K, 6, dtype=torch.float64, device="cuda")
    o_p, o_acc = p.cpu().numpy(), np.zeros((K, 6))
    for _ in range(25):
        sv.sv_av_fit_step(xd, ld, p, acc, damping_c=10.0, ridge=1e-6, do_update=True)
        o_p, o_acc = oav.fit_step(x, lab, o_p, o_acc, damping_c=10.0, ridge=1e-6, do_update=True)
    got = p.cpu().numpy()
    assert rel_close(got, o_p, 1e-5).all(), (got, o_p)
    H, _ = oav.hessian_gradient(oav.fit_sums(x, lab, got))
    sd = np.sqrt(np.diag(np.linalg.inv(H)))
    assert np.all(np.abs(got - np.array([omega] + beta)) < 4 * sd)


def test_fit_with_no_labels_keeps_parameters():
    K = 4
    p0 = torch.tensor([0.7, 0.1, 0.2, 0.3, 0.4], device="cuda")
    p = p0.clone()
    acc = torch.zeros(K, 6, dtype=torch.float64, device="cuda")
    sv.sv_av_fit_step(torch.zeros(10, K, device="cuda"), torch.full((10, K), -1, dtype=torch.int8, device="cuda"),
                      p, acc, do_update=True)
    torch.cuda.synchronize()
    assert torch.equal(p, p0)


@pytest.mark.parametrize("B", [24, 512])
def test_score_prune_verify_refit_pipeline(B):
    """Score -> prune at 0.3 -> ragged verify -> refit, all on the device with
    no host round trip, compared with the oracle run the same way (B = 512:
    the long-draft workload at full size, every request)."""
    b = gen.make_batch("bf16_b512_k8_v151936_t0.7", B=B)
    d = to_device(b)
    print(f"case pipeline B={B}: gpu", flush=True)
    s = sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], d["av_params"],
                       max_k=b.max_k, prune_threshold=b.prune_threshold)
    v = sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], s["num_kept"],
                          d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                          max_k=b.max_k)
    p = d["av_params"].clone()
    acc = torch.zeros(b.max_k, 6, dtype=torch.float64, device="cuda")
    sv.sv_av_fit_step(s["feature"], v["labels"], p, acc, do_update=True)
    torch.cuda.synchronize()
    kept = s["num_kept"].cpu().numpy()
    print(f"case pipeline B={B}: oracle", flush=True)
    os_ = oav.av_score_batch(b)
    compare_scores(b, s["feature"].cpu().numpy(), s["score"].cpu().numpy(), os_)
    # kept counts: exact unless a survival sits within tolerance of the threshold
    for r in np.nonzero(kept != os_["num_kept"])[0]:
        k = int(b.num_draft[r])
        near = np.abs(os_["survival"][r, :k] - b.prune_threshold) <= TOL[b.dtype] * b.prune_threshold
        assert near.any(), (r, kept[r], os_["num_kept"][r])
    import dataclasses
    pruned = dataclasses.replace(b, num_draft=kept.astype(np.int32))  # what the device verified
    gv = {k: t.cpu().numpy() for k, t in v.items()}
    ovr = ov.verify_batch(pruned)
    assert compare_verify(pruned, gv, ovr) <= flip_budget(ovr, pruned.num_draft)
    o_p, _ = oav.fit_step(os_["feature"].astype(np.float32), ovr["labels"], b.av_params, np.zeros((b.max_k, 6)),
                          do_update=True)
    # parameters cross zero (the bounded step can take omega from 1 to ~0):
    # tolerance scale max(1, |value|), as for the feature
    assert rel_close(p.cpu().numpy(), o_p, 2e-3, scale_floor=1.0).all(), (p.cpu().numpy(), o_p)


def test_refit_loop_of_the_benchmark_stays_bounded():
    """The benchmark's step on the device: verification of the peaked
    B=256, K=4, V=128256 batch (three input sets in turn) with the estimator
    feature, then a refit on every step from omega = 1, beta = 0.  Every
    step's update equals the oracle's from the same parameters, features and
    labels; the parameters stay bounded (the step bound), and the log-loss of
    the labelled drafts falls."""
    sets = [gen.make_batch("bf16_b256_k4_v128256_peaked", trial=t) for t in range(3)]
    devs = [to_device(b) for b in sets]
    b0 = sets[0]
    K = b0.max_k
    p = torch.tensor(b0.av_params, device="cuda")
    acc = torch.zeros(K, 6, dtype=torch.float64, device="cuda")
    ws = sv.Workspace()
    feats, labs = [], []
    for step in range(30):
        b, d = sets[step % 3], devs[step % 3]
        out = sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                d["num_draft"], d["draft_tokens"], d["temperature"], d["u_accept"],
                                d["u_residual"], d["u_bonus"], max_k=K, av_params=p, want_feature=True,
                                workspace=ws)
        before = p.cpu().numpy()
        sv.sv_av_fit_step(out["av_feature"], out["labels"], p, acc, do_update=True)
        x, lab = out["av_feature"].cpu().numpy(), out["labels"].cpu().numpy()
        want, _ = oav.fit_step(x, lab, before, np.zeros((K, 6)), do_update=True)
        got = p.cpu().numpy()
        assert rel_close(got, want, 1e-5, scale_floor=1.0).all(), (step, got, want)
        if step < 3:
            feats.append(x)
            labs.append(lab)
    print(f"case refit loop: params after 30 steps {p.cpu().numpy().tolist()}", flush=True)
    final = p.cpu().numpy()
    assert np.all(np.isfinite(final)) and np.abs(final).max() < 10.0
    X, L = np.concatenate(feats), np.concatenate(labs)
    assert oav.nll(X, L, final) < 0.75 * oav.nll(X, L, b0.av_params)
