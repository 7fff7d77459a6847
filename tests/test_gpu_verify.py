"""GPU parity of sv_spec_verify against the oracle, through the C ABI.

Sizes: every workload at a size the oracle finishes in seconds (several
segments and a ragged tail), the 256 x 4 x 128256 bf16 batch in full, the
larger two at full size with sampled requests compared one by one, plus edge
cases: ragged and misaligned rows, empty drafts, maximum draft length and
vocabulary, broadcast rows, -inf logits, identical and disjoint
distributions, greedy ties, determinism and workspace reuse."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import compare_scores, compare_verify, flip_budget, gpu_verify, to_device
from oracle import av as oav
from oracle import verify as ov
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,B", [
    ("tiny_fp32_b4_k4_v1024", 4),
    ("tiny_fp32_b4_k4_v1024", 256),
    ("bf16_b64_k5_v32000", 64),
    ("bf16_b256_k4_v128256_peaked", 24),
    ("bf16_b512_k8_v151936_t0.7", 12),
    ("fp32_b1024_k1to3_v129280_greedy_mix", 40),
])
def test_parity_workloads_small(name, B):
    b = gen.make_batch(name, B=B)
    _log(f"case {name} B={B}")
    g = gpu_verify(b)
    o = ov.verify_batch(b)
    flips = compare_verify(b, g, o)
    assert flips <= flip_budget(o, b.num_draft)


def test_parity_full_peaked_b256_k4_v128256():
    """The benchmarked batch, in the benchmarked launch (estimator feature and
    score from the same pass), every request."""
    b = gen.make_batch("bf16_b256_k4_v128256_peaked")
    _log("case peaked full, with the estimator outputs")
    g = gpu_verify(b, want_feature=True)
    o = ov.verify_batch(b)
    flips = compare_verify(b, g, o)
    assert flips <= flip_budget(o, b.num_draft)
    compare_scores(b, g["av_feature"], g["av_score"], oav.av_score_batch(b))
    # acceptance level of this recipe: about 0.16 per position, so the mean
    # accept length (~alpha / (1 - alpha) truncated at K) is about 0.16-0.19
    assert 0.08 < g["accept_len"].mean() < 0.35


def _properties(b, g):
    """Checks that hold for every request at any size."""
    a = g["accept_len"]
    assert np.all((a >= 0) & (a <= b.num_draft))
    for r in range(b.B):
        k, ar = int(b.num_draft[r]), int(a[r])
        assert np.array_equal(g["out_tokens"][r, :ar], b.draft_tokens[r, :ar])
        assert 0 <= g["out_tokens"][r, ar] < b.V
        assert np.all(g["out_tokens"][r, ar + 1:] == -1)
        lab = g["labels"][r]
        assert np.all(lab[:ar] == 1) and np.all(lab[ar + 1:] == -1)
        assert lab[ar] == (0 if ar < k else -1) if ar < b.max_k else True


@pytest.mark.parametrize("name", ["bf16_b512_k8_v151936_t0.7", "fp32_b1024_k1to3_v129280_greedy_mix"])
def test_parity_full_size_every_request(name):
    """The two largest workloads at full size, every request against the
    oracle (4096 and about 2048 positions)."""
    b = gen.make_batch(name)
    _log(f"case {name} full: gpu")
    g = gpu_verify(b)
    _properties(b, g)
    _log(f"case {name} full: oracle")
    o = ov.verify_batch(b)
    flips = compare_verify(b, g, o)
    assert flips <= flip_budget(o, b.num_draft)
    if name.startswith("fp32"):
        # greedy requests need no floating-point decision: exact, always
        greedy = np.nonzero(b.temperature == 0)[0]
        assert np.array_equal(g["accept_len"][greedy], o["accept_len"][greedy])
        assert np.array_equal(g["out_tokens"][greedy], o["out_tokens"][greedy])


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _custom_batch(zd, zt, toks, T, dtype="f32", K=None, seed=0, stride_pad=0):
    """Batch of B requests from explicit fp32 rows zd [B, K, V], zt [B, K+1, V]."""
    B, maxk, V = zd.shape
    g = np.random.default_rng(seed)
    K = np.full(B, maxk, np.int32) if K is None else np.asarray(K, np.int32)
    stride = V + stride_pad
    d = np.zeros((B * maxk, stride), np.float32)
    t = np.zeros((B * (maxk + 1), stride), np.float32)
    d[:, :V] = zd.reshape(-1, V)
    t[:, :V] = zt.reshape(-1, V)
    if dtype == "bf16":
        d, t = gen.f32_to_bf16_bits(d), gen.f32_to_bf16_bits(t)
    b = gen.Batch("custom", B, V, maxk, dtype, d, np.arange(B, dtype=np.int64) * maxk, t,
                  np.arange(B, dtype=np.int64) * (maxk + 1), K, np.asarray(toks, np.int32).reshape(B, maxk),
                  np.broadcast_to(np.asarray(T, np.float32), (B,)).copy(), g.random((B, maxk), dtype=np.float32),
                  g.random(B, dtype=np.float32), g.random(B, dtype=np.float32),
                  np.array([1.0] + [0.0] * maxk, np.float32))
    return b


def _run_custom(b, stride=None):
    """Like gpu_verify but honours a row stride larger than V."""
    d = to_device(b)
    if b.draft.shape[1] != b.V:
        d["draft"] = d["draft"][:, :b.V]
        d["target"] = d["target"][:, :b.V]
    out = sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                            d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                            max_k=b.max_k)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _oracle_custom(b):
    """Oracle on a batch whose rows may be wider than V (stride padding)."""
    if b.draft.shape[1] == b.V:
        return ov.verify_batch(b)
    import dataclasses
    return ov.verify_batch(dataclasses.replace(b, draft=b.draft[:, :b.V], target=b.target[:, :b.V]))


def _draw_tokens(zd, T, seed):
    g = np.random.default_rng(seed)
    B, K, V = zd.shape
    if T == 0:
        return np.argmax(zd, axis=2)
    return np.argmax(zd / T - np.log(g.standard_exponential((B, K, V))), axis=2)


@pytest.mark.parametrize("V,dtype,pad", [(1000, "f32", 0), (1031, "bf16", 0), (1000, "bf16", 3), (1001, "f32", 1),
                                         (5, "f32", 0), (7, "bf16", 1), (1, "f32", 0), (2, "bf16", 0),
                                         (40000, "bf16", 5), (16385, "f32", 0)])
def test_ragged_and_misaligned_rows(V, dtype, pad):
    g = np.random.default_rng(V)
    B, K = 48, 3
    zd = (2.0 * g.standard_normal((B, K, V))).astype(np.float32)
    zt = (zd[:, [0, 1, 2, 2], :] * 0 + 2.0 * g.standard_normal((B, K + 1, V))).astype(np.float32)
    zt[:, :K] = 0.7 * zd + zt[:, :K] * 0.5
    if dtype == "bf16":
        zd = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(zd))
    toks = _draw_tokens(zd, 1.0, V + 1)
    b = _custom_batch(zd, zt, toks, 1.0, dtype=dtype, stride_pad=pad, seed=V)
    _log(f"case V={V} {dtype} pad={pad}")
    gpu = _run_custom(b)
    o = _oracle_custom(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)


def test_empty_and_ragged_draft_counts():
    g = np.random.default_rng(3)
    B, K, V = 64, 6, 3000
    zd = (2.5 * g.standard_normal((B, K, V))).astype(np.float32)
    zt = np.concatenate([0.9 * zd + g.standard_normal((B, K, V)), 2.5 * g.standard_normal((B, 1, V))], 1)
    kb = g.integers(0, K + 1, B)
    kb[:4] = 0
    b = _custom_batch(zd, zt.astype(np.float32), _draw_tokens(zd, 1.0, 1), 1.0, K=kb)
    _log("case ragged K_b with zeros")
    gpu = gpu_verify(b)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)
    assert np.all(gpu["accept_len"][:4] == 0)


def test_max_k_zero_batch_draws_bonus_only():
    g = np.random.default_rng(4)
    B, V = 32, 2000
    zt = g.standard_normal((B, 1, V)).astype(np.float32)
    b = _custom_batch(np.zeros((B, 0, V), np.float32), zt, np.zeros((B, 0)), 1.0)
    d = to_device(b)
    out = sv.sv_spec_verify(d["target"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                            d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                            max_k=0)
    torch.cuda.synchronize()
    o = ov.verify_batch(b)
    got = {k: v.cpu().numpy() for k, v in out.items()}
    assert compare_verify(b, got, o) <= flip_budget(o, b.num_draft)


def test_max_draft_length_and_temperatures():
    g = np.random.default_rng(5)
    B, K, V = 24, sv.SV_MAX_K, 513
    zd = (1.0 * g.standard_normal((B, K, V))).astype(np.float32)
    zt = np.concatenate([zd + 0.05 * g.standard_normal((B, K, V)), g.standard_normal((B, 1, V))], 1)
    T = np.array([0.3, 0.7, 1.0, 1.7] * 6, np.float32)
    toks = np.stack([_draw_tokens(zd[i:i + 1], float(T[i]), i)[0] for i in range(B)])
    b = _custom_batch(zd, zt.astype(np.float32), toks, T)
    _log("case max_k=16")
    gpu = gpu_verify(b)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)
    assert gpu["accept_len"].max() >= 8  # near-identical rows accept deep


def test_largest_vocabulary():
    g = np.random.default_rng(6)
    B, K, V = 2, 1, sv.SV_MAX_V
    zd = (2.0 * g.standard_normal((B, K, V))).astype(np.float32)
    zt = (2.0 * g.standard_normal((B, K + 1, V))).astype(np.float32)
    b = _custom_batch(zd, zt, _draw_tokens(zd, 1.0, 2), 1.0)
    b.u_accept[:] = 0.999  # force the residual path
    _log("case V=2^21")
    gpu = gpu_verify(b)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)
    assert np.all(gpu["accept_len"] == 0)


def test_identical_rows_accept_all_and_draw_bonus():
    g = np.random.default_rng(7)
    B, K, V = 40, 4, 5000
    z = (2.0 * g.standard_normal((B, K + 1, V))).astype(np.float32)
    b = _custom_batch(z[:, :K], z, _draw_tokens(z[:, :K], 1.0, 3), 1.0)
    gpu = gpu_verify(b)
    assert np.all(gpu["accept_len"] == K)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)


def test_disjoint_supports_and_neg_inf():
    g = np.random.default_rng(8)
    B, K, V = 40, 3, 4096
    zd = g.standard_normal((B, K, V)).astype(np.float32)
    zt = g.standard_normal((B, K + 1, V)).astype(np.float32)
    zd[:, :, V // 2:] = -np.inf
    zt[:, :, :V // 2] = -np.inf
    b = _custom_batch(zd, zt, _draw_tokens(np.where(np.isfinite(zd), zd, -1e30), 1.0, 4), 1.0)
    gpu = gpu_verify(b)
    assert np.all(gpu["accept_len"] == 0)
    assert np.all(gpu["out_tokens"][:, 0] >= V // 2)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)
    # a draft token the draft gives probability 0 is always accepted (ratio +inf)
    zd2 = g.standard_normal((B, K, V)).astype(np.float32)
    zd2[:, :, 0] = -np.inf
    zt2 = g.standard_normal((B, K + 1, V)).astype(np.float32)
    b2 = _custom_batch(zd2, zt2, np.zeros((B, K)), 1.0)
    gpu2 = gpu_verify(b2)
    assert np.all(gpu2["accept_len"] == K)
    o2 = ov.verify_batch(b2)
    assert compare_verify(b2, gpu2, o2) <= flip_budget(o2, b2.num_draft)


def test_greedy_ties_pick_lowest_index():
    g = np.random.default_rng(9)
    B, K, V = 32, 3, 3000
    zd = np.round(g.standard_normal((B, K, V)) * 2).astype(np.float32)  # many ties
    zt = np.round(g.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    zt[:, :, 17] = 50.0
    zt[:, :, 2900] = 50.0   # tie for the maximum, across segments
    toks = np.full((B, K), 17)
    toks[::2, 1] = 2900     # tied value, higher index: rejected
    b = _custom_batch(zd, zt, toks, 0.0, dtype="bf16")
    gpu = gpu_verify(b)
    o = ov.verify_batch(b)
    assert np.array_equal(gpu["accept_len"], o["accept_len"])
    assert np.array_equal(gpu["out_tokens"], o["out_tokens"])
    assert np.all(gpu["out_tokens"][::2, 1] == 17)


def test_broadcast_rows_stride_zero_starts():
    g = np.random.default_rng(10)
    K, V = 3, 2048
    zd = (2 * g.standard_normal((K, V))).astype(np.float32)
    zt = np.vstack([zd + g.standard_normal((K, V)), 2 * g.standard_normal((1, V))]).astype(np.float32)
    b = gen.broadcast_batch(zd, zt, 3000, seed=11)
    gpu = gpu_verify(b)
    o = ov.verify_batch(b, requests=np.arange(300))
    assert compare_verify(b, gpu, o, requests=np.arange(300)) <= flip_budget(o, b.num_draft[:300])


def test_deterministic_and_workspace_reuse():
    b3 = gen.make_batch("bf16_b256_k4_v128256_peaked", B=64)
    b1 = gen.make_batch("tiny_fp32_b4_k4_v1024", B=16)
    ws = sv.Workspace()
    first = gpu_verify(b3, workspace=ws, want_feature=True)
    mid = gpu_verify(b1, workspace=ws)
    again = gpu_verify(b3, workspace=ws, want_feature=True)
    fresh = gpu_verify(b1, workspace=sv.Workspace())
    for k in first:
        assert np.array_equal(first[k], again[k], equal_nan=True), k
    for k in mid:
        assert np.array_equal(mid[k], fresh[k], equal_nan=True), k


def test_long_rows_many_drafts():
    """8 drafts of 2^20 fp32 logits: 128 segments of 32 KiB per row, so the
    draw's last segment collects 1024 slice weights."""
    g = np.random.default_rng(12)
    B, K, V = 2, 8, 1 << 20
    zd = (2.0 * g.standard_normal((B, K, V))).astype(np.float32)
    zt = np.concatenate([zd + 0.3 * g.standard_normal((B, K, V)), g.standard_normal((B, 1, V))], 1)
    b = _custom_batch(zd, zt.astype(np.float32), _draw_tokens(zd, 1.0, 13), 1.0)
    _log("case K=8 V=2^20 fp32")
    gpu = gpu_verify(b, want_feature=True)
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o) <= flip_budget(o, b.num_draft)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("filtered", [False, True])
def test_residual_without_mass_draws_from_the_target(dtype, filtered):
    """A rejection whose residual (pt - pd)+ has no mass in the arithmetic.

    Target row = draft row except a slightly lower logit at the draft token
    d, whose probability is ~1e-15: every other token's pt - pd is then
    exactly 0 (the two normalisers agree to the last bit, the term at d being
    absorbed into the sums), and pt(d) < pd(d).  u_accept lies well above the
    ratio exp(-delta), so position 0 rejects; the residual is empty and the
    token is drawn from pt itself (the no-mass convention, parity unpinned).
    The oracle's binary64 normalisers agree too, so it takes the same branch:
    tokens are compared under the usual margins, and every token must be
    valid (0 <= tok < V, finite target logit)."""
    g = np.random.default_rng(21)
    B, K, V = 64, 1, 1024
    zd = g.standard_normal((B, K, V)).astype(np.float32)
    toks = g.integers(0, V, (B, K))
    delta = 1e-3 if dtype == "f32" else 0.125  # a step the element type can hold at -30
    for r in range(B):
        zd[r, 0, toks[r, 0]] = -30.0
    zt = np.concatenate([zd, g.standard_normal((B, 1, V)).astype(np.float32)], 1)
    for r in range(B):
        zt[r, 0, toks[r, 0]] = -30.0 - delta
    b = _custom_batch(zd, zt, toks, 1.0, dtype=dtype, seed=22)
    b.u_accept[:] = 0.9995  # above the ratio exp(-delta) <= 0.99901 in both element types: rejected
    _log(f"case residual without mass {dtype} filtered={filtered}")
    if filtered:
        d = to_device(b)
        out = sv.sv_spec_verify_filtered(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                         d["num_draft"], d["draft_tokens"], d["temperature"],
                                         torch.zeros(B, dtype=torch.int32, device="cuda"),
                                         torch.ones(B, dtype=torch.float32, device="cuda"), d["u_accept"],
                                         d["u_residual"], d["u_bonus"], max_k=b.max_k)
        torch.cuda.synchronize()
        gpu = {k: v.cpu().numpy() for k, v in out.items()}
    else:
        gpu = gpu_verify(b)
    assert np.all(gpu["accept_len"] == 0)
    tok = gpu["out_tokens"][:, 0]
    assert np.all((tok >= 0) & (tok < V)), tok
    zt_rows = gen.bf16_bits_to_f32(b.target) if dtype == "bf16" else b.target
    assert np.all(np.isfinite(zt_rows[b.target_row_start, tok]))
    o = ov.verify_batch(b)
    assert compare_verify(b, gpu, o, check_probs=not filtered) <= flip_budget(o, b.num_draft)
