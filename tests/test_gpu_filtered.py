"""GPU parity of filtered verification (sv_spec_verify_filtered) against the
oracle ``oracle.filtered`` (top-k / top-p readings F1-F5; [AV] sections
"Other features considered" and "Benchmarks" sample at temperature 1 with
top-p 0.95).

Rules: accept lengths, emitted tokens, labels and per-row kept counts are
exact for every request whose oracle decision margins (accept tests, the
draw's CDF position, every filtered row's top-p boundary) exceed 1e-5;
otherwise a mismatch is a counted within-margin flip.  Filtered
probabilities agree within the verification tolerances (1e-5 relative for
fp32 rows, 2e-3 for bf16)."""
import dataclasses

import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import MARGIN, TOL, rel_close, to_device
from oracle import filtered as of
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]

DEV = torch.device("cuda")


def _log(msg):
    print(msg, flush=True)


def gpu_filtered(b, d=None, workspace=None, stride_cut=False):
    d = to_device(b) if d is None else d
    if stride_cut:
        d["draft"] = d["draft"][:, :b.V]
        d["target"] = d["target"][:, :b.V]
    tk = torch.from_numpy(np.ascontiguousarray(b.top_k, np.int32)).to(DEV)
    tp = torch.from_numpy(np.ascontiguousarray(b.top_p, np.float32)).to(DEV)
    out = sv.sv_spec_verify_filtered(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                     d["num_draft"], d["draft_tokens"], d["temperature"], tk, tp, d["u_accept"],
                                     d["u_residual"], d["u_bonus"], max_k=b.max_k, workspace=workspace)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def oracle_filtered(b, requests=None):
    if b.draft.shape[1] != b.V:
        b = dataclasses.replace(b, draft=b.draft[:, :b.V], target=b.target[:, :b.V])
    return of.verify_batch_filtered(b, b.top_k, b.top_p, requests)


def compare_filtered(b, g, o, requests=None):
    """The parity rules above; returns the number of within-margin flips."""
    idx = np.arange(b.B) if requests is None else np.asarray(requests)
    tol = TOL[b.dtype]
    mk = b.max_k
    flips = 0
    for r, q in enumerate(idx):
        k = int(b.num_draft[q])
        a_o = int(o["accept_len"][r])
        toks_o = o["out_tokens"][r, :a_o + 1]
        a_g = int(g["accept_len"][q])
        toks_g = g["out_tokens"][q, :a_g + 1]
        fm = o["filter_margin"][r]
        tight_filter = (fm <= MARGIN).any()
        # kept counts and filtered probabilities do not depend on the draw
        rows = np.r_[np.arange(k), mk + np.arange(k + 1)]
        exact = fm[rows] > MARGIN
        assert np.array_equal(g["kept"][q, rows][exact], o["kept"][r, rows][exact]), (
            q, g["kept"][q].tolist(), o["kept"][r].tolist())
        unread = np.setdiff1d(np.arange(2 * mk + 1), rows)
        assert np.all(g["kept"][q, unread] == -1), (q, g["kept"][q].tolist())
        if not tight_filter:
            okd = rel_close(g["p_draft"][q, :k], o["p_draft"][r, :k], tol)
            okt = rel_close(g["p_target"][q, :k], o["p_target"][r, :k], tol)
            assert okd.all(), (q, g["p_draft"][q, :k], o["p_draft"][r, :k])
            assert okt.all(), (q, g["p_target"][q, :k], o["p_target"][r, :k])
        assert np.isnan(g["p_target"][q, k:]).all()
        same = a_g == a_o and np.array_equal(toks_g, toks_o)
        if not same:
            m = o["accept_margin"][r, :min(a_o + 1, k)]
            tight = (m <= MARGIN).any() or o["cdf_margin"][r] <= MARGIN or tight_filter
            assert tight, (f"request {q}: gpu a={a_g} tokens={toks_g.tolist()} vs oracle a={a_o} "
                           f"tokens={toks_o.tolist()} margins={m.tolist()} cdf={o['cdf_margin'][r]} "
                           f"filter={fm.tolist()}")
            flips += 1
            continue
        assert np.all(g["out_tokens"][q, a_g + 1:] == -1), q
        assert np.array_equal(g["labels"][q], o["labels"][r]), (q, g["labels"][q], o["labels"][r])
    return flips


@pytest.mark.parametrize("name,B", [("fp32_b32_k4_v1024_filter_mix", None), ("bf16_b64_k5_v32000_filter_mix", None)])
def test_parity_filter_mix(name, B):
    b = gen.make_batch(name, B=B)
    _log(f"case filtered {name}")
    g = gpu_filtered(b)
    flips = compare_filtered(b, g, oracle_filtered(b))
    assert flips <= 1


def test_parity_benchmark_batch_top_p_095_sampled():
    """The benchmark's batch (B=256, K=4, V=128256 bf16) at top-p 0.95: every
    request checked for validity, a sample of requests against the oracle."""
    b = gen.make_batch("bf16_b256_k4_v128256_peaked_topp95", trial=0)
    _log("case filtered bench batch")
    g = gpu_filtered(b)
    K = b.num_draft
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= K))
    for q in range(b.B):
        a = int(g["accept_len"][q])
        assert np.array_equal(g["out_tokens"][q, :a], b.draft_tokens[q, :a])
        assert 0 <= g["out_tokens"][q, a] < b.V and np.all(g["out_tokens"][q, a + 1:] == -1)
        assert np.all(g["kept"][q] >= 1)
    sample = np.arange(0, b.B, 37)
    flips = compare_filtered(b, g, oracle_filtered(b, sample), sample)
    assert flips <= 1


def _batch(zd, zt, toks, T, top_k, top_p, dtype="f32", K=None, seed=0, stride_pad=0):
    """Batch from explicit fp32 rows zd [B, K, V], zt [B, K+1, V]."""
    B, maxk, V = zd.shape
    g = np.random.default_rng(seed)
    K = np.full(B, maxk, np.int32) if K is None else np.asarray(K, np.int32)
    stride = V + stride_pad
    d = np.zeros((max(B * maxk, 1), stride), np.float32)
    t = np.zeros((B * (maxk + 1), stride), np.float32)
    d[:B * maxk, :V] = zd.reshape(-1, V)
    t[:, :V] = zt.reshape(-1, V)
    if dtype == "bf16":
        d, t = gen.f32_to_bf16_bits(d), gen.f32_to_bf16_bits(t)
    bc = lambda x, dt: np.broadcast_to(np.asarray(x, dt), (B,)).copy()
    return gen.Batch("custom", B, V, maxk, dtype, d, np.arange(B, dtype=np.int64) * maxk, t,
                     np.arange(B, dtype=np.int64) * (maxk + 1), K, np.asarray(toks, np.int32).reshape(B, maxk),
                     bc(T, np.float32), g.random((B, maxk), dtype=np.float32), g.random(B, dtype=np.float32),
                     g.random(B, dtype=np.float32), np.array([1.0] + [0.0] * maxk, np.float32),
                     top_k=bc(top_k, np.int32), top_p=bc(top_p, np.float32))


def _draws(zd, T, seed):
    g = np.random.default_rng(seed)
    B, K, V = zd.shape
    return np.argmax(zd / T - np.log(g.standard_exponential((B, K, V))), axis=2)


def _run(b, **kw):
    g = gpu_filtered(b, stride_cut=b.draft.shape[1] != b.V, **kw)
    return g, oracle_filtered(b)


@pytest.mark.parametrize("V,dtype,pad,top_k,top_p", [
    (1000, "f32", 0, 0, 0.9), (1031, "bf16", 0, 20, 1.0), (1000, "bf16", 3, 50, 0.8), (1001, "f32", 1, 3, 0.99),
    (5, "f32", 0, 2, 1.0), (7, "bf16", 1, 0, 0.6), (1, "f32", 0, 1, 0.5), (2, "bf16", 0, 1, 1.0),
    (40000, "bf16", 5, 0, 0.95), (16385, "f32", 0, 700, 0.9), (70001, "f32", 2, 0, 0.3)])
def test_ragged_and_misaligned_rows(V, dtype, pad, top_k, top_p):
    g = np.random.default_rng(V + pad)
    B, K = 6, 3
    zd = g.normal(0, 2.0, (B, K, V)).astype(np.float32)
    zt = np.concatenate([zd + g.normal(0, 1.0, zd.shape), g.normal(0, 2.0, (B, 1, V))], axis=1).astype(np.float32)
    b = _batch(zd, zt, _draws(zd, 1.0, 1), 1.0, top_k, top_p, dtype=dtype, K=[0, 1, 2, 3, 3, 2], stride_pad=pad)
    _log(f"case filtered rows V={V} {dtype} pad={pad} k={top_k} p={top_p}")
    gout, o = _run(b)
    assert compare_filtered(b, gout, o) <= 1


def test_filters_off_and_greedy_requests_are_plain_verification():
    b = gen.make_batch("fp32_b32_k4_v1024_filter_mix")
    b = dataclasses.replace(b, top_k=np.where(np.arange(b.B) % 2 == 0, 0, b.V).astype(np.int32),
                            top_p=np.where(np.arange(b.B) % 3 == 0, 1.0, 7.0).astype(np.float32))
    _log("case filtered off")
    gout, o = _run(b)
    assert compare_filtered(b, gout, o) == 0
    assert np.all(gout["kept"] == -1)
    from oracle import verify as ov
    plain = ov.verify_batch(b)
    np.testing.assert_array_equal(o["accept_len"], plain["accept_len"])


def test_top1_is_greedy_and_tiny_top_p_keeps_the_maximum():
    g = np.random.default_rng(11)
    B, K, V = 8, 4, 3000
    zd = g.normal(0, 2, (B, K, V)).astype(np.float32)
    zt = g.normal(0, 2, (B, K + 1, V)).astype(np.float32)
    top_d = np.argmax(zd, axis=2)
    for q in range(B):
        for i in range(K):
            if (q + i) % 3:
                zt[q, i, top_d[q, i]] = zt[q, i].max() + 1.0  # the target agrees at some positions
    b = _batch(zd, zt, top_d, 1.0, 1, 1.0)
    _log("case filtered top-1")
    gout, o = _run(b)
    assert compare_filtered(b, gout, o) == 0
    # the greedy rule: accept while the draft is the target argmax, then emit that argmax
    for q in range(B):
        a = int(gout["accept_len"][q])
        top_t = np.argmax(zt[q], axis=1)
        assert all(top_d[q, i] == top_t[i] for i in range(a))
        assert gout["out_tokens"][q, a] == top_t[a]
    assert np.all(gout["kept"][:, :K] == 1) and np.all(gout["kept"][:, K:] == 1)
    b2 = dataclasses.replace(b, top_k=np.zeros(B, np.int32), top_p=np.full(B, 1e-6, np.float32))
    gout2, o2 = _run(b2)
    assert compare_filtered(b2, gout2, o2) == 0
    assert np.all(gout2["kept"] == 1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ties_uniform_rows_neg_inf_and_signed_zeros(dtype):
    V, K = 2048, 2
    zd = np.zeros((4, K, V), np.float32)
    zt = np.zeros((4, K + 1, V), np.float32)
    # request 0: uniform rows (one value: everything kept); 1: half the
    # vocabulary at -inf; 2: values on a coarse grid (many ties at the
    # boundary); 3: -0, +0 and tiny magnitudes around the boundary
    zd[1, :, V // 2:] = -np.inf
    zt[1, :, : V // 3] = -np.inf
    g = np.random.default_rng(5)
    zd[2] = np.round(g.normal(0, 2, (K, V)) * 2) / 2
    zt[2] = np.round(g.normal(0, 2, (K + 1, V)) * 2) / 2
    zd[3] = g.choice(np.array([-0.0, 0.0, 1e-30, -1e-30, 1e-3, -1e-3, 2.0], np.float32), (K, V))
    zt[3] = g.choice(np.array([-0.0, 0.0, 1e-30, -1e-30, 1e-3, -1e-3, 2.0], np.float32), (K + 1, V))
    toks = np.array([[3, 7], [1, 2], [int(np.argmax(zd[2, 0])), 5], [0, 9]])
    for top_k, top_p in [(0, 0.5), (1500, 1.0), (100, 0.7)]:
        b = _batch(zd, zt, toks, 1.0, top_k, top_p, dtype=dtype, seed=top_k)
        _log(f"case filtered ties {dtype} k={top_k} p={top_p}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) == 0
    b = _batch(zd, zt, toks, 1.0, 0, 0.5, dtype=dtype)
    gout, _ = _run(b)
    assert np.all(gout["kept"][0] == V)


def test_key_window_edges_bf16():
    """bf16 rows select level 0 by exact key counts in the 1024 keys below
    the row maximum's: request 0 has its maximum at +-0 (both zeros one
    key); request 1 puts tokens on the lowest key of the window and on the
    first key below it, so that top-k 600 ends in the window and top-k 601
    one key below it (the search continues over the keys below, by weight
    cells, then by key digits); requests 2 and 3 have 16384-token segments
    whose maxima lie far apart, one segment without a finite logit, the row
    maximum in the first or the last segment."""
    g = np.random.default_rng(41)
    B, K, V = 4, 2, 65536
    seg = 16384
    zd = np.zeros((B, K, V), np.float32)
    zt = np.zeros((B, K + 1, V), np.float32)
    zero_vals = np.array([-0.0, 0.0, -0.5, -3.0], np.float32)
    zd[0] = g.choice(zero_vals, (K, V), p=[0.3, 0.3, 0.2, 0.2])
    zt[0] = g.choice(zero_vals, (K + 1, V), p=[0.3, 0.3, 0.2, 0.2])
    lowest_in, first_below = 0.003936767578125, 0.00390625  # bf16 keys 0xbb81, 0xbb80 below 1.0's 0xbf80
    edge = np.full(V, -1.0, np.float32)
    edge[:100], edge[100:300], edge[300:600], edge[600:1000] = 1.0, 0.5, lowest_in, first_below
    for r in range(K):
        zd[1, r] = g.permutation(edge)
    for r in range(K + 1):
        zt[1, r] = g.permutation(edge)
    offs = np.repeat(np.array([0.0, -30.0, 0.0, -3.0], np.float32), seg)
    for q in (2, 3):
        zd[q] = g.normal(0, 1.0, (K, V)) + offs
        zt[q] = g.normal(0, 1.0, (K + 1, V)) + offs
        zd[q, :, 2 * seg:3 * seg] = -np.inf
        zt[q, :, 2 * seg:3 * seg] = -np.inf
    zd[3, :, 3 * seg:] += 10.0
    zt[3, :, 3 * seg:] += 10.0
    toks = np.array([[1, 2], [3, 4], [5, 6], [3 * seg + 1, 3 * seg + 2]])
    zeros = lambda rows: int(np.sum(gen.bf16_bits_to_f32(rows) == 0.0, axis=1)[0])
    # (0, 0.95), (300, 0.99), (40000, 0.95): thresholds below the window in
    # requests 0, 2 and 3 (N(0, 1) segments), the last with both searches
    # continuing there by weight cells
    for top_k, top_p in [(0, 0.5), (0, 0.95), (600, 1.0), (601, 1.0), (300, 0.99), (40000, 0.95)]:
        b = _batch(zd, zt, toks, 1.0, top_k, top_p, dtype="bf16", seed=top_k)
        _log(f"case filtered key window k={top_k} p={top_p}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) == 0
        if (top_k, top_p) == (600, 1.0):
            assert np.all(gout["kept"][1] == 600)
        if (top_k, top_p) == (601, 1.0):
            assert np.all(gout["kept"][1] == 1000)
        if (top_k, top_p) == (0, 0.5):  # the zeros, of both signs, and nothing else
            for r in range(K + 1):
                assert gout["kept"][0, K + r] == zeros(b.target[(K + 1) * 0 + r:(K + 1) * 0 + r + 1])


def test_long_runs_of_equal_logits_above_the_boundary():
    """60000 equal logits in one level-0 bin above the top-p boundary: that
    bin's fraction sum over the row needs more than 32 bits (a 32-bit sum
    wraps and corrupts the mass above the boundary)."""
    V, K = 128000, 1
    zd = np.full((2, K, V), -0.4, np.float32)
    zt = np.full((2, K + 1, V), -0.4, np.float32)
    zd[:, :, :60000] = 0.6
    zt[:, :, 30000:90000] = 0.6
    toks = np.array([[5], [100000]])
    for dtype in ("f32", "bf16"):
        b = _batch(zd, zt, toks, 1.0, 0, 0.99, dtype=dtype)
        _log(f"case filtered equal runs {dtype}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) == 0
        assert np.all(gout["kept"][:, [0, 1, 2]] == V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segment_maxima_far_apart(dtype):
    """Segments whose maxima lie hundreds of level-0 bins apart: some
    wholly in the last bin (fp32) or far below the row's key window (bf16),
    one without a finite logit, and in request 1 the row maximum outside the
    first segment."""
    g = np.random.default_rng(23)
    B, K, V = 4, 2, 131072
    seg = 8192 if dtype == "f32" else 16384  # elements per 32 KiB segment
    offs = -3.0 * (np.arange(V) // seg)  # 16 segments, each ~69 bins below the previous at T = 1
    zd = (g.normal(0, 1.0, (B, K, V)) + offs).astype(np.float32)
    zt = (g.normal(0, 1.0, (B, K + 1, V)) + offs).astype(np.float32)
    zd[:, :, 3 * seg:4 * seg] = -np.inf
    zt[1, :, :seg] -= 40.0  # request 1: the maxima in the second segment
    for top_k, top_p, T in [(0, 0.999, 1.0), (20000, 1.0, 1.0), (0, 0.9999999, 0.25), (5000, 0.99, 4.0)]:
        b = _batch(zd, zt, _draws(zd, T, 7), T, top_k, top_p, dtype=dtype)
        _log(f"case filtered far segments {dtype} k={top_k} p={top_p} T={T}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) <= 1


def test_boundary_among_dense_keys_near_zero():
    """bf16 logits within a few hundredths of zero: the level-0 cell of the
    boundary holds thousands of distinct keys, so the first key level
    leaves the search open and the second one, over the segments of the
    rows still searching only, finishes it; rows of ordinary spread in the
    same batch finish at the first key level."""
    g = np.random.default_rng(31)
    B, K, V = 6, 2, 40000
    zd = g.normal(0, 0.01, (B, K, V)).astype(np.float32)
    zt = g.normal(0, 0.01, (B, K + 1, V)).astype(np.float32)
    zd[3:] *= 300.0
    zt[3:] *= 300.0
    c8 = 8.0 * np.log2(np.e)
    for top_k, top_p in [(0, 0.5), (V // 3, 1.0), (V // 2, 0.3)]:
        b = _batch(zd, zt, _draws(zd, 1.0, 5), 1.0, top_k, top_p, dtype="bf16")
        _log(f"case filtered dense keys k={top_k} p={top_p}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) <= 1
        # the claim above: a boundary cell with more distinct keys than one
        # 8-bit key level resolves
        rows = gen.bf16_bits_to_f32(b.target[:K + 1])
        z = np.sort(rows[0])[::-1]
        t = z[int(o["kept"][0, K]) - 1]
        cell = np.floor(rows[0] * np.float32(c8))
        assert len(np.unique(rows[0][cell == np.floor(np.float32(t) * np.float32(c8))])) > 256


def test_temperatures_max_draft_length_and_largest_vocabulary():
    g = np.random.default_rng(2)
    B, K, V = 3, 16, 4096
    zd = g.normal(0, 3, (B, K, V)).astype(np.float32)
    zt = (np.concatenate([zd, g.normal(0, 3, (B, 1, V))], axis=1) + g.normal(0, 0.5, (B, K + 1, V))).astype(
        np.float32)
    for T in (0.3, 1.0, 2.5):
        b = _batch(zd, zt, _draws(zd, T, 3), T, 40, 0.9, dtype="bf16")
        _log(f"case filtered K=16 T={T}")
        gout, o = _run(b)
        assert compare_filtered(b, gout, o) <= 1
    V = sv.SV_MAX_V
    zd = g.normal(0, 2, (1, 1, V)).astype(np.float32)
    zt = g.normal(0, 2, (1, 2, V)).astype(np.float32)
    for dtype in ("f32", "bf16"):  # bf16: 128 segments per row, more than a wave's lanes
        b = _batch(zd, zt, _draws(zd, 1.0, 4), 1.0, 0, 0.95, dtype=dtype)
        _log(f"case filtered V=2^21 {dtype}")
        gout, o = _run(b)
        # at this vocabulary every token's probability is ~1e-6, so the draw's
        # CDF margin is below 1e-5 by construction: a differing token is a
        # within-margin flip; kept counts and probabilities are still exact
        assert compare_filtered(b, gout, o) <= 1


def test_deterministic_and_workspace_reuse():
    b = gen.make_batch("bf16_b64_k5_v32000_filter_mix", B=24)
    small = gen.make_batch("fp32_b32_k4_v1024_filter_mix", B=9)
    ws = sv.Workspace()
    _log("case filtered determinism")
    d = to_device(b)
    g1 = gpu_filtered(b, d=d, workspace=ws)
    gs = gpu_filtered(small, workspace=ws)
    g2 = gpu_filtered(b, d=d, workspace=ws)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k], err_msg=k)
    assert compare_filtered(small, gs, oracle_filtered(small)) <= 1


def test_max_k_zero_draws_bonus_from_filtered_target_rows():
    """No drafts: every request draws its bonus token from target row 0,
    filtered; the kept counts cover that one row."""
    g = np.random.default_rng(31)
    B, V = 12, 3000
    zt = g.normal(0, 2.0, (B, 1, V)).astype(np.float32)
    zd = np.zeros((B, 0, V), np.float32)
    b = _batch(zd, zt, np.zeros((B, 0), np.int32), 1.0, 0, 0.8)
    b = dataclasses.replace(b, top_k=np.array([0, 5, 0, 40] * 3, np.int32),
                            top_p=np.array([0.8, 1.0, 0.5, 0.9] * 3, np.float32))
    _log("case filtered max_k=0")
    gout, o = _run(b)
    assert compare_filtered(b, gout, o) == 0
    assert gout["out_tokens"].shape == (B, 1) and np.all(gout["accept_len"] == 0)
    assert np.all(gout["kept"][:, 0] >= 1)


def test_greedy_batch_with_filters_is_unfiltered():
    b = gen.make_batch("fp32_b32_k4_v1024_filter_mix")
    b = dataclasses.replace(b, temperature=np.zeros(b.B, np.float32))
    _log("case filtered all greedy")
    gout, o = _run(b)
    assert compare_filtered(b, gout, o) == 0
    assert np.all(gout["kept"] == -1)
    assert np.all(np.isnan(gout["p_draft"]))
