"""The largest batch the library accepts (SV_MAX_B requests) at a small
vocabulary: the verification with the estimator's feature and score, the
scoring pass with its survival prune, and the segmented distillation
gradient on the verification's workspace (one arrival counter per request
slot, so every slot of the arena is used).  Sampled requests against the
oracle under the parity rules; properties that hold at any size for every
request."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import compare_verify, compare_scores, flip_budget, to_device
from oracle import av as oav
from oracle import tts as ot
from oracle import verify as ov
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]

DEV = torch.device("cuda")


def _batch(seed=41):
    B, K, V = sv.SV_MAX_B, 2, 64
    g = np.random.default_rng(seed)
    zd = g.normal(0.0, 1.5, (B, K, V)).astype(np.float32)
    zt = np.concatenate([zd + g.normal(0.0, 0.7, zd.shape), g.normal(0.0, 1.5, (B, 1, V))], axis=1).astype(np.float32)
    T = np.where(np.arange(B) % 4 == 0, 0.0, np.where(np.arange(B) % 4 == 1, 0.7, 1.0)).astype(np.float32)
    K_b = (np.arange(B) % 3).astype(np.int32)  # 0, 1, 2 drafts
    gumbel = -np.log(g.standard_exponential((B, K, V)))
    toks = np.argmax(zd / np.where(T > 0, T, 1.0)[:, None, None] + gumbel, axis=2).astype(np.int32)
    d = zd.reshape(-1, V)
    t = zt.reshape(-1, V)
    b = gen.Batch("max_batch", B, V, K, "f32", d, np.arange(B, dtype=np.int64) * K, t,
                  np.arange(B, dtype=np.int64) * (K + 1), K_b, toks, T, g.random((B, K), dtype=np.float32),
                  g.random(B, dtype=np.float32), g.random(B, dtype=np.float32),
                  np.array([0.5, 0.3, -0.2], np.float32))
    return b


def _sample(B, n, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, 2, 3, B // 2, B - 3, B - 2, B - 1], g.choice(B, n, replace=False)]))


def test_largest_batch_verification_scoring_and_gradient():
    b = _batch()
    B, K, V = b.B, b.max_k, b.V
    print(f"case max batch B={B} K={K} V={V}", flush=True)
    d = to_device(b)
    ws = sv.Workspace()
    params = torch.from_numpy(b.av_params).to(DEV)
    g = sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                          d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                          max_k=K, av_params=params, want_feature=True, workspace=ws)
    sc = sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], params, max_k=K,
                        prune_threshold=0.3, workspace=ws)
    w = torch.tensor([1.0, 0.5], device=DEV)
    tg = sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                        d["temperature"], w, K, 0.0, verify_workspace=ws)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in g.items()}
    sc = {k: v.cpu().numpy() for k, v in sc.items()}
    loss = tg["loss"].cpu().numpy()

    # every request: accept lengths within [0, K_b], the emitted prefix is the
    # accepted drafts, the emitted token a vocabulary index, then -1; labels
    # 1 up to the accept length, 0 at a rejection, -1 after
    a = g["accept_len"]
    assert np.all((a >= 0) & (a <= b.num_draft))
    pos = np.arange(K + 1)[None, :]
    prefix = pos < a[:, None]
    drafts = np.concatenate([b.draft_tokens, np.full((B, 1), -1, np.int32)], axis=1)
    assert np.all(np.where(prefix, g["out_tokens"] == drafts, True))
    at = np.take_along_axis(g["out_tokens"], a[:, None].astype(np.int64), axis=1)[:, 0]
    assert np.all((at >= 0) & (at < V))
    assert np.all(np.where(pos > a[:, None], g["out_tokens"] == -1, True))
    lab = g["labels"]
    p2 = np.arange(K)[None, :]
    want = np.where(p2 < a[:, None], 1, np.where((p2 == a[:, None]) & (a[:, None] < b.num_draft[:, None]), 0, -1))
    assert np.array_equal(lab, want.astype(np.int8))
    # the survival prune keeps a prefix of the submitted drafts
    assert np.all((sc["num_kept"] >= 0) & (sc["num_kept"] <= b.num_draft))

    # sampled requests against the oracle
    idx = _sample(B, 3000, 7)
    o = ov.verify_batch(b, requests=idx)
    flips = compare_verify(b, g, o, requests=idx)
    assert flips <= flip_budget(o, b.num_draft[idx])
    s = oav.av_score_batch(b, threshold=0.3, requests=idx)
    compare_scores(b, g["av_feature"], g["av_score"], s, requests=idx)
    compare_scores(b, sc["feature"], sc["score"], s, requests=idx)
    # kept counts: exact wherever no survival lies within 1e-5 of the threshold
    near = np.nanmin(np.abs(np.nan_to_num(s["survival"], nan=1.0) - 0.3), axis=1) <= 1e-5
    assert np.array_equal(sc["num_kept"][idx][~near], s["num_kept"][~near])
    for r in idx[:400]:
        k_b = int(b.num_draft[r])
        T = float(b.temperature[r])
        for k in range(k_b):
            _, lref = ot.position(b.draft[r * K + k], b.target[r * (K + 1) + k], None, T, float(w[k]), 0.0)
            assert loss[r, k] == pytest.approx(lref, rel=1e-4, abs=1e-6), (r, k)
        assert np.all(np.isnan(loss[r, k_b:]))


def test_largest_batch_filtered():
    """Filtered verification at the largest batch: top-k / top-p mixed per
    request (some requests unfiltered, a quarter greedy)."""
    import dataclasses

    from test_gpu_filtered import compare_filtered, gpu_filtered, oracle_filtered

    b = _batch(seed=43)
    B = b.B
    r = np.arange(B)
    b = dataclasses.replace(b, top_k=np.array([0, 5, 0, 20, 3], np.int32)[r % 5],
                            top_p=np.array([0.9, 1.0, 0.5, 0.95, 1.0], np.float32)[r % 5])
    print(f"case max batch filtered B={B}", flush=True)
    g = gpu_filtered(b)
    a = g["accept_len"]
    assert np.all((a >= 0) & (a <= b.num_draft))
    at = np.take_along_axis(g["out_tokens"], a[:, None].astype(np.int64), axis=1)[:, 0]
    assert np.all((at >= 0) & (at < b.V))
    # kept counts: -1 where a row is not filtered or not read, else 1..V
    kept = g["kept"]
    assert np.all((kept == -1) | ((kept >= 1) & (kept <= b.V)))
    idx = _sample(B, 2000, 11)
    o = oracle_filtered(b, idx)
    assert compare_filtered(b, g, o, requests=idx) <= 2
