"""Verification captured in a HIP graph and replayed: each replay must give
what an eager call on the same inputs gives, with eager calls sharing the
workspace and the inputs changed in place between replays (the kernels keep
hand-off state in the workspace; nothing may carry over from one replay to
the next)."""
import numpy as np
import pytest
import torch

import draft_token_verification_spec_amd as sv
from gpu_harness import to_device
from synth import gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


def _call(b, d, ws, out):
    return sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                             d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                             max_k=b.max_k, av_params=d["av_params"], want_feature=True, workspace=ws, out=out)


def _snapshot(out):
    return {k: v.cpu().numpy().copy() for k, v in out.items()}


def _same(x, y):
    for k in x:
        np.testing.assert_array_equal(x[k], y[k], err_msg=k)


@pytest.mark.parametrize("workload", ["bf16_b64_k5_v32000", "fp32_b1024_k1to3_v129280_greedy_mix"])
def test_graph_replays_match_eager(workload):
    B = 64 if workload.startswith("bf16") else 48
    b = gen.make_batch(workload, trial=2, B=B)
    d = to_device(b)
    print(f"case graph {workload} B={B}", flush=True)
    ws = sv.Workspace()
    eager_out, graph_out = {}, {}
    _call(b, d, ws, eager_out)  # allocates the outputs and sizes the workspace
    _call(b, d, ws, graph_out)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _call(b, d, ws, graph_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    for rep in range(4):
        if rep:  # new uniforms in place: the replay must not reuse anything of the last one
            d["u_accept"].copy_(torch.from_numpy(rng.random(d["u_accept"].shape, dtype=np.float32)))
            d["u_residual"].copy_(torch.from_numpy(rng.random(B, dtype=np.float32)))
            d["u_bonus"].copy_(torch.from_numpy(rng.random(B, dtype=np.float32)))
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(graph_out)
        _call(b, d, ws, eager_out)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        _same(got, _snapshot(eager_out))


def test_filtered_verification_graph_replays_match_eager():
    """The filtered call's search states and histograms are rewritten by every
    call before they are read, so replays on a workspace shared with eager
    calls equal the eager result."""
    b = gen.make_batch("bf16_b64_k5_v32000_filter_mix", trial=1, B=32)
    d = to_device(b)
    tk = torch.from_numpy(b.top_k).cuda()
    tp = torch.from_numpy(b.top_p).cuda()
    print("case graph filtered", flush=True)
    ws = sv.Workspace()

    def call(out):
        return sv.sv_spec_verify_filtered(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                          d["num_draft"], d["draft_tokens"], d["temperature"], tk, tp,
                                          d["u_accept"], d["u_residual"], d["u_bonus"], max_k=b.max_k, workspace=ws,
                                          out=out)

    eager_out, graph_out = {}, {}
    call(eager_out)
    call(graph_out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(graph_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for rep in range(4):
        if rep:
            d["u_accept"].copy_(torch.from_numpy(rng.random(d["u_accept"].shape, dtype=np.float32)))
            d["u_residual"].copy_(torch.from_numpy(rng.random(b.B, dtype=np.float32)))
            tp.copy_(torch.from_numpy(rng.choice(np.array([1.0, 0.9, 0.7], np.float32), b.B)))
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(graph_out)
        call(eager_out)
        torch.cuda.synchronize()
        _same(got, _snapshot(eager_out))


def test_segmented_distillation_gradient_graph_replays_match_eager():
    """The segmented gradient sums each position's loss through an arrival
    counter that every call leaves at zero: replays interleaved with eager
    calls on the same workspace equal the eager result."""
    b = gen.make_batch("bf16_b64_k5_v32000", trial=5, B=24)
    d = to_device(b)
    print("case graph distillation", flush=True)
    ws = sv.Workspace()
    w = torch.linspace(1.0, 0.5, b.max_k, device="cuda")
    vout = {}

    def verify():
        sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                          d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                          max_k=b.max_k, want_feature=True, workspace=ws, out=vout)

    def tts(out):
        return sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                              d["temperature"], w, b.max_k, 0.0, verify_workspace=ws, out=out)

    eager_out, graph_out = {}, {}
    verify()
    tts(eager_out)
    tts(graph_out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            verify()
            tts(graph_out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.float().cpu().numpy().copy() for k, v in graph_out.items()}
        verify()
        tts(eager_out)
        torch.cuda.synchronize()
        want = {k: v.float().cpu().numpy().copy() for k, v in eager_out.items()}
        for k in want:
            np.testing.assert_array_equal(np.nan_to_num(got[k], nan=-7.0), np.nan_to_num(want[k], nan=-7.0), err_msg=k)
