#!/usr/bin/env python3
"""Throughput of one verification step on one MI355X.

A step is one pass of the whole hot path over one batch already resident in
HBM: ``sv_spec_verify`` (softmax statistics of every draft and target row,
accept tests, first-rejection scan, residual or bonus sample, plus the
estimator feature and score of every draft row from the same pass) followed
by ``sv_av_fit_step`` (one damped IRLS step over the batch's labels).

Default workload: B=256 requests, K=4 drafts, V=128256, bf16 logits
(``bf16_b256_k4_v128256_peaked``).  Several independently drawn input sets
rotate between steps so that no step reads rows the previous one left in the
256 MB Infinity Cache.

Prints one JSON line: positions/s over the timed steps, the roofline of the
dominant kernel - the statistics kernel, which reads every logit once
(algorithmic HBM bytes per launch / its mean duration from HIP events on the
launching stream, against the 8 TB/s HBM3E peak) - with the whole
verification call (statistics kernel + verdict and draw kernel) beside it,
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec at B=256,K=4,V=128256 bf16; achieved HBM GB/s"
PEAK_HBM_GBS = 8000.0


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_b256_k4_v128256_peaked")
    p.add_argument("--rotate", type=int, default=3, help="input sets cycled between steps")
    p.add_argument("--graph", type=int, default=1, help="replay the steps from a captured HIP graph")
    p.add_argument("--kernel", choices=["resident", "streaming", "auto"], default="auto",
                   help="verification kernel (sv_set_verify_kernel)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="per-launch HBM bytes measured with rocprofv3 counters (optional)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, copy a MIB-sized device buffer 3 times (reference for HBM counters)")
    p.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                        "rocprofv3 pass (run with --copy-calibration) into per-launch HBM bytes, print them and "
                        "store them in --traffic")
    return p.parse_args()


def summarize_counters(args):
    """Per-launch HBM bytes of the library's kernels from two rocprofv3
    counter passes.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled
    by what they read for the calibration copy of known size (the largest
    copyBuffer dispatches: the copy reads and writes --copy-calibration MiB)."""
    import csv
    import re

    per = {}
    scale = {}
    for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), args.counters):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        top = max(copies)
        cal = [v for v in copies if v > 0.9 * top]
        mib = args.copy_calibration or 512
        scale[counter] = mib * 1024.0 / (sum(cal) / len(cal))
        for r in rows:
            m = re.search(r"sv::(?:\(anonymous namespace\)::)?(\w+)", r["Kernel_Name"])
            if m and "copyBuffer" not in r["Kernel_Name"]:
                per.setdefault(m.group(1), {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    out = {}
    for k, d in sorted(per.items()):
        f = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"]) * scale["FETCH_SIZE"] * 1024
        w = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"]) * scale["WRITE_SIZE"] * 1024
        out[k] = {"dispatches": len(d["FETCH_SIZE"]), "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
                  "bytes_per_launch": f + w}
        print(f"{k:16s} {len(d['FETCH_SIZE']):3d} dispatches  fetch {f / 1e6:9.2f} MB  write {w / 1e6:8.2f} MB")
    print(f"scales: FETCH_SIZE x{scale['FETCH_SIZE']:.5f}, WRITE_SIZE x{scale['WRITE_SIZE']:.5f}")
    rec = {"workload": args.workload, "kernel": "stats_kernel",
           "bytes_per_launch": out["stats_kernel"]["bytes_per_launch"],
           "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"], "kernels": out,
           "kernel_source_sha256": kernel_source_hash()}
    with open(args.traffic, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


def to_device(batch, dev):
    import numpy as np
    import torch

    def rows(a):
        if batch.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)
    return dict(draft=rows(batch.draft), draft_row_start=t(batch.draft_row_start, torch.int64),
                target=rows(batch.target), target_row_start=t(batch.target_row_start, torch.int64),
                num_draft=t(batch.num_draft, torch.int32), draft_tokens=t(batch.draft_tokens, torch.int32),
                temperature=t(batch.temperature, torch.float32), u_accept=t(batch.u_accept, torch.float32),
                u_residual=t(batch.u_residual, torch.float32), u_bonus=t(batch.u_bonus, torch.float32))


def kernel_source_hash() -> str:
    """sha256 over the sources the verification kernels are built from, to
    tell whether stored counter measurements still describe them."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_spec_amd", "csrc")
    for name in ("stream.hip", "sv_device.hpp", "sv_internal.hpp"):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def cpu_baseline(batch, budget_s):
    """The oracle, untuned, on the requests of input set 0 in order (cycling
    through the batch) until the time budget is spent: verification,
    estimator feature/score of the request's draft rows, and one refit step
    over the labels of each full pass."""
    import numpy as np

    from oracle import av as oav
    from oracle import verify as ov

    t0 = time.perf_counter()
    n = pos = 0
    feats, labs = [], []

    def refit():
        oav.fit_step(np.array(feats), np.array(labs), batch.av_params, np.zeros((batch.max_k, 6)), do_update=True)
        feats.clear()
        labs.clear()

    while time.perf_counter() - t0 < budget_s or n < 4:
        r = n % batch.B
        k = int(batch.num_draft[r])
        ds, ts = int(batch.draft_row_start[r]), int(batch.target_row_start[r])
        zd = ov.decode_rows(batch.draft[ds:ds + k], batch.dtype)
        zt = ov.decode_rows(batch.target[ts:ts + k + 1], batch.dtype)
        res = ov.verify_request(zd, zt, batch.draft_tokens[r, :k], float(batch.temperature[r]),
                                batch.u_accept[r, :k], float(batch.u_residual[r]), float(batch.u_bonus[r]))
        f = np.full(batch.max_k, np.nan, np.float32)
        for i in range(k):
            f[i] = oav.feature(zd[i], float(batch.temperature[r]))
            oav.score(f[i], batch.av_params, i)
        lab = np.full(batch.max_k, -1, np.int8)
        lab[:k] = res.labels
        feats.append(f)
        labs.append(lab)
        n += 1
        pos += k
        if n % batch.B == 0:
            refit()
    if feats:
        refit()
    dt = time.perf_counter() - t0
    return {"value": pos / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} requests ({pos} positions) of input set 0, in order, cycling through its "
                      f"{batch.B}; fp64 numpy verify + feature/score + one refit per pass, "
                      f"{dt:.1f} s single-threaded"}


_POOL_BATCH = None  # the batch the forked workers read (inherited, never copied)


def _pool_worker(job):
    """One worker of the all-cores baseline: requests w, w + P, ... of the
    batch, verification + feature/score each, one refit per B requests,
    until its time budget is spent."""
    import numpy as np

    from oracle import av as oav
    from oracle import verify as ov

    from threadpoolctl import threadpool_limits

    threadpool_limits(1)
    w, P, budget_s = job
    batch = _POOL_BATCH
    t0 = time.perf_counter()
    n = pos = 0
    feats, labs = [], []
    r = w % batch.B
    while time.perf_counter() - t0 < budget_s or n < 2:
        k = int(batch.num_draft[r])
        ds, ts = int(batch.draft_row_start[r]), int(batch.target_row_start[r])
        zd = ov.decode_rows(batch.draft[ds:ds + k], batch.dtype)
        zt = ov.decode_rows(batch.target[ts:ts + k + 1], batch.dtype)
        res = ov.verify_request(zd, zt, batch.draft_tokens[r, :k], float(batch.temperature[r]),
                                batch.u_accept[r, :k], float(batch.u_residual[r]), float(batch.u_bonus[r]))
        f = np.full(batch.max_k, np.nan, np.float32)
        for i in range(k):
            f[i] = oav.feature(zd[i], float(batch.temperature[r]))
            oav.score(f[i], batch.av_params, i)
        lab = np.full(batch.max_k, -1, np.int8)
        lab[:k] = res.labels
        feats.append(f)
        labs.append(lab)
        n += 1
        pos += k
        r = (r + P) % batch.B
        if n % batch.B == 0:
            oav.fit_step(np.array(feats), np.array(labs), batch.av_params, np.zeros((batch.max_k, 6)), do_update=True)
            feats.clear()
            labs.clear()
    return n, pos, time.perf_counter() - t0


def cpu_baseline_pool(batch, budget_s):
    """The oracle on every core of the host's share (at most 16 processes,
    one BLAS thread each), forked before the GPU is touched; workers take
    interleaved requests of input set 0.  Positions over the wall time."""
    import multiprocessing as mp

    from oracle import av as _oav, verify as _ov  # noqa: F401  (imported once, inherited by the workers)

    global _POOL_BATCH
    _POOL_BATCH = batch
    P = max(1, min(16, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(P) as pool:
        out = pool.map(_pool_worker, [(w, P, budget_s) for w in range(P)])
    dt = time.perf_counter() - t0
    n = sum(o[0] for o in out)
    pos = sum(o[1] for o in out)
    return {"value": pos / dt, "unit": "positions/s", "cores": P, "kind": "oracle",
            "sample": f"{n} requests ({pos} positions) of input set 0 over {P} processes (interleaved "
                      f"requests, cycling); fp64 numpy verify + feature/score + one refit per {batch.B} "
                      f"requests of a process; {budget_s:.0f} s per process, {dt:.1f} s wall"}


def main():
    args = parse_args()
    if args.counters:
        summarize_counters(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (requests shard across GPUs "
              "with no exchange, so the one-GPU rate is the per-GPU rate).", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_token_verification_spec_amd as sv
    from synth import gen

    dev = torch.device("cuda:0")
    log = lambda msg: print(f"bench: {msg}", file=sys.stderr, flush=True)
    log(f"drawing {args.rotate} input sets of {args.workload}")
    batches = [gen.make_batch(args.workload, trial=r) for r in range(args.rotate)]  # before any GPU use
    pool_baseline = None
    if not args.no_cpu_baseline:
        # the all-cores oracle baseline forks its workers before the GPU is used
        log("timing the CPU oracle on all cores")
        pool_baseline = cpu_baseline_pool(batches[0], args.cpu_seconds)
    log("moving inputs to the device")
    sets = [(b, to_device(b, dev)) for b in batches]
    b0 = sets[0][0]
    B, K, V = b0.B, b0.max_k, b0.V
    positions = int(b0.num_draft.sum())
    assert all(int(s[0].num_draft.sum()) == positions for s in sets)
    bytes_per_launch = b0.algorithmic_bytes()

    params = torch.tensor(b0.av_params, device=dev)
    accum = torch.zeros(K, 6, dtype=torch.float64, device=dev)
    ws = sv.Workspace()
    outs = []
    for _, d in sets:
        o = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
             "out_tokens": torch.empty(B, K + 1, dtype=torch.int32, device=dev),
             "labels": torch.empty(B, K, dtype=torch.int8, device=dev),
             "p_draft": torch.empty(B, K, dtype=torch.float32, device=dev),
             "p_target": torch.empty(B, K, dtype=torch.float32, device=dev),
             "av_feature": torch.empty(B, K, dtype=torch.float32, device=dev),
             "av_score": torch.empty(B, K, dtype=torch.float32, device=dev)}
        outs.append(o)
    ws.get(dev, sv.sv_workspace_size(B, V, K, sv.SV_BF16 if b0.dtype == "bf16" else sv.SV_F32))

    def step(i):
        _, d = sets[i % len(sets)]
        o = outs[i % len(sets)]
        sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                          d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                          max_k=K, av_params=params, want_feature=True, workspace=ws, out=o)
        sv.sv_av_fit_step(o["av_feature"], o["labels"], params, accum, do_update=True)

    kernel = args.kernel
    sv.sv_set_verify_kernel({"resident": sv.SV_KERNEL_RESIDENT, "streaming": sv.SV_KERNEL_STREAMING,
                             "auto": sv.SV_KERNEL_AUTO}[kernel])
    # phase 0 of a call is its dominant kernel: the statistics kernel (which
    # reads every logit once), or the whole resident kernel
    kernel_name = "resident_kernel" if kernel == "resident" else "stats_kernel"
    log(f"warming up ({kernel_name})")
    for w in range(args.warmup):
        step(w)
    torch.cuda.synchronize(dev)
    log("timing")

    steps = args.steps
    graph = None
    if args.graph:
        # capture one rotation period per graph replay; the library issues no
        # memset and allocates nothing, so the steps capture as plain kernels
        period = len(sets)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(period):
                step(i)
        graph.replay()
        torch.cuda.synchronize(dev)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    start.record()
    if graph is not None:
        reps = max(1, steps // len(sets))
        steps = reps * len(sets)
        for _ in range(reps):
            graph.replay()
        end.record()
        torch.cuda.synchronize(dev)
        # kernel times from a separate pass of eagerly launched steps, with
        # the library's HIP events on the launching stream
        nk = min(steps, 30 * len(sets))
        sv.sv_timing_enable(nk)
        for k in range(nk):
            step(k)
        phases = sv.sv_timing_read(nk)
    else:
        sv.sv_timing_enable(steps)
        for k in range(steps):
            step(k)
        end.record()
        torch.cuda.synchronize(dev)
        phases = sv.sv_timing_read(steps)
    sv.sv_timing_enable(0)
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / steps
    kernel_ms = float(np.mean(phases[:, 0]))
    second_ms = float(np.mean(phases[:, 1]))
    call_ms = kernel_ms + second_ms
    pct = lambda x: [float(np.percentile(x, q)) for q in (10, 50, 90)]
    kernel_pct, call_pct = pct(phases[:, 0]), pct(phases[:, 0] + phases[:, 1])
    value = positions / (ms_per_step * 1e-3)
    achieved = bytes_per_launch / (kernel_ms * 1e-3) / 1e9
    call_gbs = bytes_per_launch / (call_ms * 1e-3) / 1e9

    # HBM bytes per launch from rocprofv3 counters, valid only for the kernel
    # sources they were measured on
    traffic = None
    if os.path.exists(args.traffic):
        try:
            tr = json.load(open(args.traffic))
            if (tr.get("workload") == args.workload and tr.get("kernel") == kernel_name
                    and tr.get("kernel_source_sha256") == kernel_source_hash()):
                traffic = tr.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    al = outs[0]["accept_len"].float().mean().item()
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "logits": b0.dtype,
                   "step": "sv_spec_verify (with estimator feature+score) + sv_av_fit_step",
                   "input_sets_rotated": len(sets), "graph_replay": bool(graph is not None),
                   "kernel": kernel},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": kernel_name, "kernel_ms": kernel_ms,
                     "algorithmic_bytes_per_launch": bytes_per_launch},
        "extra": {"mean_accept_len": al, "positions_per_step": positions, "wall_s": wall,
                  "sv_spec_verify_call": {"kernels": "stats_kernel + draw_kernel" if kernel != "resident"
                                          else "resident_kernel",
                                          "ms": call_ms, "draw_kernel_ms": second_ms,
                                          "achieved_gbs": call_gbs, "frac": call_gbs / PEAK_HBM_GBS,
                                          "ms_p10_p50_p90": call_pct},
                  "stats_kernel_ms_p10_p50_p90": kernel_pct},
    }
    # streaming-read probe over a buffer of the same size: the statistics
    # kernel's access pattern with no arithmetic (the ceiling a read reaches)
    log("timing the read probe")
    pbuf = torch.ones(bytes_per_launch // 4, dtype=torch.int32, device=dev)
    sink = sv.sv_read_probe(pbuf)
    for _ in range(3):
        sv.sv_read_probe(pbuf, sink=sink)
    torch.cuda.synchronize(dev)
    preps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(preps):
        sv.sv_read_probe(pbuf, sink=sink)
    e1.record()
    torch.cuda.synchronize(dev)
    probe_ms = e0.elapsed_time(e1) / preps
    probe_gbs = bytes_per_launch / (probe_ms * 1e-3) / 1e9
    res["extra"]["read_probe"] = {"bytes": bytes_per_launch, "ms": probe_ms, "achieved_gbs": probe_gbs,
                                  "frac": probe_gbs / PEAK_HBM_GBS,
                                  "stats_kernel_frac_of_probe": achieved / probe_gbs,
                                  "note": "back-to-back calls between two events (launch gaps included)"}
    del pbuf
    # the estimator's global draft budget over the same batch's scores (one
    # workgroup, latency-bound): the decision of how many drafts to verify
    log("timing the global draft budget")
    n = B * K
    jj = torch.arange(n + 1, dtype=torch.float32, device=dev)
    draft_cost = 0.0005 * jj
    verify_cost = 8.0 + 0.0005 * jj
    score = outs[0]["av_score"].nan_to_num(0.0)
    nd = sets[0][1]["num_draft"]
    bo = sv.sv_av_budget(score, nd, draft_cost, verify_cost)
    torch.cuda.synchronize(dev)
    reps = 200
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        sv.sv_av_budget(score, nd, draft_cost, verify_cost, out=bo)
    e1.record()
    torch.cuda.synchronize(dev)
    res["extra"]["av_budget"] = {"us_per_call": e0.elapsed_time(e1) * 1000 / reps, "positions": n,
                                 "bound": "latency (one workgroup)", "budget": int(bo["budget"].item()),
                                 "note": "back-to-back calls between two events; synthetic linear cost tables"}
    # calibration metrics of the estimator: one step's labelled items added to
    # the stream accumulator, then AUC / log-loss / ECE (one workgroup each)
    log("timing the calibration metrics")
    acc = torch.zeros(sv.SV_CALIB_WORDS, dtype=torch.float64, device=dev)
    sv.sv_av_calib_accumulate(score, outs[0]["labels"], acc)
    torch.cuda.synchronize(dev)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(reps):
        sv.sv_av_calib_accumulate(score, outs[0]["labels"], acc)
    e1.record()
    for _ in range(reps):
        m = sv.sv_av_calib_metrics(acc)
    e2.record()
    torch.cuda.synchronize(dev)
    mh = m.cpu().tolist()
    res["extra"]["av_calibration"] = {"accumulate_us_per_call": e0.elapsed_time(e1) * 1000 / reps,
                                      "metrics_us_per_call": e1.elapsed_time(e2) * 1000 / reps,
                                      "positions": n, "bound": "latency (one workgroup)",
                                      "auc": mh[0], "log_loss": mh[1], "ece": mh[2]}
    # the TTS distillation gradient over the same batch's canvas (draft rows
    # against the target rows at the same positions), gradient rows in bf16
    log("timing the distillation gradient")
    d0 = sets[0][1]
    wts = torch.ones(K, dtype=torch.float32, device=dev)
    row_bytes = V * (2 if b0.dtype == "bf16" else 4)
    alg = 3 * positions * row_bytes  # draft and target canvas rows read once, gradient rows written once
    step(0)  # a verification of input set 0 on the workspace: its row statistics serve the second mode
    tg = sv.sv_tts_grad(d0["draft"], d0["draft_row_start"], d0["target"], d0["target_row_start"], nd,
                        d0["temperature"], wts, K, 0.0)
    torch.cuda.synchronize(dev)
    treps = 40
    res["extra"]["tts_grad"] = {"algorithmic_bytes": alg, "bound": "hbm"}
    for mode, vws in (("two_pass", None), ("verify_statistics", ws)):
        tts = lambda: sv.sv_tts_grad(d0["draft"], d0["draft_row_start"], d0["target"], d0["target_row_start"], nd,
                                     d0["temperature"], wts, K, 0.0, verify_workspace=vws, out=tg)
        for _ in range(10):  # untimed: the first calls of a mode run slower
            tts()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(treps):
            tts()
        e1.record()
        torch.cuda.synchronize(dev)
        tts_ms = e0.elapsed_time(e1) / treps
        res["extra"]["tts_grad"][mode] = {"ms_per_call": tts_ms, "achieved_gbs": alg / (tts_ms * 1e-3) / 1e9,
                                          "frac": alg / (tts_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # verification on top-p 0.95 filtered rows (the sampling setting of the
    # estimator page's measurements) over input set 0: statistics pass, the
    # threshold searches' histogram passes, then the verdict and draw
    log("timing the filtered verification")
    tk = torch.zeros(B, dtype=torch.int32, device=dev)
    tp = torch.full((B,), 0.95, dtype=torch.float32, device=dev)
    fws = sv.Workspace()
    fcall = lambda: sv.sv_spec_verify_filtered(d0["draft"], d0["draft_row_start"], d0["target"],
                                               d0["target_row_start"], d0["num_draft"], d0["draft_tokens"],
                                               d0["temperature"], tk, tp, d0["u_accept"], d0["u_residual"],
                                               d0["u_bonus"], max_k=K, workspace=fws, out=fo)
    fo = None
    fo = fcall()
    for _ in range(5):
        fcall()
    torch.cuda.synchronize(dev)
    freps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(freps):
        fcall()
    e1.record()
    torch.cuda.synchronize(dev)
    f_ms = e0.elapsed_time(e1) / freps
    fbytes = b0.algorithmic_bytes()
    res["extra"]["filtered_verify"] = {
        "top_p": 0.95, "ms_per_call": f_ms, "positions_per_s": positions / (f_ms * 1e-3),
        "algorithmic_bytes": fbytes, "achieved_gbs": fbytes / (f_ms * 1e-3) / 1e9,
        "frac": fbytes / (f_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kept_tokens_mean": float(fo["kept"][fo["kept"] >= 0].float().mean()),
        "mean_accept_len": float(fo["accept_len"].float().mean()),
        "note": "back-to-back calls between two events; every logit read once counts as the algorithmic bytes"}
    if args.copy_calibration > 0:
        log("copy calibration")
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        res["extra"]["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = pool_baseline
        res["extra"]["cpu_baseline_one_core"] = cpu_baseline(b0, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
