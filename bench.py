#!/usr/bin/env python3
"""Throughput of one verification step on one MI355X.

A step is one pass of the whole hot path over one batch already resident in
HBM.  For the default workload - B=256 requests, K=4 drafts, V=128256, bf16
logits (``bf16_b256_k4_v128256_peaked``) - it is ``sv_spec_verify``
(softmax statistics of every draft and target row, accept tests,
first-rejection scan, residual or bonus draw, plus the estimator feature and
score of every draft row from the same pass) followed by ``sv_av_fit_step``
(one damped IRLS step over the batch's labels).  For the long-draft workload
with pruning (``bf16_b512_k8_v151936_t0.7``) it is ``sv_av_score`` (feature,
score, survival prune at 0.3) -> ``sv_spec_verify`` on the kept prefixes ->
``sv_av_fit_step``.  Several independently drawn input sets rotate between
steps so that no step reads rows the previous one left in the 256 MB
Infinity Cache; the timed steps replay from a captured HIP graph.

Prints one JSON line:
  value / ms_per_step   positions per second over the timed steps;
  roofline              the whole verification call (or, with pruning, the
                        scoring pass plus the verification call): the
                        algorithmic HBM bytes per call (every logit the call
                        must read, read once) over the call's time from a
                        graph of back-to-back calls timed with HIP events on
                        the launching stream, against the 8 TB/s HBM3E peak;
                        traffic: the HBM bytes rocprofv3 counters measured
                        for the same kernels (profiles/traffic_<workload>.json),
                        if they describe the current kernel sources, and
                        sustained_frac: those bytes over the call's time
                        against the peak (the re-reads included), and
                        design_bound_frac: the algorithmic fraction the call
                        would reach if it moved those bytes at the read
                        probe's rate;
  parity                the GPU's outputs for input set 0 against the CPU
                        oracle's for the requests the oracle baseline ran;
  cpu_baseline          the oracle, untuned, on the host's cores over a
                        bounded sample of the same workload;
  extra                 call_ms_spread: the 10th, 50th and 90th percentiles
                        of the call time over the graph's replays; and
                        the other entry points on the same batch: the
                        scoring pass alone, the global draft budget,
                        calibration metrics, the distillation gradient, the
                        filtered verification, and a read-bandwidth probe.
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


def metric_name(wl) -> str:
    """The headline metric for the default workload; for another workload the
    same metric at its own shape."""
    k = f"1..{wl.max_k}" if wl.ragged else str(wl.max_k)
    dt = "bf16" if wl.dtype == "bf16" else "fp32"
    name = f"verified draft positions/sec at B={wl.B},K={k},V={wl.V} {dt}; achieved HBM GB/s"
    return METRIC if name.split(";")[0] == METRIC.split(";")[0] else name
PEAK_HBM_GBS = 8000.0
MARGIN = 1e-5  # parity: decisions closer than this to their threshold may flip


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="bf16_b256_k4_v128256_peaked")
    p.add_argument("--rotate", type=int, default=3, help="input sets cycled between steps")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="time the step and the call only")
    p.add_argument("--traffic", default=None,
                   help="per-launch HBM bytes measured with rocprofv3 counters (optional; default "
                        "profiles/traffic_<workload>.json)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after timing, copy a MIB-sized device buffer 3 times (reference for HBM counters)")
    p.add_argument("--counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                        "rocprofv3 pass (run with --copy-calibration) into per-launch HBM bytes, print them and "
                        "store them in --traffic")
    args = p.parse_args(argv)
    if args.traffic is None:
        args.traffic = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    return args


# ---------------------------------------------------------------------------
# HBM counters (no GPU work)
# ---------------------------------------------------------------------------

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
            # the library's kernels, and the read probe of the measurement library
            m = (re.search(r"sv::(?:\(anonymous namespace\)::)?(\w+)", r["Kernel_Name"])
                 or re.search(r"(read_probe_kernel)", r["Kernel_Name"]))
            if m and "copyBuffer" not in r["Kernel_Name"]:
                per.setdefault(m.group(1), {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    out = {}
    for k, d in sorted(per.items()):
        f = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"]) * scale["FETCH_SIZE"] * 1024
        w = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"]) * scale["WRITE_SIZE"] * 1024
        out[k] = {"dispatches": len(d["FETCH_SIZE"]), "fetch_bytes_per_launch": f, "write_bytes_per_launch": w,
                  "bytes_per_launch": f + w}
        print(f"{k:24s} {len(d['FETCH_SIZE']):3d} dispatches  fetch {f / 1e6:9.2f} MB  write {w / 1e6:8.2f} MB")
    print(f"scales: FETCH_SIZE x{scale['FETCH_SIZE']:.5f}, WRITE_SIZE x{scale['WRITE_SIZE']:.5f}")
    from synth import workload

    kernels = (SCORE_KERNELS if workload(args.workload).prune_threshold > 0.0 else ()) + CALL_KERNELS
    call = [k for k in kernels if k in out]
    rec = {"workload": args.workload, "kernels_of_the_call": call,
           "bytes_per_call": sum(out[k]["bytes_per_launch"] for k in call),
           "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"], "kernels": out,
           "kernel_source_sha256": kernel_source_hash()}
    if FILTERED_KERNELS[0] in out:
        # a call launches the first pass once and some kernels several times
        # (bf16: the later key levels twice): bytes of all their dispatches
        # over the number of calls
        calls = out[FILTERED_KERNELS[0]]["dispatches"]
        rec["filtered_bytes_per_call"] = sum(out[k]["bytes_per_launch"] * out[k]["dispatches"]
                                             for k in FILTERED_KERNELS if k in out) / calls
        rec["filtered_kernel_source_sha256"] = kernel_source_hash(filtered=True)
    with open(args.traffic, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


# the kernels one sv_spec_verify call launches, and those of the scoring pass
# that precedes it in a pruning workload's step
CALL_KERNELS = ("stats_kernel", "draw_kernel")
SCORE_KERNELS = ("score_stats_kernel", "score_finish_kernel")


def kernel_source_hash(filtered: bool = False) -> str:
    """sha256 over the sources the verification kernels (or, with filtered,
    the filtered verification's kernels) are built from, to tell whether
    stored counter measurements still describe them."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_spec_amd", "csrc")
    names = ("filter.hip",) if filtered else ("stream.hip",)
    for name in names + ("sv_segment.hpp", "sv_device.hpp", "sv_internal.hpp"):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


# the kernels of one sv_spec_verify_filtered call
FILTERED_KERNELS = ("filt_stats0_kernel", "filt_select0_kernel", "filt_keys_first_kernel", "filt_select_kernel",
                    "filt_keys_next_kernel", "filt_verdict_kernel", "filt_weight_kernel", "filt_search_kernel")


def stored_traffic(args, filtered: bool = False):
    """Measured HBM bytes per call (of the filtered call, with filtered), if
    recorded for this workload and the current kernel sources; else None."""
    if not os.path.exists(args.traffic):
        return None
    try:
        tr = json.load(open(args.traffic))
    except (OSError, ValueError):
        return None
    key = "filtered_" if filtered else ""
    if tr.get("workload") != args.workload or tr.get(key + "kernel_source_sha256") != kernel_source_hash(filtered):
        return None
    return tr.get(key + "bytes_per_call")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def prunes(batch) -> bool:
    """The workload scores and prunes its drafts before verification."""
    return batch.prune_threshold > 0.0


def elem_bytes(batch) -> int:
    return 2 if batch.dtype == "bf16" else 4


def verify_bytes(batch, num_draft) -> int:
    """Algorithmic bytes of a verification call that also produces the
    estimator feature (so greedy requests read their draft rows too): each
    submitted position's draft and target row and each request's bonus row,
    read once."""
    import numpy as np

    k = np.asarray(num_draft, np.int64)
    return int((2 * k + 1).sum() * batch.V * elem_bytes(batch))


def score_bytes(batch) -> int:
    """Algorithmic bytes of the scoring pass: every draft row read once."""
    return int(batch.num_draft.astype("int64").sum() * batch.V * elem_bytes(batch))


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


# ---------------------------------------------------------------------------
# CPU oracle baseline (the only part of the bench that runs the oracle)
# ---------------------------------------------------------------------------

def oracle_request(batch, r, params):
    """The step of one request on the oracle: feature and score of each draft
    row, the survival prune (when the workload prunes), verification of the
    kept positions.  Returns (positions, kept, features [max_k], labels
    [max_k], the verification result)."""
    import numpy as np

    from oracle import av as oav
    from oracle import verify as ov

    k = int(batch.num_draft[r])
    ds, ts = int(batch.draft_row_start[r]), int(batch.target_row_start[r])
    T = float(batch.temperature[r])
    zd = ov.decode_rows(batch.draft[ds:ds + k], batch.dtype)
    f = np.full(batch.max_k, np.nan, np.float32)
    sc = np.zeros(k)
    for i in range(k):
        f[i] = oav.feature(zd[i], T)
        sc[i] = oav.score(f[i], params, i)
    kept = oav.survival_and_kept(sc, batch.prune_threshold)[1] if prunes(batch) else k
    zt = ov.decode_rows(batch.target[ts:ts + kept + 1], batch.dtype)
    res = ov.verify_request(zd[:kept], zt, batch.draft_tokens[r, :kept], T, batch.u_accept[r, :kept],
                            float(batch.u_residual[r]), float(batch.u_bonus[r]))
    lab = np.full(batch.max_k, -1, np.int8)
    lab[:kept] = res.labels
    return k, kept, f, lab, res


def _record(res, kept):
    """The parts of an oracle result the parity block compares."""
    return {"kept": kept, "a": res.accept_len, "tokens": [int(t) for t in res.tokens],
            "margins": [float(m) for m in res.accept_margin[:min(res.accept_len + 1, kept)]],
            "cdf": float(res.cdf_margin), "pd": [float(x) for x in res.p_draft],
            "pt": [float(x) for x in res.p_target]}


def cpu_baseline(batch, budget_s):
    """The oracle, untuned, on the requests of input set 0 in order (cycling
    through the batch) until the time budget is spent, one refit step per
    full pass over the batch."""
    import numpy as np

    from oracle import av as oav

    t0 = time.perf_counter()
    n = pos = 0
    feats, labs = [], []

    def refit():
        oav.fit_step(np.array(feats), np.array(labs), batch.av_params, np.zeros((batch.max_k, 6)), do_update=True)
        feats.clear()
        labs.clear()

    while time.perf_counter() - t0 < budget_s or n < 4:
        k, _, f, lab, _ = oracle_request(batch, n % batch.B, batch.av_params)
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
                      f"{batch.B}; {step_text(batch)} per request, one refit per pass; "
                      f"{dt:.1f} s single-threaded"}


def step_text(batch) -> str:
    return ("fp64 numpy feature/score, survival prune, verification of the kept drafts" if prunes(batch)
            else "fp64 numpy verification + feature/score")


_POOL_BATCH = None  # the batch the forked workers read (inherited, never copied)


def _pool_worker(job):
    """One worker of the all-cores baseline: requests w, w + P, ... of the
    batch, one refit per B requests, until its time budget is spent.
    Returns the counts and the oracle's results for the requests it ran
    (first pass), which the parity block compares with the GPU's."""
    import numpy as np

    from threadpoolctl import threadpool_limits

    from oracle import av as oav

    threadpool_limits(1)
    w, P, budget_s = job
    batch = _POOL_BATCH
    t0 = time.perf_counter()
    n = pos = 0
    feats, labs = [], []
    seen = {}
    r = w % batch.B
    while time.perf_counter() - t0 < budget_s or n < 2:
        k, kept, f, lab, res = oracle_request(batch, r, batch.av_params)
        if r not in seen:
            seen[r] = _record(res, kept)
        feats.append(f)
        labs.append(lab)
        n += 1
        pos += k
        r = (r + P) % batch.B
        if n % batch.B == 0:
            oav.fit_step(np.array(feats), np.array(labs), batch.av_params, np.zeros((batch.max_k, 6)), do_update=True)
            feats.clear()
            labs.clear()
    return n, pos, time.perf_counter() - t0, seen


def cpu_baseline_pool(batch, budget_s):
    """The oracle on every core of the host's share (at most 16 processes,
    one BLAS thread each), forked before the GPU is touched; workers take
    interleaved requests of input set 0.  Positions over the wall time.
    Returns (baseline record, oracle results by request)."""
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
    seen = {}
    for o in out:
        seen.update(o[3])
    rec = {"value": pos / dt, "unit": "positions/s", "cores": P, "kind": "oracle",
           "sample": f"{n} requests ({pos} positions) of input set 0 over {P} processes (interleaved "
                     f"requests, cycling); {step_text(batch)} per request, one refit per {batch.B} "
                     f"requests of a process; {budget_s:.0f} s per process, {dt:.1f} s wall"}
    return rec, seen


def parity_block(batch, gpu, seen, gpu_kept=None):
    """Compare the GPU's outputs for input set 0 with the oracle's, request by
    request, under the parity rules: accept lengths must agree unless an
    oracle decision margin is within MARGIN, the emitted token unless (with
    equal accept lengths) the CDF margin is; pd(d), pt(d) within tolerance.
    Requests whose kept count differs (a survival at the prune threshold) are
    not compared."""
    import numpy as np

    tol = 2e-3 if batch.dtype == "bf16" else 1e-5
    compared = flips = failures = skipped = 0
    err_d = err_t = 0.0
    for r, o in sorted(seen.items()):
        kept = int(gpu_kept[r]) if gpu_kept is not None else int(batch.num_draft[r])
        if kept != o["kept"]:
            skipped += 1
            continue
        compared += 1
        a_g = int(gpu["accept_len"][r])
        toks_g = [int(t) for t in gpu["out_tokens"][r, :a_g + 1]]
        if a_g != o["a"] or toks_g != o["tokens"]:
            tight = (min(o["margins"]) <= MARGIN if o["margins"] else False) if a_g != o["a"] else o["cdf"] <= MARGIN
            flips += 1 if tight else 0
            failures += 0 if tight else 1
            continue
        for key, store in (("p_draft", "pd"), ("p_target", "pt")):
            g, w = np.asarray(gpu[key][r, :kept], np.float64), np.asarray(o[store][:kept], np.float64)
            sel = np.isfinite(w) & (w != 0)
            if sel.any():
                e = float(np.max(np.abs(g[sel] - w[sel]) / np.abs(w[sel])))
                if key == "p_draft":
                    err_d = max(err_d, e)
                else:
                    err_t = max(err_t, e)
    return {"input_set": 0, "requests_compared": compared, "within_margin_flips": flips,
            "failures": failures, "kept_count_differs": skipped, "max_rel_err_p_draft": err_d,
            "max_rel_err_p_target": err_t, "tolerance": tol, "margin": MARGIN,
            "ok": failures == 0 and err_d <= tol and err_t <= tol}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def graph_ms(fns, reps, dev, spread=None):
    """Milliseconds per call of fns[0], fns[1], ... (one call each per
    rotation), captured once into a HIP graph and replayed ``reps`` times,
    timed with events on the launching stream.  With ``spread`` (a dict),
    an event also follows every replay, and the 10th, 50th and 90th
    percentiles of the per-call time over the replays go into it."""
    import numpy as np
    import torch

    for f in fns:
        f()
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(reps)] if spread is not None else []
    e0.record()
    for r in range(reps):
        g.replay()
        if marks:
            marks[r].record()
    e1.record()
    torch.cuda.synchronize(dev)
    if marks:
        per = [a.elapsed_time(b) / len(fns) for a, b in zip([e0] + marks[:-1], marks)]
        p10, p50, p90 = np.percentile(per, [10, 50, 90])
        spread.update({"p10": float(p10), "median": float(p50), "p90": float(p90), "replays": reps,
                       "calls_per_replay": len(fns)})
    return e0.elapsed_time(e1) / (reps * len(fns)), reps * len(fns)


def roofline(nbytes, ms, traffic=None, **kw):
    """achieved / frac: algorithmic bytes per launch over the launch time;
    with counter-measured traffic, also the HBM rate those bytes moved at
    (sustained_gbs, sustained_frac), which counts the call's re-reads."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
           "traffic": traffic, "algorithmic_bytes_per_launch": int(nbytes), "ms_per_launch": ms}
    if traffic:
        moved = traffic / (ms * 1e-3) / 1e9
        out["sustained_gbs"] = moved
        out["sustained_frac"] = moved / PEAK_HBM_GBS
    out.update(kw)
    return out


def main(argv=None):
    args = parse_args(argv)
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
    b0 = batches[0]
    pool_baseline, seen = None, {}
    if not args.no_cpu_baseline:
        # the all-cores oracle baseline forks its workers before the GPU is used
        log("timing the CPU oracle on all cores")
        pool_baseline, seen = cpu_baseline_pool(b0, args.cpu_seconds)
    log("moving inputs to the device")
    sets = [to_device(b, dev) for b in batches]
    B, K, V = b0.B, b0.max_k, b0.V
    # positions per step: the rotated sets' mean (ragged workloads draw K_b per set)
    positions = float(np.mean([b.positions for b in batches]))
    dcode = sv.SV_BF16 if b0.dtype == "bf16" else sv.SV_F32
    pruning = prunes(b0)

    params = torch.tensor(b0.av_params, device=dev)
    accum = torch.zeros(K, 6, dtype=torch.float64, device=dev)
    ws = sv.Workspace()
    ws.get(dev, sv.sv_workspace_size(B, V, K, dcode))

    def new_out():
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        o = {"accept_len": e(B, torch.int32), "out_tokens": e((B, K + 1), torch.int32),
             "labels": e((B, K), torch.int8), "p_draft": e((B, K), torch.float32),
             "p_target": e((B, K), torch.float32)}
        if not pruning:  # the scoring pass gives the features when the workload prunes
            o["av_feature"] = e((B, K), torch.float32)
            o["av_score"] = e((B, K), torch.float32)
        s = {"feature": e((B, K), torch.float32), "score": e((B, K), torch.float32),
             "num_kept": e(B, torch.int32)}
        return o, s

    outs = [new_out() for _ in sets]

    def score(i, outs=outs, params=params):
        d, (_, s) = sets[i], outs[i]
        sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], params, max_k=K,
                       prune_threshold=b0.prune_threshold, workspace=ws, out=s)

    def verify(i, outs=outs):
        d, (o, s) = sets[i], outs[i]
        nd = s["num_kept"] if pruning else d["num_draft"]
        sv.sv_spec_verify(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], nd,
                          d["draft_tokens"], d["temperature"], d["u_accept"], d["u_residual"], d["u_bonus"],
                          max_k=K, av_params=None if pruning else params, want_feature=not pruning,
                          workspace=ws, out=o)

    def call(i):
        if pruning:
            score(i)
        verify(i)

    def step(i):
        call(i)
        o, s = outs[i]
        sv.sv_av_fit_step(s["feature"] if pruning else o["av_feature"], o["labels"], params, accum,
                          do_update=True)

    log("warming up")
    for w in range(max(args.warmup, len(sets))):
        step(w % len(sets))
    torch.cuda.synchronize(dev)

    log("timing the step")
    reps = max(1, args.steps // len(sets))
    t0 = time.perf_counter()
    ms_per_step, steps = graph_ms([lambda i=i: step(i) for i in range(len(sets))], reps, dev)
    wall = time.perf_counter() - t0
    log("timing the call")
    call_reps = max(1, min(reps, 60 // len(sets) + 1))
    call_spread = {}
    call_ms, _ = graph_ms([lambda i=i: call(i) for i in range(len(sets))], call_reps, dev, spread=call_spread)
    # the kept counts the timed calls verified (parameters fixed while the
    # call graph ran)
    kept = [outs[i][1]["num_kept"].cpu().numpy().copy() if pruning else batches[i].num_draft for i in
            range(len(sets))]
    call_alg = float(np.mean([(score_bytes(batches[i]) if pruning else 0) + verify_bytes(batches[i], kept[i])
                              for i in range(len(sets))]))

    value = positions / (ms_per_step * 1e-3)
    kernels = ("score_stats_kernel + score_finish_kernel + stats_kernel + draw_kernel" if pruning
               else "stats_kernel + draw_kernel")
    rl = roofline(call_alg, call_ms, stored_traffic(args), kernel=("sv_av_score + " if pruning else "")
                  + "sv_spec_verify call (" + kernels + ")",
                  note="call time from a graph of back-to-back calls over the rotated input sets")
    res = {
        "metric": metric_name(gen.workload(args.workload)),
        "value": value,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b0.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "logits": b0.dtype,
                   "arithmetic": "f32 (logits widened exactly), refit sums f64",
                   "step": ("sv_av_score (prune at %g) + sv_spec_verify on the kept drafts + sv_av_fit_step"
                            % b0.prune_threshold) if pruning else
                           "sv_spec_verify (with estimator feature+score) + sv_av_fit_step",
                   "positions": "submitted draft positions per step (sum of K_b)",
                   "input_sets_rotated": len(sets), "graph_replay": True},
        "roofline": rl,
        "extra": {"mean_accept_len": float(outs[0][0]["accept_len"].float().mean()),
                  "positions_per_step": positions, "timed_region_wall_s": wall,
                  "call_ms": call_ms, "call_ms_spread": call_spread,
                  "step_minus_call_ms": ms_per_step - call_ms},
    }
    if pruning:
        res["extra"]["verified_positions_per_step"] = float(np.mean([k.sum() for k in kept]))
    res["extra"]["fitted_params"] = params.cpu().tolist()

    if seen:
        # input set 0 at the starting parameters, as the oracle ran it
        p0 = torch.tensor(b0.av_params, device=dev)
        chk = [new_out()]
        if pruning:
            score(0, outs=chk, params=p0)
        verify(0, outs=chk)
        torch.cuda.synchronize(dev)
        gpu = {k: v.cpu().numpy() for k, v in chk[0][0].items()}
        res["parity"] = parity_block(b0, gpu, seen, chk[0][1]["num_kept"].cpu().numpy() if pruning else None)

    if not args.no_extra:
        extras(args, res, sv, sets, batches, outs, params, ws, call, dev, log)

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
        log("timing the CPU oracle on one core")
        res["cpu_baseline"] = pool_baseline
        res["extra"]["cpu_baseline_one_core"] = cpu_baseline(b0, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def extras(args, res, sv, sets, batches, outs, params, ws, call, dev, log):
    """The other entry points on the same batches, each from a graph of
    back-to-back calls over the rotated input sets."""
    import numpy as np
    import torch

    b0 = batches[0]
    B, K, V = b0.B, b0.max_k, b0.V
    ex = res["extra"]
    n_sets = len(sets)
    rot = lambda f: [lambda i=i: f(i) for i in range(n_sets)]

    # the scoring pass alone (what runs before the target forward when
    # drafts are trimmed): every draft row read once
    log("timing the scoring pass")

    def score_only(i):
        d, (_, s) = sets[i], outs[i]
        sv.sv_av_score(d["draft"], d["draft_row_start"], d["num_draft"], d["temperature"], params, max_k=K,
                       prune_threshold=0.3, workspace=ws, out=s)

    ms, _ = graph_ms(rot(score_only), 20, dev)
    ex["av_score"] = roofline(score_bytes(b0), ms, kernel="score_stats_kernel + score_finish_kernel",
                              prune_threshold=0.3)

    # read-bandwidth probe over a buffer of the verification's size: the
    # statistics kernel's access pattern with no arithmetic
    log("timing the read probe")
    from draft_token_verification_spec_amd import measure

    nbytes = verify_bytes(b0, b0.num_draft)
    pbufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n_sets)]
    sink = measure.read_probe(pbufs[0])
    ms, _ = graph_ms([lambda p=p: measure.read_probe(p, sink=sink) for p in pbufs], 20, dev)
    ex["read_probe"] = {"bytes": nbytes, "ms": ms, "achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
                        "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "call_frac_of_probe": ms / res["roofline"]["ms_per_launch"]}
    rl = res["roofline"]
    if rl.get("traffic") and not prunes(b0):
        # the ceiling of the call's design: its counter-measured bytes moved at
        # the probe's rate, against the algorithmic bytes
        rl["design_bound_frac"] = (rl["algorithmic_bytes_per_launch"] * ex["read_probe"]["achieved_gbs"]
                                   / rl["traffic"] / PEAK_HBM_GBS)
        rl["frac_of_design_bound"] = rl["frac"] / rl["design_bound_frac"]
    del pbufs

    # the estimator's global draft budget over the batch's scores (one
    # workgroup, latency-bound): the decision of how many drafts to verify
    log("timing the global draft budget")
    n = B * K
    if n <= sv.SV_BUDGET_MAX_ITEMS:
        jj = torch.arange(n + 1, dtype=torch.float32, device=dev)
        draft_cost = 0.0005 * jj
        verify_cost = 8.0 + 0.0005 * jj
        score = outs[0][1]["score"].nan_to_num(0.0)
        nd = sets[0]["num_draft"]
        bo = sv.sv_av_budget(score, nd, draft_cost, verify_cost)
        ms, _ = graph_ms([lambda: sv.sv_av_budget(score, nd, draft_cost, verify_cost, out=bo)], 100, dev)
        ex["av_budget"] = {"us_per_call": ms * 1000, "positions": n, "bound": "latency (one workgroup)",
                           "budget": int(bo["budget"].item()), "note": "synthetic linear cost tables"}

    # calibration metrics of the estimator over the step's labelled drafts
    log("timing the calibration metrics")
    acc = torch.zeros(sv.SV_CALIB_WORDS, dtype=torch.float64, device=dev)
    sc0 = outs[0][0]["av_score"] if b0.prune_threshold <= 0 else outs[0][1]["score"]
    lab0 = outs[0][0]["labels"]
    ms_acc, _ = graph_ms([lambda: sv.sv_av_calib_accumulate(sc0, lab0, acc)], 100, dev)
    mout = torch.empty(3, dtype=torch.float64, device=dev)
    ms_met, _ = graph_ms([lambda: sv.sv_av_calib_metrics(acc, out=mout)], 100, dev)
    mh = mout.cpu().tolist()
    ex["av_calibration"] = {"accumulate_us_per_call": ms_acc * 1000, "metrics_us_per_call": ms_met * 1000,
                            "positions": n, "bound": "latency (one workgroup)",
                            "auc": mh[0], "log_loss": mh[1], "ece": mh[2],
                            "note": "metrics of the scores at the fitted parameters over repeated steps"}

    # the TTS distillation gradient over each batch's canvas (draft rows
    # against the target rows at the same positions), gradient rows in the
    # logits' type; the second mode reuses the verification's statistics
    log("timing the distillation gradient")
    wts = torch.ones(K, dtype=torch.float32, device=dev)
    pos = b0.positions
    alg = 3 * pos * V * elem_bytes(b0)  # canvas draft and target rows read once, gradient rows written once
    grads = []
    for i in range(n_sets):
        d = sets[i]
        grads.append(sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                    d["num_draft"], d["temperature"], wts, K, 0.0))
    ex["tts_grad"] = {"algorithmic_bytes": alg, "bound": "hbm"}

    def tts(i, reuse):
        d = sets[i]
        if reuse:
            call(i)  # the verification whose workspace statistics the gradient takes
        sv.sv_tts_grad(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"], d["num_draft"],
                       d["temperature"], wts, K, 0.0, verify_workspace=ws if reuse else None, out=grads[i])

    if b0.prune_threshold <= 0 and bool((b0.temperature > 0).all()):
        ms2, _ = graph_ms(rot(lambda i: tts(i, False)), 20, dev)
        ms_pair, _ = graph_ms(rot(lambda i: tts(i, True)), 20, dev)
        ms1 = ms_pair - res["roofline"]["ms_per_launch"]
        ex["tts_grad"]["two_pass"] = roofline(alg, ms2, kernel="tts_grad_kernel")
        ex["tts_grad"]["verify_statistics"] = roofline(
            alg, ms1, kernel="tts_seg_kernel",
            note="graph of (verification + gradient) pairs minus the verification call's time")

    # verification on top-p 0.95 filtered rows (the sampling setting of the
    # estimator page's measurements)
    if b0.prune_threshold <= 0:
        log("timing the filtered verification")
        tk = torch.zeros(B, dtype=torch.int32, device=dev)
        tp = torch.full((B,), 0.95, dtype=torch.float32, device=dev)
        fws = sv.Workspace()
        fo = [None] * n_sets

        def fcall(i):
            d = sets[i]
            fo[i] = sv.sv_spec_verify_filtered(d["draft"], d["draft_row_start"], d["target"], d["target_row_start"],
                                               d["num_draft"], d["draft_tokens"], d["temperature"], tk, tp,
                                               d["u_accept"], d["u_residual"], d["u_bonus"], max_k=K,
                                               workspace=fws, out=fo[i])

        for i in range(n_sets):
            fcall(i)
        ms, _ = graph_ms(rot(fcall), 10, dev)
        fbytes = verify_bytes(b0, b0.num_draft)
        ex["filtered_verify"] = roofline(fbytes, ms, stored_traffic(args, filtered=True),
                                         kernel="sv_spec_verify_filtered call", top_p=0.95,
                                         positions_per_s=pos / (ms * 1e-3),
                                         kept_tokens_mean=float(fo[0]["kept"][fo[0]["kept"] >= 0].float().mean()),
                                         mean_accept_len=float(fo[0]["accept_len"].float().mean()))
        if b0.dtype == "bf16" and args.copy_calibration == 0:
            # (not in a counter pass, whose filtered bytes are the call above's)
            # the same rows with their logits halved (noise N(0, 1)): the top-p
            # 0.95 thresholds then lie below zero, under the 1024-key window
            # below each maximum, so every search goes on through the
            # weight-cell and key-digit levels, reading its row again
            half = [dict(d, draft=d["draft"] * 0.5, target=d["target"] * 0.5) for d in sets]
            ho = [None] * n_sets

            def hcall(i):
                d = half[i]
                ho[i] = sv.sv_spec_verify_filtered(d["draft"], d["draft_row_start"], d["target"],
                                                   d["target_row_start"], d["num_draft"], d["draft_tokens"],
                                                   d["temperature"], tk, tp, d["u_accept"], d["u_residual"],
                                                   d["u_bonus"], max_k=K, workspace=fws, out=ho[i])

            for i in range(n_sets):
                hcall(i)
            ms_h, _ = graph_ms(rot(hcall), 10, dev)
            ex["filtered_verify"]["thresholds_below_window"] = roofline(
                fbytes, ms_h, kernel="sv_spec_verify_filtered call, logits halved",
                kept_tokens_mean=float(ho[0]["kept"][ho[0]["kept"] >= 0].float().mean()))
            del half, ho
    st = sv.sv_workspace_status(ws, dev)
    ex["workspace_status"] = int(st.item())


if __name__ == "__main__":
    main()
