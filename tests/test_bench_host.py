"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the
HBM-counter summary (copy calibration, per-launch bytes) and the two CPU
oracle baselines."""
import argparse
import csv
import json
import os
import subprocess
import sys

import numpy as np

import bench
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "not supported" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    """FETCH_SIZE reads half the bytes of a 512 MiB copy, WRITE_SIZE all of
    them (KiB per dispatch): the per-launch bytes of a kernel are its mean
    counter value times those scales; small copies are not calibration."""
    mib = 512
    stats = "void sv::(anonymous namespace)::stats_kernel<unsigned short>(sv::VerifyArgs)"
    draw = "void sv::(anonymous namespace)::draw_kernel<unsigned short>(sv::VerifyArgs)"
    fetch_rows = [("__amd_rocclr_copyBuffer", mib * 1024 / 2)] * 3 + [("__amd_rocclr_copyBuffer", 4.0)]
    fetch_rows += [(stats, 288576.0), (stats, 288578.0), (draw, 66700.0)]
    write_rows = [("__amd_rocclr_copyBuffer", mib * 1024.0)] * 3 + [(stats, 600.0), (stats, 624.0), (draw, 280.0)]
    f, w = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", fetch_rows)
    _counter_csv(w, "WRITE_SIZE", write_rows)
    out = tmp_path / "traffic.json"
    args = argparse.Namespace(counters=[str(f), str(w)], copy_calibration=mib, traffic=str(out),
                              workload="bf16_b256_k4_v128256_peaked")
    bench.summarize_counters(args)
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    s = rec["kernels"]["stats_kernel"]
    assert s["dispatches"] == 2
    assert s["fetch_bytes_per_launch"] == 288577.0 * 2 * 1024
    assert s["write_bytes_per_launch"] == 612.0 * 1024
    d = rec["kernels"]["draw_kernel"]
    assert rec["kernels_of_the_call"] == ["stats_kernel", "draw_kernel"]
    assert rec["bytes_per_call"] == s["bytes_per_launch"] + d["bytes_per_launch"]
    assert rec["kernels"]["draw_kernel"]["fetch_bytes_per_launch"] == 66700.0 * 2 * 1024
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()


def test_cpu_baselines_report_their_cores_and_rate():
    b = gen.make_batch("tiny_fp32_b4_k4_v1024", trial=0)
    one = bench.cpu_baseline(b, 0.2)
    assert one["cores"] == 1 and one["kind"] == "oracle" and one["unit"] == "positions/s"
    assert one["value"] > 0 and np.isfinite(one["value"])
    pool, seen = bench.cpu_baseline_pool(b, 0.2)
    assert set(seen) == set(range(b.B))
    assert pool["cores"] == max(1, min(16, len(os.sched_getaffinity(0))))
    assert pool["kind"] == "oracle" and pool["value"] > 0 and np.isfinite(pool["value"])
    assert f"over {pool['cores']} processes" in pool["sample"]


def _oracle_as_gpu(b, seen):
    """Library-shaped outputs holding the oracle's own results."""
    g = {"accept_len": np.zeros(b.B, np.int32), "out_tokens": np.full((b.B, b.max_k + 1), -1, np.int32),
         "p_draft": np.full((b.B, b.max_k), np.nan, np.float32), "p_target": np.full((b.B, b.max_k), np.nan, np.float32)}
    for r, o in seen.items():
        g["accept_len"][r] = o["a"]
        g["out_tokens"][r, :o["a"] + 1] = o["tokens"]
        g["p_draft"][r, :o["kept"]] = o["pd"]
        g["p_target"][r, :o["kept"]] = o["pt"]
    return g


def test_parity_block_counts_flips_and_failures():
    b = gen.make_batch("tiny_fp32_b4_k4_v1024", trial=0, B=24)
    _, seen = bench.cpu_baseline_pool(b, 0.2)
    g = _oracle_as_gpu(b, seen)
    ok = bench.parity_block(b, g, seen)
    assert ok["ok"] and ok["requests_compared"] == b.B and ok["within_margin_flips"] == 0
    assert ok["max_rel_err_p_draft"] < 1e-6 and ok["max_rel_err_p_target"] < 1e-6
    # a different emitted token where the CDF margin is wide is a failure
    r = max(seen, key=lambda q: seen[q]["cdf"])
    bad = {k: v.copy() for k, v in g.items()}
    bad["out_tokens"][r, bad["accept_len"][r]] ^= 1
    rep = bench.parity_block(b, bad, seen)
    assert rep["failures"] == 1 and not rep["ok"]
    # the same change where the oracle's CDF margin is within 1e-5 is a flip
    seen2 = {q: dict(o) for q, o in seen.items()}
    seen2[r]["cdf"] = 1e-6
    rep = bench.parity_block(b, bad, seen2)
    assert rep["failures"] == 0 and rep["within_margin_flips"] == 1
    # a probability off by more than the tolerance fails
    off = {k: v.copy() for k, v in g.items()}
    off["p_target"][0, 0] *= 1.01
    assert not bench.parity_block(b, off, seen)["ok"]


def test_roofline_fields_follow_from_bytes_and_time():
    # 591 MB in 123 us: 4.80 TB/s, 0.600 of 8 TB/s; 729 MB moved in that time
    # is 5.93 TB/s, 0.741 of peak
    rl = bench.roofline(591.0e6, 0.123, traffic=729.0e6)
    assert abs(rl["achieved"] - 591.0e6 / 0.123e-3 / 1e9) < 1e-6
    assert abs(rl["frac"] - 591.0e6 / 0.123e-3 / 1e9 / 8000.0) < 1e-12
    assert abs(rl["sustained_frac"] - 729.0e6 / 0.123e-3 / 1e9 / 8000.0) < 1e-12
    assert rl["sustained_frac"] > rl["frac"]
    # without counter data there is no sustained rate
    rl = bench.roofline(591.0e6, 0.123)
    assert rl["traffic"] is None and "sustained_frac" not in rl

