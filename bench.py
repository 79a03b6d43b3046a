"""Benchmark of the Compressor hot path on one MI355X.

Headline: 128K-token C4A prefill with the Hadamard rotation (T = 131072,
H = 7168, D = 512, ratio 4): compressed tokens (windows) per second and ms per
call.  One step is one compressor_prefill call over the whole batch, every
kernel of the path included, inputs resident in HBM.  Also reported: the
32-request decode step (C4A and C128A, H = 7168) in microseconds, each timed
over weight / input copies rotated beyond the 256 MB last-level cache.

Prints one JSON line.  Only the cpu_baseline leg uses the oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


def kernel_source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_kv_wkv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(profile_name, sha):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", profile_name)
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


def bench_prefill(steps, warmup):
    import torch
    import gpu_harness
    import long_context_kv_wkv_amd as cmp
    import workloads

    w = workloads.build_named("c4a_128k")
    case = gpu_harness.DeviceCase(w)
    for _ in range(warmup):
        case.prefill()
    torch.cuda.synchronize()
    # the timed steps run without per-kernel events
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        case.prefill()
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    # per-kernel breakdown: a separate pass with every launch bracketed by
    # events on the library's stream
    cmp.compressor_timing_enable(True)
    for _ in range(max(1, min(steps, 10))):
        case.prefill()
    torch.cuda.synchronize()
    kernels = {}
    for k in ("plan", "hadamard_pack", "prefix", "gemm", "post"):
        n, ms = cmp.compressor_timing_query(k)
        if n:
            kernels[k] = ms / n
    cmp.compressor_timing_enable(False)
    windows = w["T"] // w["ratio"]
    return dict(w=w, ms_per_step=total_ms / steps, windows=windows, kernels=kernels,
                device=torch.cuda.get_device_name(0))


def bench_decode(name, steps, warmup, copies=12):
    """Decode step time with `copies` distinct weight panels / inputs rotated
    so that the 256 MB last-level cache cannot hold the streamed panel."""
    import torch
    import gpu_harness
    import long_context_kv_wkv_amd as cmp
    import workloads

    w = workloads.build_named(name)
    case = gpu_harness.DeviceCase(w)
    panels = [case.w_packed] + [case.w_packed.clone() for _ in range(copies - 1)]
    xs = [case.x] + [case.x.clone() for _ in range(copies - 1)]

    def run(i):
        case.decode(w_packed=panels[i % copies], x=xs[i % copies])

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        run(i)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1000.0 / steps
    # per-kernel durations in a second pass
    cmp.compressor_timing_enable(True)
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    kern = {}
    for k in ("gemv", "decode_tail"):
        n, ms = cmp.compressor_timing_query(k)
        kern[k] = ms * 1000.0 / max(n, 1)
    cmp.compressor_timing_enable(False)
    panel_bytes = case.w_packed.numel() * 2
    return dict(us_per_step=us, kernels_us=kern, panel_bytes=panel_bytes)


def cpu_baseline(w, budget_s=12.0):
    """The oracle, untuned, on a bounded sample of the 128K workload: whole
    windows (projection of their rows, pooling, RMSNorm, RoPE, Hadamard)."""
    from oracle import compressor_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    rng = np.random.default_rng(0)
    n = 32
    t0 = time.perf_counter()
    O.compressor(w, windows=rng.choice(w["out_rows"], n, replace=False), project_all=False)
    dt = time.perf_counter() - t0
    n2 = int(max(n, min(4096, n * budget_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    O.compressor(w, windows=rng.choice(w["out_rows"], n2, replace=False), project_all=False)
    dt2 = time.perf_counter() - t0
    return {"value": n2 / dt2, "unit": "compressed tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n2} random windows of the 128K C4A workload (their 8 projected rows "
                      f"each, pooling, RMSNorm, RoPE, Hadamard) plus the state rows, fp64 numpy, "
                      f"{dt2:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode workloads (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (scales HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return
    if a.decode_only:
        for name in ("decode_c4a", "decode_c128a", "decode_c4a_all", "decode_c128a_all"):
            print(name, json.dumps(bench_decode(name, a.decode_steps, 5)), flush=True)
        return
    pre = bench_prefill(a.steps, a.warmup)
    w = pre["w"]
    T, H, N = w["T"], w["hidden"], 2 * w["coff"] * w["head_dim"]
    gemm_ms = pre["kernels"]["gemm"]
    flops = 2.0 * T * H * N
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    sha = kernel_source_sha("gemm.hpp", "pool.hpp", "common.hpp")
    traffic = load_traffic("gemm_c4a_128k_traffic.json", sha)
    result = {
        "metric": "compressed tokens/s for 128K-token C4A prefill (T=131072, H=7168, D=512, "
                  "ratio 4, rotate); also us per 32-request decode",
        "value": pre["windows"] / (pre["ms_per_step"] * 1e-3),
        "unit": "compressed tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "c4a_128k_prefill", "T": T, "hidden": H, "head_dim": 512,
                   "ratio": 4, "coff": 2, "rotate": True, "batch": 1, "block_size": 128,
                   "out_rows": w["out_rows"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "gemm_pool_kernel",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": gemm_ms},
        "kernels_ms": pre["kernels"],
        "device": pre["device"],
    }
    if not a.no_decode:
        dec = {}
        for name in ("decode_c4a", "decode_c128a", "decode_c4a_all", "decode_c128a_all"):
            d = bench_decode(name, a.decode_steps, 20)
            gv = d["kernels_us"]["gemv"]
            dec[name] = {"us_per_step": d["us_per_step"], "kernels_us": d["kernels_us"],
                         "gemv_hbm_frac": d["panel_bytes"] / (gv * 1e-6) / 1e9 / PEAK_HBM_GBS}
        result["decode"] = dec
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
