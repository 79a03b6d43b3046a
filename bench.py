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
DECODE_WORKLOADS = ("decode_c4a", "decode_c128a", "decode_c4a_all", "decode_c128a_all",
                    "decode_c4a_mtp2")


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


def bench_prefill(steps, warmup, name="c4a_128k"):
    import torch
    import gpu_harness
    import long_context_kv_wkv_amd as cmp
    import workloads

    w = workloads.build_named(name)
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


def decode_bytes(w):
    """Algorithmic HBM bytes of one decode step: the panel, x, the ring rows
    the completed windows read (kv and score of their channel set), the state
    rows written, the output rows."""
    r, coff, D, H, B = w["ratio"], w["coff"], w["head_dim"], w["hidden"], w["batch"]
    N = 2 * coff * D
    total = N * H * 2 + w["T"] * H * 2 + w["out_rows"] * D * 2
    slots = np.diff(w["cu_seqlens"]).astype(np.int64)
    seq = w["seqused"] if w["seqused"] is not None else slots
    for b in range(B):
        n = int(seq[b])
        if n == 0:
            continue
        s = int(w["start_pos"][b]) if w["start_pos"] is not None else 0
        e = s + n
        for wi in range(s // r, e // r):
            lo = (wi - (coff - 1)) * r
            total += sum(1 for p in range(lo, (wi + 1) * r) if 0 <= p < s) * D * 8
        total += (e - max(s, r * (e // r) - (coff - 1) * r)) * coff * D * 8
    return total


def bench_decode(name, steps, warmup, copies=12):
    """Decode step time with `copies` distinct weight panels, inputs and state
    pools rotated so that the 256 MB last-level cache cannot hold them."""
    import torch
    import gpu_harness
    import long_context_kv_wkv_amd as cmp
    import workloads

    w = workloads.build_named(name)
    case = gpu_harness.DeviceCase(w)
    panels = [case.w_packed] + [case.w_packed.clone() for _ in range(copies - 1)]
    xs = [case.x] + [case.x.clone() for _ in range(copies - 1)]
    kvs = [case.kv_state] + [case.kv_state.clone() for _ in range(copies - 1)]
    scs = [case.score_state] + [case.score_state.clone() for _ in range(copies - 1)]

    cu = case.cu_seqlens if w["T"] != w["batch"] else None

    def run(i):
        j = i % copies
        case.decode(w_packed=panels[j], x=xs[j], kv_state=kvs[j], score_state=scs[j],
                    cu_seqlens=cu)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # host-driven steps (Python marshalling and launch per step), for context
    ev0.record()
    for i in range(steps):
        run(i)
    ev1.record()
    torch.cuda.synchronize()
    us_eager = ev0.elapsed_time(ev1) * 1000.0 / steps
    # device time per step: one step per copy captured in a HIP graph (the
    # calls do no host sync, allocation or memset) and replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(copies):
            run(j)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    ev0.record()
    for _ in range(reps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1000.0 / (reps * copies)
    # per-kernel durations in a second pass
    cmp.compressor_timing_enable(True)
    for i in range(steps):
        run(i)
    torch.cuda.synchronize()
    kern = {}
    for k in ("decode_main", "decode_tail"):
        n, ms = cmp.compressor_timing_query(k)
        kern[k] = ms * 1000.0 / max(n, 1)
    cmp.compressor_timing_enable(False)
    panel_bytes = case.w_packed.numel() * 2
    return dict(us_per_step=us, us_per_step_eager=us_eager, kernels_us=kern,
                panel_bytes=panel_bytes, step_bytes=decode_bytes(w))


def bench_epilog(steps, copies=9):
    """One compressor_epilog call on the 128K C4A output shape (32768 rows of
    D = 512 into a 40000-row FP8 cache, every 7th row without a slot) in
    device time: calls over `copies` sets of rows and caches (> the 256 MB
    last-level cache) captured in a HIP graph and replayed."""
    import torch
    import long_context_kv_wkv_amd as cmp
    import workloads

    w = workloads.build_epilog(workloads.EPILOG_C4A, workloads.SEED_BASE + 710)
    dev = "cuda:0"
    rows = torch.from_numpy(w["rows"].view(np.int16)).to(dev).view(torch.bfloat16)
    slots = torch.from_numpy(w["slot_mapping"]).to(dev)
    sets = [(rows.clone(), torch.from_numpy(w["cache"]).to(dev),
             torch.from_numpy(w["cache_scale"]).to(dev)) for _ in range(copies)]

    def run(j):
        r, c, sc = sets[j % copies]
        cmp.compressor_epilog(r, slots, c, sc)

    for j in range(3):
        run(j)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(copies):
            run(j)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1000.0 / (reps * copies)
    n, d = w["rows"].shape
    written = int(np.sum(w["slot_mapping"] >= 0))
    nbytes = n * d * 2 + n * 4 + written * (d + 4 * (d // 128))
    return {"us_per_call": us, "rows": n, "rows_written": written, "algorithmic_bytes": nbytes,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "config": "32768 rows x 512 bf16 -> FP8 E4M3 cache rows + fp32 scale per 128"}


def bench_nsa(steps, copies=9):
    """One NsaCompressWithCache call (128 sequences that all compress) in
    device time: calls over `copies` caches (> the 256 MB last-level cache in
    the bytes they read) captured in a HIP graph and replayed."""
    import torch
    import gpu_harness
    import workloads

    w = workloads.build_nsa(workloads.NSA_DECODE, workloads.SEED_BASE + 560)
    case = gpu_harness.NsaCase(w)
    inputs = [case.input] + [case.input.clone() for _ in range(copies - 1)]

    def run(j):
        case.run(input=inputs[j % copies])

    for j in range(3):
        run(j)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for j in range(copies):
            run(j)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // copies)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1000.0 / (reps * copies)
    lens, cbs, stride = w["act_seq_len"], w["cbs"], w["stride"]
    fires = int(np.sum((lens >= cbs) & ((lens - cbs) % stride == 0)))
    row = w["head_num"] * w["head_dim"] * 2
    nbytes = fires * (cbs + 1) * row + w["weight"].size * 2
    return {"us_per_call": us, "compressions": fires, "algorithmic_bytes": nbytes,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "config": "128 sequences, 32 heads x 128, window 32, stride 16, page 128, bf16"}


def cpu_baseline(w, budget_s=20.0):
    """The oracle, untuned, on a bounded sample of the 128K workload: whole
    windows (projection of their rows, pooling, RMSNorm, RoPE, Hadamard),
    as many as fit the time budget (at most every window of the workload)."""
    from oracle import compressor_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    rng = np.random.default_rng(0)

    def run(n):
        t0 = time.perf_counter()
        O.compressor(w, windows=rng.choice(w["out_rows"], n, replace=False), project_all=False)
        return time.perf_counter() - t0

    # a call has a fixed part (the whole output and pool arrays) and a part per
    # window: size the sample from both
    na, nb = 32, 512
    ta, tb = run(na), run(nb)
    per = max((tb - ta) / (nb - na), 1e-6)
    fixed = max(ta - na * per, 0.0)
    n2 = int(max(nb, min(w["out_rows"], (budget_s - fixed) / per)))
    t0 = time.perf_counter()
    O.compressor(w, windows=rng.choice(w["out_rows"], n2, replace=False), project_all=False)
    dt2 = time.perf_counter() - t0
    return {"value": n2 / dt2, "unit": "compressed tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n2} random windows of the 128K C4A workload (their 8 projected rows "
                      f"each, pooling, RMSNorm, RoPE, Hadamard) plus the state rows, fp64 numpy, "
                      f"{dt2:.1f} s"}


# ---------------------------------------------------------------------------
# Profile summaries (run on the host after the rocprofv3 runs listed in
# PROFILE_COMMANDS; they read the CSV files those runs leave under a folder)
# ---------------------------------------------------------------------------
PROFILE_COMMANDS = {
    "kt": "rocprofv3 --kernel-trace --stats -T --output-format csv -d {out}/kt -o run -- "
          "python3 bench.py --steps 20 --warmup 15 --decode-steps 50 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -T --output-format csv -d {out}/fetch -o run -- "
             "python3 bench.py --steps 2 --warmup 1 --no-decode --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE -T --output-format csv -d {out}/write -o run -- "
             "python3 bench.py --steps 2 --warmup 1 --no-decode --no-cpu-baseline",
    "cfetch": "rocprofv3 --pmc FETCH_SIZE -T --output-format csv -d {out}/cfetch -o run -- "
              "python3 bench.py --copy-calibration",
    "cwrite": "rocprofv3 --pmc WRITE_SIZE -T --output-format csv -d {out}/cwrite -o run -- "
              "python3 bench.py --copy-calibration",
}
GEMM_KERNEL = "gemm_pool_kernel"


def _find_csv(folder, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {folder}")
    return hits[0]


def _counter_values(folder, counter, kernel_part):
    import csv
    vals = []
    for r in csv.DictReader(open(_find_csv(folder, "counter_collection.csv"))):
        if r["Counter_Name"] == counter and kernel_part in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    return vals


def summarize_profiles(out):
    """Write profiles/bench_kernel_stats.md and profiles/gemm_c4a_128k_traffic.json
    from the CSV files of the PROFILE_COMMANDS runs under `out`."""
    import csv
    sha = kernel_source_sha("gemm.hpp", "pool.hpp", "common.hpp")
    rows = list(csv.DictReader(open(_find_csv(os.path.join(out, "kt"), "kernel_stats.csv"))))
    lines = ["# Kernel-time summary: bench.py (128K C4A prefill + 32-request decode)", "",
             "Command (from the repository root, on one MI355X):", "", "```",
             PROFILE_COMMANDS["kt"].format(out="gpurun_out"), "```", "",
             "The prefill kernels run 45 times (15 warm-up + 20 timed; the per-kernel event "
             "pass adds 10 more); the decode kernels run for each decode workload x (warm-up + "
             "timed + event-timed) steps.  Durations in ns.", "",
             "| kernel | calls | total ns | average ns | % | min ns | max ns |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].split("(")[0].replace("void ", "")
        name = name.split("<")[0].split("::")[-1][:60]
        lines.append(f"| {name} | {r['Calls']} | {r['TotalDurationNs']} | "
                     f"{float(r['AverageNs']):.0f} | {float(r['Percentage']):.2f} | "
                     f"{r['MinNs']} | {r['MaxNs']} |")
    # per-launch durations of the GEMM from the trace: the first launches of a
    # process run slower while clocks and translation caches settle, so the
    # all-launch average above sits above the warm figure bench.py reports
    trace = [r for r in csv.DictReader(open(_find_csv(os.path.join(out, "kt"), "kernel_trace.csv")))
             if GEMM_KERNEL in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in trace]
    # the command's 128K C4A launches come first: 15 warm-up, 20 timed and 10
    # in the per-kernel event pass; the other prefill workloads follow
    n_head = 15 + 20 + 10
    if len(dur) >= n_head:
        head, rest = dur[:n_head], dur[n_head:]
        lines += ["", f"`{GEMM_KERNEL}` per launch of the 128K C4A prefill (ms, from the kernel "
                  "trace, in launch order): " + ", ".join(f"{x:.3f}" for x in head) + ".",
                  f"Average after the 15 warm-up launches: {np.mean(head[15:]):.3f} ms; average "
                  f"of its last 10 (the per-kernel event pass that bench.py's roofline times): "
                  f"{np.mean(head[-10:]):.3f} ms."]
        if rest:
            lines += ["", "Later launches (the 8192-token C128A prefill, then the packed "
                      "variable-length C4A prefill, each warm-up + timed + event pass; ms): "
                      + ", ".join(f"{x:.3f}" for x in rest) + "."]
    lines += ["", f"Kernel source hash (gemm.hpp + pool.hpp + common.hpp): `{sha}`."]
    open(os.path.join(ROOT, "profiles", "bench_kernel_stats.md"), "w").write("\n".join(lines) + "\n")

    fetch = _counter_values(os.path.join(out, "fetch"), "FETCH_SIZE", GEMM_KERNEL)
    write = _counter_values(os.path.join(out, "write"), "WRITE_SIZE", GEMM_KERNEL)
    cfetch = _counter_values(os.path.join(out, "cfetch"), "FETCH_SIZE", "copy")
    cwrite = _counter_values(os.path.join(out, "cwrite"), "WRITE_SIZE", "copy")
    copy_bytes = 1 << 30
    # counters are KiB per dispatch; a plain copy of known size fixes the scale
    fscale = copy_bytes / (np.median(cfetch) * 1024.0)
    wscale = copy_bytes / (np.median(cwrite) * 1024.0)
    fb = float(np.median(fetch)) * 1024.0 * fscale
    wb = float(np.median(write)) * 1024.0 * wscale
    doc = {
        "kernel": GEMM_KERNEL,
        "workload": "c4a_128k prefill (T=131072, H=7168, N=2048)",
        "kernel_source_sha": sha,
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "copy_calibration": {"bytes": copy_bytes, "fetch_size_kib": cfetch,
                             "write_size_kib": cwrite, "fetch_scale": fscale,
                             "write_scale": wscale},
        "fetch_bytes_per_launch": fb,
        "write_bytes_per_launch": wb,
        "hbm_bytes_per_launch": fb + wb,
        "commands": [PROFILE_COMMANDS[k].format(out="gpurun_out")
                     for k in ("fetch", "write", "cfetch", "cwrite")],
    }
    json.dump(doc, open(os.path.join(ROOT, "profiles", "gemm_c4a_128k_traffic.json"), "w"),
              indent=1)
    print(json.dumps({"kernel_stats_rows": len(rows), "hbm_bytes_per_launch": fb + wb,
                      "sha": sha}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~10 calls of the 128K prefill run slower while clocks and
    # translation caches settle; the default warm-up covers that ramp
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode workloads (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (scales HBM byte counters)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="host only: write profiles/ summaries from rocprofv3 CSVs under DIR")
    a = ap.parse_args()
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles)
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
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
        for name in DECODE_WORKLOADS:
            print(name, json.dumps(bench_decode(name, a.decode_steps, 5)), flush=True)
        print("epilog_fp8", json.dumps(bench_epilog(a.decode_steps)), flush=True)
        return
    pre = bench_prefill(a.steps, a.warmup)
    w = pre["w"]
    T, H, N = w["T"], w["hidden"], 2 * w["coff"] * w["head_dim"]
    gemm_ms = pre["kernels"]["gemm"]
    flops = 2.0 * T * H * N
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    sha = kernel_source_sha("gemm.hpp", "pool.hpp", "common.hpp")
    traffic = load_traffic("gemm_c4a_128k_traffic.json", sha)   # bytes per launch, or None
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
        for name in DECODE_WORKLOADS:
            d = bench_decode(name, a.decode_steps, 20)
            dec[name] = {"us_per_step": d["us_per_step"],
                         "us_per_step_eager": d["us_per_step_eager"],
                         "kernels_us": d["kernels_us"],
                         "algorithmic_bytes": d["step_bytes"],
                         "hbm_frac": d["step_bytes"] / (d["us_per_step"] * 1e-6) / 1e9
                         / PEAK_HBM_GBS}
        result["decode"] = dec
        result["nsa_compress"] = bench_nsa(a.decode_steps)
        result["epilog_fp8"] = bench_epilog(a.decode_steps)
        # the other prefill workloads: the 8192-token C128A call and the
        # packed variable-length C4A continuation (8 requests, 88826 tokens)
        other = {}
        for name in ("c128a_8192", "varlen_c4a"):
            p = bench_prefill(10, 5, name)
            pw = p["w"]
            fl = 2.0 * pw["T"] * pw["hidden"] * 2 * pw["coff"] * pw["head_dim"]
            other[name] = {"ms_per_step": p["ms_per_step"], "kernels_ms": p["kernels"],
                           "gemm_tflops": fl / (p["kernels"]["gemm"] * 1e-3) / 1e12,
                           "gemm_mfma_frac": fl / (p["kernels"]["gemm"] * 1e-3) / 1e12
                           / PEAK_BF16_TFLOPS, "tokens": pw["T"]}
        result["prefill_other"] = other
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
