"""Throughput of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--no-cpu-baseline]

Workload (default): causal bf16 attention forward, B=2, H=16, N=4096, d=128,
Q/K/V iid N(0,1) from a seeded CPU generator, already resident in device
memory when timing starts. A timed step is one fa_fwd launch over the whole
batch (value = forward TFLOP/s at 4*B*H*N^2*d/2 FLOPs). The backward pass is
timed the same way and reported beside it ("bwd"), together with one full
forward+backward pass ("fwd_bwd_step").

Prints ONE JSON line. Timing uses HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes to
libfa). The roofline's kernel duration is the mean of per-launch event pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_causal_b2h16n4096d128_traffic.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "exact_io_aware_17_amd", "csrc", f)
    for f in ("fa_fwd_bf16.hip", "fa_device.h", "fa_internal.h")
]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(x, w, budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on a bounded sample: whole heads of the
    same workload, one after another, until the time budget is used."""
    import numpy as np
    from oracle import attention as orc
    from exact_io_aware_17_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the process's CPU count
        blas_threads = os.cpu_count() or 1
    q = x["q"].double().numpy()
    k = x["k"].double().numpy()
    v = x["v"].double().numpy()
    kv = None if "kv_lens" not in x else [int(a) for a in x["kv_lens"].tolist()]
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for bh in heads:
        orc.attn_fwd_naive(q, k, v, w.scale, w.causal, kv, heads=[bh])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = W.fwd_flops(1, done, w.N, w.d, w.causal)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads (full N={w.N} rows each), fp64 numpy, "
                  f"{dt:.1f} s",
    }


COPY_BYTES = 256 * 2 ** 20  # calibration copy: 256 MiB read + 256 MiB written


def profile_run(w) -> int:
    """A short run for counter collection: a plain copy of known size, then the
    forward kernel, three times each."""
    import torch
    import exact_io_aware_17_amd as fa
    from exact_io_aware_17_amd import workloads as W

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    x = W.make_inputs(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kv = x["kv_lens"].to(dev) if "kv_lens" in x else None
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    for _ in range(3):
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_lens=kv)
    torch.cuda.synchronize()
    print("profile run done", flush=True)
    return 0


def summarize_traffic(fetch_dir: str, write_dir: str, command: str) -> int:
    """HBM bytes per fa_fwd launch from FETCH_SIZE / WRITE_SIZE counter runs of
    --profile-run, each scaled by what the counter reads for the known copy."""
    import csv
    import glob

    def read(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    out = {"kernel_source_hash": kernel_source_hash(), "command": command,
           "copy_bytes": COPY_BYTES}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        rows = read(d, counter)
        copy = [v for n, v in rows if "fwd_bf16" not in n and v > 0.5 * COPY_BYTES / 1024]
        fwd = [v for n, v in rows if "fwd_bf16" in n]
        if not copy or not fwd:
            print(f"no {counter} readings for the copy or the forward kernel", file=sys.stderr)
            return 1
        scale = COPY_BYTES / (sorted(copy)[len(copy) // 2] * 1024.0)
        per_launch = sorted(fwd)[len(fwd) // 2] * 1024.0 * scale
        out[key + "_kib_raw"] = sorted(fwd)[len(fwd) // 2]
        out[key + "_scale"] = scale
        out[key + "_bytes_per_launch"] = per_launch
    out["hbm_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run (copy calibration + forward) for rocprofv3 counters")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn FETCH_SIZE / WRITE_SIZE runs of --profile-run into "
                         "the committed traffic summary")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command recorded in the traffic summary")
    args = ap.parse_args()
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.traffic_command)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch
    import exact_io_aware_17_amd as fa
    from exact_io_aware_17_amd import workloads as W

    w = W.BY_ID[args.workload]
    if args.profile_run:
        return profile_run(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = W.make_inputs(W.with_shape(w, backward=True))
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    kv = x["kv_lens"].to(dev) if "kv_lens" in x else None
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd_once():
        fa.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_lens=kv, out=o, lse=lse)

    for _ in range(args.warmup):
        fwd_once()
    torch.cuda.synchronize()

    # Whole timed region: K launches back to back.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        fwd_once()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # Per-launch durations (event pair around each launch) for the roofline.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        fwd_once()
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) for a, b in evs)
    ms_kernel = sum(per_launch) / len(per_launch)

    flops = W.fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    tflops = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    traffic = measured_traffic()

    out = {
        "metric": "attention fwd TFLOP/s & % bf16 MFMA peak (causal, N=4096, d=128) on 1 MI355X",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "fwd_bf16_kernel<128,32,2,causal>",
            "flops_per_launch": flops,
            "kernel_ms_mean": round(ms_kernel, 5),
            "kernel_ms_min": round(per_launch[0], 5),
            "algorithmic_hbm_bytes": W.fwd_bytes(w.B, w.H, w.N, w.d, 2),
        },
    }

    if not args.no_bwd:
        ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)

        def bwd_once():
            return fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, kv_lens=kv,
                          workspace=ws)

        for _ in range(max(2, args.warmup // 2)):
            bwd_once()
        torch.cuda.synchronize()
        nb = max(5, args.steps // 2)
        t_start.record(stream)
        for _ in range(nb):
            bwd_once()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_bwd = t_start.elapsed_time(t_end) / nb
        t_start.record(stream)
        for _ in range(nb):
            fwd_once()
            bwd_once()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_fb = t_start.elapsed_time(t_end) / nb
        bflops = W.bwd_flops(w.B, w.H, w.N, w.d, w.causal)
        out["bwd"] = {"ms": round(ms_bwd, 5), "tflops": round(bflops / (ms_bwd * 1e-3) / 1e12, 2),
                      "flop_convention": "10*B*H*N^2*d, halved for causal"}
        out["fwd_bwd_step"] = {"ms": round(ms_fb, 5),
                               "tflops": round((flops + bflops) / (ms_fb * 1e-3) / 1e12, 2)}

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
