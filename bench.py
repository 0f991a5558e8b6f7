"""Throughput of the exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--no-cpu-baseline]

Workload (default): causal bf16 attention forward, B=2, H=16, N=4096, d=128,
Q/K/V iid N(0,1) from a seeded CPU generator, already resident in device
memory when timing starts. A timed step is one fa_fwd launch over the whole
batch (value = forward TFLOP/s at 4*B*H*N^2*d/2 FLOPs). The backward pass is
timed the same way and reported beside it ("bwd"), together with one full
forward+backward pass ("fwd_bwd_step"), fa_fwd_ex (split-KV) is compared with
fa_fwd on a grid too small to fill the GPU ("split_kv") and on decode, one
query row per head over a long cache, against the HBM peak and the rate of
the forward's HBM -> LDS load path alone ("decode"), with --large-batch the
forward and the backward at large batches whose grids take the
head-sequential order ("large_batch"), and a naive forward that materialises S and P in device memory (PyTorch matmul +
softmax, the comparison path, not part of libfa) is timed on the same inputs
("naive").

Prints ONE JSON line. Timing uses HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes to
libfa). The device raises its clock over the first tens of milliseconds of
load after idling, so after the W warmup launches K launches are timed once
as they come ("cold_start", reported only), then forward launches keep the
device busy for --settle-ms ("settle"), then W warmup launches and the timed
region whose mean is the value. The roofline's kernel duration is the average launch duration over
the timed region (its two events divided by the K launches it holds); an
event pair around each of K further launches is reported beside it
("per_launch_events", mean, median and min), and so is a third set of K
launches each preceded by a 512 MiB write that evicts the L2 and the
Infinity Cache ("per_launch_flushed": Q, K and V then come from HBM). The
matrix-core ceiling of the device at hand is measured too ("mfma_probe":
libfa_probe's bf16 MFMA-only kernel, launches of the forward's FLOPs timed
the same two ways), so that the forward's rate can be read against the
published peak and against what the matrix cores sustain here.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector (the fp32 forward uses FMAs, not MFMA)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_causal_b2h16n4096d128_traffic.json")
TRAFFIC_WORKLOAD = 5  # the workload (causal B=2 H=16 N=4096 d=128) TRAFFIC_FILE was measured on
PROBE_LIB = os.path.join(ROOT, "exact_io_aware_17_amd", "libfa_probe.so")
FLUSH_BYTES = 512 * 2 ** 20  # > 8 x 4 MB of L2 + 256 MB of Infinity Cache
SWEEP_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_causal_bh32d128_traffic_sweep.json")
SWEEP_N = (1024, 2048, 4096, 8192, 16384)  # causal, B=2, H=16, d=128
# causal d=128 bf16 batches of 16 or more rounds of workgroups, which run
# each XCD's heads one after another: (B, H, N)
LARGE_BATCHES = ((16, 32, 2048), (8, 32, 4096))
KERNEL_SOURCES = [
    os.path.join(ROOT, "exact_io_aware_17_amd", "csrc", f)
    for f in ("fa_fwd.hip", "fa_device.h", "fa_internal.h")
]
FWD_KERNEL_TAG = "fwd_kernel"  # in the forward kernel's name, mangled or not
BWD_KERNEL_TAG = "bwd_"        # in the backward kernels' names (dQ, dK/dV)


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
    same workload, one after another, until the time budget is used. With
    per-batch key lengths the sample starts with one seeded head of every
    batch (so every length is in it) and the line also reports the seconds
    per head and, labelled as such, their extrapolation to every head."""
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
    if kv is not None:
        rng = np.random.default_rng(w.seed)
        first = [(b, int(rng.integers(0, w.H))) for b in range(w.B)]
        heads = first + [bh for bh in heads if bh not in first]
    done = 0
    t0 = time.perf_counter()
    for bh in heads:
        orc.attn_fwd_naive(q, k, v, w.scale, w.causal, kv, heads=[bh])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = W.fwd_flops(1, done, w.N, w.d, w.causal)
    out = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        # threads the oracle ran on: one process, numpy's BLAS on blas_threads
        "cores": int(blas_threads),
        "host_cpus": os.cpu_count(),
        "blas_threads": int(blas_threads),
        "processes": 1,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads (full N={w.N} rows each), fp64 numpy, "
                  f"{dt:.1f} s",
        "s_per_head": round(dt / done, 3),
    }
    if done < len(heads):
        out["extrapolated_all_heads_s"] = round(dt / done * len(heads), 1)
    if kv is not None:
        out["note"] = ("FLOPs counted as the nominal 4*N^2*d (/2 causal) per head: the oracle "
                       "forms every score and hides the keys past kv_len; heads of batches "
                       + ", ".join(f"{b} (kv_len {kv[b]})" for b, _ in heads[:min(done, w.B)])
                       + " in the sample")
    return out


COPY_BYTES = 256 * 2 ** 20  # calibration copy: 256 MiB read + 256 MiB written


def profile_run(w) -> int:
    """A short run for counter collection: a plain copy of known size three
    times, the forward kernel on the workload three times, then once at each
    N of the traffic sweep (causal, B=2, H=16, d=128) and once on each of
    LARGE_BATCHES, then the naive forward once on the workload, then one
    fa_bwd on the workload."""
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
        o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale, kv_lens=kv)
    torch.cuda.synchronize()
    print("profile run: workload done", flush=True)
    for n in SWEEP_N:
        ws = W.with_shape(W.BY_ID[5], N=n)
        xs = W.make_inputs(ws)
        qs, ks, vs = (xs[c].to(dev) for c in ("q", "k", "v"))
        fa.fwd(qs, ks, vs, causal=True, scale=ws.scale)
        torch.cuda.synchronize()
        del qs, ks, vs
        print(f"profile run: sweep N={n} done", flush=True)
    for B, H, n in LARGE_BATCHES:
        ws = W.with_shape(W.BY_ID[5], B=B, H=H, N=n)
        xs = W.make_inputs(ws)
        qs, ks, vs = (xs[c].to(dev) for c in ("q", "k", "v"))
        del xs
        fa.fwd(qs, ks, vs, causal=True, scale=ws.scale)
        torch.cuda.synchronize()
        del qs, ks, vs
        print(f"profile run: batch B={B} H={H} N={n} done", flush=True)
    naive_forward(q, k, v, w.scale, w.causal)
    torch.cuda.synchronize()
    print("profile run: naive forward done", flush=True)
    do = W.make_inputs(W.with_shape(w, backward=True))["do"].to(dev)
    fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, kv_lens=kv)
    torch.cuda.synchronize()
    print("profile run: backward done", flush=True)
    return 0


def summarize_traffic(fetch_dir: str, write_dir: str, command: str) -> int:
    """HBM bytes per fa_fwd launch from FETCH_SIZE / WRITE_SIZE counter runs of
    --profile-run, each scaled by what the counter reads for the known copy."""
    import csv
    import glob

    from exact_io_aware_17_amd import workloads as W

    def read(d, counter):
        rows = []  # (dispatch id, kernel name, value in KiB), dispatch order
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"],
                                 float(r["Counter_Value"])))
        return sorted(rows)

    out = {"kernel_source_hash": kernel_source_hash(), "command": command,
           "copy_bytes": COPY_BYTES}
    sweep = {"kernel_source_hash": out["kernel_source_hash"], "command": command,
             "shape": "causal, B=2, H=16, d=128, bf16", "rows": []}
    per_key = {}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "fetch"), ("WRITE_SIZE", write_dir, "write")):
        rows = read(d, counter)
        first_fwd = min((i for i, n, _ in rows if FWD_KERNEL_TAG in n), default=-1)
        # dispatches before the first forward that moved at least a quarter of
        # the copy's bytes: the copies (FETCH_SIZE reads about half of them)
        copy = [v for i, n, v in rows
                if i < first_fwd and FWD_KERNEL_TAG not in n and v >= 0.25 * COPY_BYTES / 1024]
        fwd = [v for _, n, v in rows if FWD_KERNEL_TAG in n]
        nfwd = 3 + len(SWEEP_N) + len(LARGE_BATCHES)
        if not copy or len(fwd) != nfwd:
            print(f"{counter}: expected copy readings and {nfwd} forward "
                  f"dispatches, got {len(copy)} and {len(fwd)}", file=sys.stderr)
            return 1
        scale = COPY_BYTES / (sorted(copy)[len(copy) // 2] * 1024.0)
        last_fwd = max(i for i, n, _ in rows if FWD_KERNEL_TAG in n)
        naive = sum(v for i, n, v in rows if i > last_fwd and BWD_KERNEL_TAG not in n) * 1024.0 * scale
        out["naive_" + key + "_bytes"] = naive
        # one fa_bwd call (dQ + dK/dV) on the workload, after the naive forward
        out["bwd_" + key + "_bytes"] = sum(v for _, n, v in rows if BWD_KERNEL_TAG in n) * 1024.0 * scale
        wl = sorted(fwd[:3])[1]
        out[key + "_kib_raw"] = wl
        out[key + "_scale"] = scale
        out[key + "_bytes_per_launch"] = wl * 1024.0 * scale
        per_key[key] = [v * 1024.0 * scale for v in fwd[3:]]  # sweep, then batches
    out["hbm_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    out["naive_hbm_bytes"] = out["naive_fetch_bytes"] + out["naive_write_bytes"]
    out["naive_over_fa_fwd"] = out["naive_hbm_bytes"] / out["hbm_bytes_per_launch"]
    for i, n in enumerate(SWEEP_N):
        alg = W.fwd_bytes(2, 16, n, 128, 2)
        meas = per_key["fetch"][i] + per_key["write"][i]
        sweep["rows"].append({"N": n, "fetch_bytes": per_key["fetch"][i],
                              "write_bytes": per_key["write"][i], "hbm_bytes": meas,
                              "algorithmic_bytes": alg, "ratio": meas / alg,
                              "s_p_roundtrip_bytes": 2 * 2 * 16 * W.score_matrix_bytes(n, 2)})
    sweep["large_batches"] = []
    for j, (B, H, n) in enumerate(LARGE_BATCHES):
        i = len(SWEEP_N) + j
        alg = W.fwd_bytes(B, H, n, 128, 2)
        meas = per_key["fetch"][i] + per_key["write"][i]
        sweep["large_batches"].append({"B": B, "H": H, "N": n, "fetch_bytes": per_key["fetch"][i],
                                       "write_bytes": per_key["write"][i], "hbm_bytes": meas,
                                       "algorithmic_bytes": alg, "ratio": meas / alg})
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    with open(SWEEP_FILE, "w") as f:
        json.dump(sweep, f, indent=1)
    print(json.dumps(out))
    print(json.dumps(sweep))
    return 0


def summarize_trace(trace_dir: str, bench_file: str, command: str) -> int:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this
    script: the libfa kernels' statistics, and the metric forward's kernel
    durations per phase of the run (cold start, settle, timed region, ...),
    found by dispatch order from the counts the profiled bench line reports."""
    import csv
    import glob

    line = json.loads(open(bench_file).read().strip().splitlines()[-1])
    stats_f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace_f = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if len(stats_f) != 1 or len(trace_f) != 1:
        print("expected one kernel_stats.csv and one kernel_trace.csv", file=sys.stderr)
        return 1
    names = {"fwd_kernel": "fwd_kernel", "bwd_dkdv": "bwd_dkdv_kernel", "bwd_dq": "bwd_dq_kernel",
             "mfma_peak": "mfma_peak_kernel"}
    rows = []
    for r in csv.DictReader(open(stats_f[0])):
        if any(t in r["Name"] for t in names):
            rows.append(r)
    metric_kernel = None
    for r in csv.DictReader(open(trace_f[0])):
        if FWD_KERNEL_TAG in r["Kernel_Name"]:
            metric_kernel = r["Kernel_Name"]  # the first forward dispatch is the metric's
            break
    durs = [(int(r["Dispatch_Id"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            for r in csv.DictReader(open(trace_f[0])) if r["Kernel_Name"] == metric_kernel]
    durs = [d for _, d in sorted(durs)]
    W, K = line["warmup"], line["steps"]
    S = line["settle"]["launches"]
    phases = [("warm-up", W), ("cold start (K launches)", K), ("settle", S), ("warm-up", W),
              ("timed region", K), ("per-launch event pairs", K), ("after a 512 MiB fill", K)]
    out = ["# rocprofv3 kernel trace: libfa kernels, " + line["config"]["workload"], "",
           "Command (repository root, one MI355X):", "", "    " + command, "",
           "Kernel statistics (`*_kernel_stats.csv`, libfa kernels):", "",
           "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                   f"{r['MinNs']} | {r['MaxNs']} |")
    out += ["", f"Metric forward (`{metric_kernel[:90]}`), kernel durations by phase of the run "
            "(dispatch order, from `*_kernel_trace.csv`):", "",
            "| phase | launches | mean us | min us | max us |", "|---|---|---|---|---|"]
    i = 0
    timed = None
    for name, n in phases:
        seg = durs[i:i + n]
        i += n
        if not seg:
            break
        if name == "timed region":
            timed = sum(seg) / len(seg)
        out.append(f"| {name} | {len(seg)} | {sum(seg) / len(seg):.1f} | {min(seg):.1f} | "
                   f"{max(seg):.1f} |")
    flops = line["roofline"]["flops_per_launch"]
    out += ["", f"The profiled bench line: value {line['value']} TFLOP/s, ms_per_step "
            f"{line['ms_per_step']} (the timed region's events, gaps between launches included); "
            f"the trace's timed-region mean kernel time {timed:.1f} us is "
            f"{flops / (timed * 1e-6) / 1e12:.0f} TFLOP/s of kernel time, "
            f"{100 * timed * 1e-3 / line['ms_per_step']:.1f} % of ms_per_step."]
    print("\n".join(out))
    return 0


def summarize_counters(dirs, workload: int) -> int:
    """Median, over the workload's three forward dispatches of a --profile-run,
    of every counter in the rocprofv3 --pmc output directories `dirs`, and
    the per-wave, per-key-block readings (JSON)."""
    import csv
    import glob

    from exact_io_aware_17_amd import workloads as W

    w = W.BY_ID[workload]
    vals = {}
    kernel = None
    for d in dirs:
        per = {}  # dispatch id -> counter -> summed value
        names = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if FWD_KERNEL_TAG not in r["Kernel_Name"]:
                    continue
                i = int(r["Dispatch_Id"])
                names[i] = r["Kernel_Name"]
                c = per.setdefault(i, {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        first = sorted(per)[:3]  # --profile-run: the workload's three forward launches come first
        kernel = names[first[0]]
        for name in per[first[0]]:
            vals[name] = statistics.median(per[i][name] for i in first)
    waves = vals.get("SQ_WAVES")
    out = {"workload": w.name, "kernel": kernel, "median_of_3_dispatches": vals}
    if waves and "SQ_INSTS_MFMA" in vals:
        mfma_per_block = 2 * (w.d // 16) * 2  # S and P V: (D/16) x 2 key tiles each per 64-key block
        blocks = vals["SQ_INSTS_MFMA"] / waves / mfma_per_block
        out["key_blocks_per_wave"] = round(blocks, 2)
        per_block = lambda k: round(vals[k] / waves / blocks, 1) if k in vals else None
        out["per_wave_and_block"] = {
            "mfma": per_block("SQ_INSTS_MFMA"),
            "valu_other_than_mfma": round((vals["SQ_INSTS_VALU"] - vals["SQ_INSTS_MFMA"]) / waves / blocks, 1)
            if "SQ_INSTS_VALU" in vals else None,
            "exp2": per_block("SQ_INSTS_VALU_TRANS_F32"),
            "lds": per_block("SQ_INSTS_LDS"),
            "salu": per_block("SQ_INSTS_SALU")}
        if "SQ_WAVE_CYCLES" in vals:
            out["share_of_wave_time"] = {k: round(vals[k] / vals["SQ_WAVE_CYCLES"], 3)
                                         for k in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                                                   "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS")
                                         if k in vals}
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            out["valu_coissued_share_of_mfma_busy"] = round(
                vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / vals["SQ_VALU_MFMA_BUSY_CYCLES"], 3)
    print(json.dumps(out, indent=1))
    return 0


def summarize_bwd_counters(dirs) -> int:
    """Counters of the backward's kernels from the fa_bwd call that ends a
    --profile-run (one dispatch each of the dQ and dK/dV kernels), summed
    over the --pmc output directories `dirs`, with per-MFMA and share-of-time
    readings (JSON)."""
    import csv
    import glob

    per = {}  # kernel short name -> counter -> value (its last dispatch)
    for d in dirs:
        rows = {}  # short name -> dispatch id -> counter -> summed value
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                short = next((t for t in ("bwd_dkdv", "bwd_dq") if t in r["Kernel_Name"]), None)
                if short is None:
                    continue
                c = rows.setdefault(short, {}).setdefault(int(r["Dispatch_Id"]), {})
                c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for short, by_id in rows.items():
            per.setdefault(short, {}).update(by_id[max(by_id)])
    out = {}
    for short, v in sorted(per.items()):
        o = {"counters": v}
        m = v.get("SQ_INSTS_MFMA")
        if m:
            o["per_mfma"] = {k: round(x, 3) for k, x in (
                ("valu_other_than_mfma", (v["SQ_INSTS_VALU"] - m) / m if "SQ_INSTS_VALU" in v else None),
                ("exp2", v["SQ_INSTS_VALU_TRANS_F32"] / m if "SQ_INSTS_VALU_TRANS_F32" in v else None),
                ("lds", v["SQ_INSTS_LDS"] / m if "SQ_INSTS_LDS" in v else None)) if x is not None}
        if "SQ_WAVE_CYCLES" in v:
            o["share_of_wave_time"] = {k: round(v[k] / v["SQ_WAVE_CYCLES"], 3)
                                       for k in ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY",
                                                 "SQ_WAIT_INST_LDS") if k in v}
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in v and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            o["valu_coissued_share_of_mfma_busy"] = round(
                v["SQ_VALU_MFMA_COEXEC_CYCLES"] / v["SQ_VALU_MFMA_BUSY_CYCLES"], 3)
        out[short] = o
    if not out:
        print("no backward dispatches in " + " ".join(dirs), file=sys.stderr)
        return 1
    print(json.dumps(out, indent=1))
    return 0


def naive_forward(q, k, v, scale, causal):
    """The unfused path the pages contrast with: S = scale Q K^T and
    P = softmax(S) written to and read back from device memory (bf16), then
    O = P V. A comparison baseline only."""
    import torch
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = q.shape[-2]
        hidden = torch.ones(n, n, dtype=torch.bool, device=q.device).triu_(1)
        s = s.masked_fill(hidden, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v)


def naive_comparison(w, q, k, v, o, stream, reps=5):
    import torch
    from exact_io_aware_17_amd import workloads as W

    for _ in range(2):
        on = naive_forward(q, k, v, w.scale, w.causal)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        on = naive_forward(q, k, v, w.scale, w.causal)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = W.fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    diff = (on.float() - o.float()).abs()
    return {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "what": "torch bf16 matmul + scale + mask + softmax + matmul (S, P in HBM)",
            "max_abs_diff_vs_fa_fwd": round(float(diff.max().item()), 5)}


def split_kv_comparison(dev, stream, B=1, H=2, N=16384, d=128, reps=10):
    """fa_fwd vs fa_fwd_ex with the split-KV workspace on a causal grid too small to fill the GPU."""
    import torch
    import exact_io_aware_17_amd as fa
    from exact_io_aware_17_amd import workloads as W

    g = torch.Generator().manual_seed(17099)
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
    res = {"shape": f"causal B={B} H={H} N={N} d={d}",
           "workspace_bytes": fa.split_workspace_bytes(B, H, N, d, True)}
    flops = W.fwd_flops(B, H, N, d, True)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    for name, split in (("fa_fwd", False), ("fa_fwd_ex_split", True)):
        for _ in range(3):
            fa.fwd(q, k, v, causal=True, split=split)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fa.fwd(q, k, v, causal=True, split=split)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[name] = {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    return res


def large_batch_comparison(dev, stream, reps=10, settle_ms=100.0):
    """Large batches, whose grids of 16 or more rounds of resident workgroups
    run each XCD's heads one after another (fa_fwd_tile_order and
    fa_bwd_tile_order report the orders): the forward at three shapes and the
    backward at one, bf16, d = 128, inputs drawn on the device. Each call is
    timed after settle_ms of the same calls (the clock settle of the main
    measurement)."""
    import torch
    import exact_io_aware_17_amd as fa
    from exact_io_aware_17_amd import workloads as W

    names = {fa.FA_FWD_ORDER_HEAVY_FIRST: "heavy-first", fa.FA_FWD_ORDER_PAIRED: "paired",
             fa.FA_FWD_ORDER_HEAD_SEQUENTIAL: "head-sequential"}
    res = {}
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)

    def timed(f):
        settle_clock(f, settle_ms, stream, group=5)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for B, H, N, causal, bwd in ((16, 32, 2048, True, False), (8, 32, 4096, True, True),
                                 (8, 32, 4096, False, False)):
        d = 128
        g = torch.Generator(device=dev).manual_seed(17100 + N)
        q, k, v = (torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
                   for _ in range(3))
        key = f"{'causal' if causal else 'non-causal'} B={B} H={H} N={N} d={d}"
        ms = timed(lambda: fa.fwd(q, k, v, causal=causal))
        ent = {"tile_order": names[fa.tile_order(N, B * H, d, causal)], "fwd_ms": round(ms, 5),
               "fwd_tflops": round(W.fwd_flops(B, H, N, d, causal) / (ms * 1e-3) / 1e12, 1)}
        if bwd:
            o, lse = fa.fwd(q, k, v, causal=causal)
            do = torch.randn(B, H, N, d, generator=g, device=dev).to(torch.bfloat16)
            ms = timed(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal))
            ent["bwd_order"] = fa.bwd_tile_order(B, H, N, d)
            ent["bwd_ms"] = round(ms, 5)
            ent["bwd_tflops"] = round(W.bwd_flops(B, H, N, d, causal) / (ms * 1e-3) / 1e12, 1)
            del o, lse, do
        res[key] = ent
        del q, k, v
    return res


def timed_region(fn, steps, stream):
    """Mean ms per launch of `steps` launches back to back between two events."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def settle_clock(fn, settle_ms, stream, group=20):
    """Launch `fn` in groups of `group` back to back until at least
    `settle_ms` of wall time has passed. The device raises its clock over the
    first tens of milliseconds of load after idling (the same forward runs
    about 15-20 % slower per launch during that ramp), so a rate taken right
    after a short warmup measures the ramp rather than the kernel. Returns
    what was run and the per-launch time of the first and last groups."""
    times = []
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms or len(times) < 2:
        times.append(timed_region(fn, group, stream))
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "launches": group * len(times),
            "first_group_ms_per_launch": round(times[0], 5),
            "last_group_ms_per_launch": round(times[-1], 5)}


def timing_summary(ms, flops):
    """mean / median / min of per-launch times (ms) and the mean's TFLOP/s."""
    mean = sum(ms) / len(ms)
    return {"ms_mean": round(mean, 5), "ms_median": round(statistics.median(ms), 5),
            "ms_min": round(min(ms), 5), "tflops_mean": round(flops / (mean * 1e-3) / 1e12, 2)}


def mfma_probe(dev, stream, flops_target, reps, warmup=3):
    """The matrix-core rate this device sustains: libfa_probe's kernel (bf16
    32x32x16 MFMAs only, two 256-thread workgroups per CU), each launch sized
    to about flops_target, timed back to back and with an event pair around
    each launch."""
    import torch
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it with "
                           "python -m exact_io_aware_17_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fa_probe_mfma_bf16.restype = ctypes.c_int
    lib.fa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.fa_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = max(1, round(flops_target / lib.fa_probe_mfma_bf16_flops(wgs, 1)))
    flops = lib.fa_probe_mfma_bf16_flops(wgs, iters)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def once():
        r = lib.fa_probe_mfma_bf16(wgs, iters, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(stream.cuda_stream))
        if r != 0:
            raise RuntimeError(f"fa_probe_mfma_bf16 returned {r}")

    for _ in range(warmup):
        once()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        once()
    b.record(stream)
    torch.cuda.synchronize()
    ms_b2b = a.elapsed_time(b) / reps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        once()
        b.record(stream)
    torch.cuda.synchronize()
    per = timing_summary([a.elapsed_time(b) for a, b in evs], flops)
    return {"what": "bf16 v_mfma_f32_32x32x16 only: 4 independent chains per wave, "
                    "2 workgroups of 4 waves per CU, launches of the forward's FLOPs",
            "workgroups": wgs, "iters": iters, "flops_per_launch": flops,
            "back_to_back": {"ms_mean": round(ms_b2b, 5),
                             "tflops_mean": round(flops / (ms_b2b * 1e-3) / 1e12, 2)},
            "per_launch_events": per}


def hbm_probe(dev, stream, reps=10, warmup=3, blocks=64):
    """The HBM -> LDS rate this device sustains: libfa_probe's streaming
    kernel (the forward's buffer-load-to-LDS path and two-stage ring, two
    workgroups per CU), each workgroup reading `blocks` 32 KB blocks."""
    import torch
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it with "
                           "python -m exact_io_aware_17_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fa_probe_stream_lds.restype = ctypes.c_int
    lib.fa_probe_stream_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_stream_lds_bytes.restype = ctypes.c_double
    lib.fa_probe_stream_lds_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    wgs = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = lib.fa_probe_stream_lds_bytes(wgs, blocks)
    src = torch.ones(int(nbytes) // 2, dtype=torch.bfloat16, device=dev)
    sums = torch.empty(wgs, dtype=torch.float32, device=dev)

    def once():
        r = lib.fa_probe_stream_lds(ctypes.c_void_p(src.data_ptr()), wgs, blocks,
                                    ctypes.c_void_p(sums.data_ptr()),
                                    ctypes.c_void_p(stream.cuda_stream))
        if r != 0:
            raise RuntimeError(f"fa_probe_stream_lds returned {r}")

    for _ in range(warmup):
        once()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        once()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    del src
    return {"what": "HBM -> LDS streaming alone: 16-byte buffer loads into LDS, two 32 KB "
                    "stages, two workgroups of 4 waves per CU (the forward's K/V path)",
            "bytes": int(nbytes), "ms": round(ms, 5), "gb_s": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}


def decode_shapes(dev, stream):
    """Decode on a batch of sequences and on one long sequence (few K/V heads
    over a 131k-token cache, where a tile's key range is split in up to 64
    parts), beside the HBM -> LDS streaming rate of the device."""
    out = {"batch": decode_comparison(dev, stream),
           "one_long_sequence": decode_comparison(dev, stream, B=1, Nk=131072),
           "hbm_probe": hbm_probe(dev, stream)}
    for key in ("batch", "one_long_sequence"):
        for name in ("fa_fwd_ex", "fa_fwd_ex_split"):
            out[key][name]["frac_of_probe"] = round(
                out[key][name]["gb_s"] / out["hbm_probe"]["gb_s"], 4)
    return out


def decode_comparison(dev, stream, B=8, H=32, Hkv=8, Nk=32768, d=128, reps=20):
    """Decode: one query row per head over a long K/V cache with grouped heads
    (causal, so the query sees every key). Bound by HBM, not the matrix
    cores: the rate is the bytes of Q, K, V, O and lse per second against
    the 8 TB/s peak. fa_fwd_ex without and with the split-KV plan (a single
    query tile per head is one workgroup unless its key range is split)."""
    import torch
    import exact_io_aware_17_amd as fa

    g = torch.Generator().manual_seed(17098)
    q = torch.randn(B, H, 1, d, generator=g).to(torch.bfloat16).to(dev)
    k, v = (torch.randn(B, Hkv, Nk, d, generator=g).to(torch.bfloat16).to(dev) for _ in range(2))
    nbytes = 2 * q.numel() * 2 + (k.numel() + v.numel()) * 2 + B * H * 4
    res = {"shape": f"causal B={B} H={H} Hkv={Hkv} Nq=1 Nk={Nk} d={d}", "bytes": nbytes}
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    for name, split in (("fa_fwd_ex", False), ("fa_fwd_ex_split", True)):
        for _ in range(3):
            fa.fwd(q, k, v, causal=True, split=split)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fa.fwd(q, k, v, causal=True, split=split)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 5), "gb_s": round(gbs, 1),
                     "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="wall time of forward launches run before the W warmup steps so that "
                         "the timed region starts at the device's sustained clock (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--large-batch", action="store_true",
                    help="also time the forward and backward at large batches (the "
                         "head-sequential orders); off by default, since those launches of "
                         "the metric kernel would change its average in a kernel trace")
    ap.add_argument("--no-split-kv", action="store_true",
                    help="skip the split-KV comparison (it launches the forward kernel "
                         "at another shape)")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time only the fp64 oracle on the workload (no GPU needed)")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the matrix-core rate probe")
    ap.add_argument("--profile-run", action="store_true",
                    help="short run (copy calibration + forward) for rocprofv3 counters")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn FETCH_SIZE / WRITE_SIZE runs of --profile-run into "
                         "the committed traffic summary")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command recorded in the traffic summary")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LINE_FILE"),
                    help="markdown summary of a rocprofv3 --kernel-trace --stats run of this "
                         "script, with the bench line it printed")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="median SQ counters of the workload's forward in rocprofv3 --pmc runs "
                         "of --profile-run (one directory per counter pass)")
    ap.add_argument("--summarize-bwd-counters", nargs="+", metavar="PMC_DIR",
                    help="SQ counters of the backward kernels of the fa_bwd call that ends "
                         "--profile-run, in rocprofv3 --pmc runs (one directory per pass)")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.workload)
    if args.summarize_bwd_counters:
        return summarize_bwd_counters(args.summarize_bwd_counters)
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.traffic_command)
    if args.summarize_trace:
        return summarize_trace(*args.summarize_trace, args.traffic_command)

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
    if args.cpu_baseline_only:
        print(json.dumps({"workload": w.name, "cpu_baseline": cpu_baseline(W.make_inputs(w), w),
                          "cpus": os.cpu_count()}), flush=True)
        return 0
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

    # Cold start: K launches right after the W warmup launches, with the
    # device clock still ramping up from idle (reported, not the value).
    cold = timed_region(fwd_once, args.steps, stream)
    # Settle: keep the device busy with the same launches until its clock
    # has left the ramp (about 30 ms of load on the devices measured), then
    # W warmup launches again and the timed region.
    settle = settle_clock(fwd_once, args.settle_ms, stream)
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

    # Per-launch durations (an event pair around each of K more launches),
    # reported beside the roofline.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        fwd_once()
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in evs]

    # The same with L2 and the Infinity Cache flushed before each launch (a
    # fill kernel over 512 MiB between the launches, outside the event pair).
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for a, b in evs:
        flush.zero_()
        a.record(stream)
        fwd_once()
        b.record(stream)
    torch.cuda.synchronize()
    per_launch_flushed = [a.elapsed_time(b) for a, b in evs]
    del flush

    flops = W.fwd_flops(w.B, w.H, w.N, w.d, w.causal)
    tflops = flops / (ms_step * 1e-3) / 1e12
    paired = (w.dtype != "f32" and bool(w.causal) and
              fa.tile_order(w.N, w.B * w.H, w.d, w.causal) == fa.FA_FWD_ORDER_PAIRED)
    # One step is one forward launch: the timed region's average launch
    # duration is ms_step.
    achieved = tflops
    traffic = measured_traffic() if args.workload == TRAFFIC_WORKLOAD else None
    f32 = w.dtype == "f32"
    peak = PEAK_F32_VECTOR_TFLOPS if f32 else PEAK_BF16_TFLOPS

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
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, resident in HBM)",
        "config": {"workload": W.forward_name(w), "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale,
                   "timed": "forward (fa_fwd); backward reported beside it in bwd"},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "alu" if f32 else "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": (f"fwd_f32_kernel<{w.d}, {'true' if w.causal else 'false'}>" if f32 else
                       f"fwd_kernel<__bf16, {w.d}, {fa.block_keys(w.B, w.H, w.N, w.d, w.causal)}, "
                       f"{'true' if w.causal else 'false'}, {'true' if paired else 'false'}>"),
            "flops_per_launch": flops,
            "kernel_ms_mean": round(ms_step, 5),
            "algorithmic_hbm_bytes": W.fwd_bytes(w.B, w.H, w.N, w.d, 2),
        },
        "cold_start": {"what": "K launches right after the first W warmup launches, the device "
                               "clock still ramping up from idle (not the value)",
                       "ms_per_step": round(cold, 5),
                       "tflops": round(flops / (cold * 1e-3) / 1e12, 2)},
        "settle": dict({"what": "forward launches run between the cold-start region and the W "
                                "warmup launches before the timed region"}, **settle),
        "per_launch_events": dict(
            {"what": "event pair around each of K launches after the timed region"},
            **timing_summary(per_launch, flops)),
        "per_launch_flushed": dict(
            {"what": "the same, a 512 MiB fill (L2 and Infinity Cache evicted) before each launch"},
            **timing_summary(per_launch_flushed, flops)),
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
        # As for the forward: the calls right after the warm-up (reported),
        # then backward calls back to back for the settle time, then the
        # timed calls.
        ms_bwd_cold = timed_region(bwd_once, nb, stream)
        bwd_settle = settle_clock(bwd_once, args.settle_ms, stream, group=5)
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
                      "flop_convention": "10*B*H*N^2*d, halved for causal",
                      "calls": nb,
                      "cold_start": {"ms": round(ms_bwd_cold, 5),
                                     "tflops": round(bflops / (ms_bwd_cold * 1e-3) / 1e12, 2)},
                      "settle": bwd_settle}
        out["fwd_bwd_step"] = {"ms": round(ms_fb, 5),
                               "tflops": round((flops + bflops) / (ms_fb * 1e-3) / 1e12, 2)}

    if not args.no_bwd:
        if not args.no_split_kv:
            out["split_kv"] = split_kv_comparison(dev, stream)
            out["decode"] = decode_shapes(dev, stream)
        if args.large_batch:
            out["large_batch"] = large_batch_comparison(dev, stream)
        out["naive"] = naive_comparison(w, q, k, v, o, stream)
        out["naive"]["speedup_fa_fwd"] = round(out["naive"]["ms"] / ms_step, 2)

    if not args.no_mfma_probe:
        pr = mfma_probe(dev, stream, flops, args.steps)
        pr["fwd_over_probe_back_to_back"] = round(
            tflops / pr["back_to_back"]["tflops_mean"], 4)
        pr["fwd_over_probe_per_launch"] = round(
            out["per_launch_events"]["tflops_mean"] / pr["per_launch_events"]["tflops_mean"], 4)
        out["mfma_probe"] = pr

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
