"""Host logic of bench.py (CPU only): the one-GPU refusal, the traffic
summary built from rocprofv3 counter CSVs, and the rule that the measured
traffic is reported only while the kernel sources match."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def _write_counter_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for i, (name, kib) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                         "Counter_Value": kib})


def _profile_dispatches(copy_kib, fwd_kib, sweep_kib, naive_kib, bwd_kib=()):
    # the dispatch order of --profile-run: a fill, three copies, three
    # workload forwards, one forward per sweep N, the naive kernels, then the
    # backward's dQ and dK/dV kernels
    fwd = "_ZN2fa12_GLOBAL__N_110fwd_kernelIDF16bLi128ELi64ELb1EEEvNS_9FwdParamsENS_7FwdPlanE"
    rows = [("fill_kernel", 1.0)]
    rows += [("copy_kernel", copy_kib)] * 3
    rows += [(fwd, v) for v in fwd_kib]
    rows += [(fwd, v) for v in sweep_kib]
    rows += [("gemm", v) for v in naive_kib]
    bwd = ("bwd_dq_kernel", "bwd_dkdv_kernel")
    rows += [("_ZN2fa12_GLOBAL__N_1" + bwd[i % 2], v) for i, v in enumerate(bwd_kib)]
    return rows


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "SWEEP_FILE", str(tmp_path / "sweep.json"))
    copy = bench.COPY_BYTES / 1024.0
    # FETCH_SIZE reads half the bytes (scale 2), WRITE_SIZE all of them (scale 1)
    fetch_rows = _profile_dispatches(copy / 2, [60000.0, 61000.0, 70000.0],
                                     [100.0, 200.0, 300.0, 400.0, 500.0, 600.0, 700.0],
                                     [1000.0, 2000.0], [80007.0, 90000.0])
    write_rows = _profile_dispatches(copy, [30000.0, 30000.0, 30000.0],
                                     [10.0, 20.0, 30.0, 40.0, 50.0, 60.0, 70.0], [500.0],
                                     [3.0, 3.0])
    _write_counter_csv(str(tmp_path / "f" / "vm" / "1_counter_collection.csv"), "FETCH_SIZE",
                       fetch_rows)
    _write_counter_csv(str(tmp_path / "w" / "vm" / "1_counter_collection.csv"), "WRITE_SIZE",
                       write_rows)
    assert bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd") == 0
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    # the median of the three workload dispatches, in bytes
    assert t["fetch_bytes_per_launch"] == pytest.approx(61000.0 * 1024 * 2)
    assert t["write_bytes_per_launch"] == pytest.approx(30000.0 * 1024)
    assert t["hbm_bytes_per_launch"] == pytest.approx(61000.0 * 2048 + 30000.0 * 1024)
    assert t["naive_fetch_bytes"] == pytest.approx(3000.0 * 2048)  # the backward is not in it
    assert t["naive_write_bytes"] == pytest.approx(500.0 * 1024)
    assert t["bwd_fetch_bytes"] == pytest.approx(170007.0 * 2048)
    assert t["bwd_write_bytes"] == pytest.approx(6.0 * 1024)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    s = json.load(open(tmp_path / "sweep.json"))
    assert [r["N"] for r in s["rows"]] == list(bench.SWEEP_N)
    r0 = s["rows"][0]
    assert r0["hbm_bytes"] == pytest.approx(100.0 * 2048 + 10.0 * 1024)
    # algorithmic bytes of causal B=2, H=16, N=1024, d=128 bf16: Q, K, V, O and lse
    assert r0["algorithmic_bytes"] == 4 * 2 * 16 * 1024 * 128 * 2 + 2 * 16 * 1024 * 4
    # the large batches follow the sweep's dispatches, in order
    assert [(r["B"], r["H"], r["N"]) for r in s["large_batches"]] == list(bench.LARGE_BATCHES)
    lb = s["large_batches"][0]
    assert lb["hbm_bytes"] == pytest.approx(600.0 * 2048 + 60.0 * 1024)
    B, H, N = bench.LARGE_BATCHES[0]
    assert lb["algorithmic_bytes"] == 4 * B * H * N * 128 * 2 + B * H * N * 4


def test_traffic_summary_rejects_missing_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "SWEEP_FILE", str(tmp_path / "sweep.json"))
    copy = bench.COPY_BYTES / 1024.0
    rows = _profile_dispatches(copy, [1.0, 1.0],
                               [1.0] * (len(bench.SWEEP_N) + len(bench.LARGE_BATCHES)), [])
    _write_counter_csv(str(tmp_path / "f" / "a_counter_collection.csv"), "FETCH_SIZE", rows)
    _write_counter_csv(str(tmp_path / "w" / "a_counter_collection.csv"), "WRITE_SIZE", rows)
    assert bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "cmd") == 1
    assert not os.path.exists(tmp_path / "traffic.json")


def test_measured_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    p = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    p.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                             "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic() == 123.0
    p.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123.0}))
    assert bench.measured_traffic() is None
    p.unlink()
    assert bench.measured_traffic() is None


def test_cpu_baseline_only_times_the_oracle_without_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "1",
                        "--cpu-baseline-only"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cb = line["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["sample"].startswith("1 of 1 heads")
    assert "extrapolated_all_heads_s" not in cb  # the whole workload was timed


FWD = "_ZN2fa12_GLOBAL__N_110fwd_kernelIDF16bLi128ELi64ELb1EEEvNS_9FwdParamsENS_7FwdPlanE"


def test_trace_summary_finds_the_timed_region(tmp_path, capsys):
    """The timed region's launches are found by dispatch order from the counts
    the bench line reports (warm-up, cold start, settle, warm-up, timed)."""
    W, K, S = 5, 20, 40
    durs = [140.0] * W + [160.0] * K + [135.0] * S + [131.0] * W + [130.0] * K + [129.0] * K
    d = tmp_path / "trace" / "vm"
    d.mkdir(parents=True)
    with open(d / "1_kernel_trace.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                           "End_Timestamp"])
        wr.writeheader()
        t = 1000
        for i, us in enumerate(durs):
            wr.writerow({"Dispatch_Id": 2 * i + 1, "Kernel_Name": FWD, "Start_Timestamp": t,
                         "End_Timestamp": t + int(us * 1000)})
            wr.writerow({"Dispatch_Id": 2 * i + 2, "Kernel_Name": "other", "Start_Timestamp": t,
                         "End_Timestamp": t + 1})
            t += 10 ** 6
    with open(d / "1_kernel_stats.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        wr.writeheader()
        wr.writerow({"Name": FWD, "Calls": len(durs), "AverageNs": 1.0, "MinNs": 1, "MaxNs": 2})
    line = {"warmup": W, "steps": K, "settle": {"launches": S}, "value": 1.0,
            "ms_per_step": 0.132, "config": {"workload": "w"},
            "roofline": {"flops_per_launch": 137438953472.0}}
    (tmp_path / "line.json").write_text("noise\n" + json.dumps(line) + "\n")
    assert bench.summarize_trace(str(tmp_path / "trace"), str(tmp_path / "line.json"), "cmd") == 0
    out = capsys.readouterr().out
    assert "| timed region | 20 | 130.0 | 130.0 | 130.0 |" in out
    assert "| cold start (K launches) | 20 | 160.0 |" in out
    assert "| settle | 40 | 135.0 |" in out
    assert "98.5 % of ms_per_step" in out


def test_counter_summary_medians_and_per_block_readings(tmp_path, capsys):
    """Medians over the workload's three forward dispatches (the first three of
    the forward kernel), counters of one pass summed over their rows."""
    vals = {1: 4096.0, 2: 4096.0, 3: 4096.0}
    rows = []
    for i, name in ((1, FWD), (2, "copy"), (3, FWD), (4, FWD), (5, FWD)):
        for c, v in (("SQ_WAVES", 4096.0), ("SQ_INSTS_MFMA", 4259840.0 + i),
                     ("SQ_INSTS_VALU", 23650304.0), ("SQ_WAVE_CYCLES", 100.0)):
            half = v / 2  # two rows per counter (e.g. two shader engines)
            rows += [(i, name, c, half), (i, name, c, half)]
    d = tmp_path / "pmc" / "vm"
    d.mkdir(parents=True)
    with open(d / "1_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        wr.writeheader()
        for i, n, c, v in rows:
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": c,
                         "Counter_Value": v})
    assert bench.summarize_counters([str(tmp_path / "pmc")], 5) == 0
    out = json.loads(capsys.readouterr().out)
    assert out["median_of_3_dispatches"]["SQ_WAVES"] == 4096.0
    assert out["median_of_3_dispatches"]["SQ_INSTS_MFMA"] == 4259840.0 + 3  # dispatches 1, 3, 4
    # d = 128: 32 MFMAs per wave and 64-key block
    assert out["key_blocks_per_wave"] == pytest.approx(32.5, abs=1e-3)
    assert out["per_wave_and_block"]["mfma"] == pytest.approx(32.0)
    assert out["per_wave_and_block"]["valu_other_than_mfma"] == pytest.approx(145.7, abs=0.1)


def test_bwd_counter_summary_takes_the_last_backward_call(tmp_path, capsys):
    """Each backward kernel's counters come from its last dispatch (the
    fa_bwd call that ends --profile-run), summed over rows and passes."""
    dq = "_ZN2fa12_GLOBAL__N_113bwd_dq_kernelIDF16bLi128ELb1EEEvNS_9BwdParamsE"
    dkdv = "_ZN2fa12_GLOBAL__N_115bwd_dkdv_kernelIDF16bLi128ELb1ELi3EEEvNS_9BwdParamsE"
    for pas, counters in (("a", (("SQ_INSTS_MFMA", 1000.0), ("SQ_INSTS_VALU", 4000.0))),
                          ("b", (("SQ_INSTS_LDS", 2000.0), ("SQ_WAVE_CYCLES", 100.0),
                                 ("SQ_WAIT_INST_ANY", 25.0)))):
        rows = []
        for i, name, mul in ((1, FWD, 1.0), (7, dq, 0.5), (8, dkdv, 0.5), (9, dq, 1.0), (10, dkdv, 2.0)):
            for c, v in counters:
                rows += [(i, name, c, v * mul / 2), (i, name, c, v * mul / 2)]
        d = tmp_path / pas / "vm"
        d.mkdir(parents=True)
        with open(d / "1_counter_collection.csv", "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                               "Counter_Value"])
            wr.writeheader()
            for i, n, c, v in rows:
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": c,
                             "Counter_Value": v})
    assert bench.summarize_bwd_counters([str(tmp_path / "a"), str(tmp_path / "b")]) == 0
    out = json.loads(capsys.readouterr().out)
    assert out["bwd_dq"]["counters"]["SQ_INSTS_MFMA"] == 1000.0      # dispatch 9
    assert out["bwd_dkdv"]["counters"]["SQ_INSTS_MFMA"] == 2000.0    # dispatch 10
    assert out["bwd_dq"]["per_mfma"]["valu_other_than_mfma"] == pytest.approx(3.0)
    assert out["bwd_dq"]["per_mfma"]["lds"] == pytest.approx(2.0)
    assert out["bwd_dkdv"]["share_of_wave_time"]["SQ_WAIT_INST_ANY"] == pytest.approx(0.25)
    assert bench.summarize_bwd_counters([str(tmp_path / "nothing")]) == 1


def test_settle_runs_for_the_requested_time(monkeypatch):
    calls = []

    def fake_region(fn, steps, stream):
        calls.append(steps)
        import time
        time.sleep(0.002)
        return 0.15 if len(calls) == 1 else 0.13

    monkeypatch.setattr(bench, "timed_region", fake_region)
    s = bench.settle_clock(lambda: None, 20.0, None, group=20)
    assert s["ms"] >= 20.0 and s["launches"] == 20 * len(calls) >= 40
    assert s["first_group_ms_per_launch"] == 0.15 and s["last_group_ms_per_launch"] == 0.13
    s = bench.settle_clock(lambda: None, 0.0, None)
    assert s["launches"] >= 40  # at least two groups, so first and last are reported
