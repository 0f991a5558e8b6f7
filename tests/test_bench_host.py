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
    # backward's prep, dK/dV and dQ kernels
    fwd = "_ZN2fa12_GLOBAL__N_110fwd_kernelIDF16bLi128ELi64ELb1EEEvNS_9FwdParamsENS_7FwdPlanE"
    rows = [("fill_kernel", 1.0)]
    rows += [("copy_kernel", copy_kib)] * 3
    rows += [(fwd, v) for v in fwd_kib]
    rows += [(fwd, v) for v in sweep_kib]
    rows += [("gemm", v) for v in naive_kib]
    bwd = ("bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel")
    rows += [("_ZN2fa12_GLOBAL__N_1" + bwd[i % 3], v) for i, v in enumerate(bwd_kib)]
    return rows


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "SWEEP_FILE", str(tmp_path / "sweep.json"))
    copy = bench.COPY_BYTES / 1024.0
    # FETCH_SIZE reads half the bytes (scale 2), WRITE_SIZE all of them (scale 1)
    fetch_rows = _profile_dispatches(copy / 2, [60000.0, 61000.0, 70000.0],
                                     [100.0, 200.0, 300.0, 400.0, 500.0], [1000.0, 2000.0],
                                     [7.0, 80000.0, 90000.0])
    write_rows = _profile_dispatches(copy, [30000.0, 30000.0, 30000.0],
                                     [10.0, 20.0, 30.0, 40.0, 50.0], [500.0], [1.0, 2.0, 3.0])
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


def test_traffic_summary_rejects_missing_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "SWEEP_FILE", str(tmp_path / "sweep.json"))
    copy = bench.COPY_BYTES / 1024.0
    rows = _profile_dispatches(copy, [1.0, 1.0], [1.0] * len(bench.SWEEP_N), [])
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
