"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the scaling of
rocprofv3 byte counters by the calibration copy, the lower bounds the line
reports against, and the use of a counter record only for the kernel source it
was taken on."""
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
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, values in rows:
            for v in values:  # one row per counter instance, summed per dispatch
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    mib = 256
    # the copy moves 256 MiB each way; FETCH_SIZE reports half of it (factor 2), WRITE_SIZE all of it
    fetch = [(1, "neg_kernel(float*)", [mib * 1024 / 2 / 4] * 4),
             (2, "void twell::gate_pack256_kernel<...>(PackArgs)", [1000.0, 1000.0]),
             (3, "void twell::gate_pack256_kernel<...>(PackArgs)", [3000.0, 3000.0]),
             (4, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [500.0]),
             (5, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [300.0]),
             (6, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [500.0]),
             (7, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [300.0])]
    write = [(1, "neg_kernel(float*)", [mib * 1024 / 4] * 4),
             (2, "void twell::gate_pack256_kernel<...>(PackArgs)", [10.0]),
             (3, "void twell::gate_pack256_kernel<...>(PackArgs)", [30.0]),
             (4, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [7.0]),
             (5, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [3.0]),
             (6, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [7.0]),
             (7, "void twell::fused_updown_sync_kernel<...>(FusedArgs)", [3.0])]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    bench.traffic_summary(str(f), str(w), mib, "cmd", out_dir=str(tmp_path))
    g = json.loads((tmp_path / "traffic_gate_pack.json").read_text())
    # per dispatch: mean of (2000, 6000) KiB fetched x factor 2; mean of (10, 30) KiB written x 1
    assert g["fetch_factor"] == pytest.approx(2.0)
    assert g["write_factor"] == pytest.approx(1.0)
    assert g["read_bytes_per_launch"] == int(4000 * 1024 * 2.0)
    assert g["write_bytes_per_launch"] == int(20 * 1024)
    assert g["dispatches"] == [2, 2]
    assert g["source_hash"] == bench.kernel_source_hash(bench.KERNEL_SOURCES["gate_pack"])
    # two fused dispatches per call (one per generation of workgroups): bytes per call sum them
    u = json.loads((tmp_path / "traffic_fused_updown.json").read_text())
    assert u["calls"] == 2
    assert u["read_bytes_per_launch"] == int(800 * 1024 * 2.0)
    assert u["write_bytes_per_launch"] == int(10 * 1024)


def test_step_bounds_closed_forms():
    """The lower bounds the bench reports against, recomputed from the workload's
    sizes: MFMA time of the gate GEMM, HBM time of the fused kernel's required
    bytes (every weight row touched once at 16384 tokens), MFMA time of the
    dense FFN; at 16 tokens the gate is bound by reading W_gate."""
    from activation_sparse_feedforward_amd import workloads as W
    w = W.workload(3)
    b = bench.step_bounds(w, 0.005)
    x = 16384 * 2048 * 2
    wt = 8192 * 2048 * 2
    twell = 16384 * 64 * (4 + 16 * 3)
    assert b["gate_pack"] == pytest.approx(2 * 16384 * 2048 * 8192 / 2.5e15 * 1e6, abs=0.01)
    assert b["fused"] == pytest.approx((2 * x + twell + 2 * wt) / 8e12 * 1e6, abs=0.01)
    assert b["dense"] == pytest.approx(6 * 16384 * 2048 * 8192 / 2.5e15 * 1e6, abs=0.01)
    assert b["twell_step"] == pytest.approx(b["gate_pack"] + b["fused"], abs=0.02)
    s = bench.step_bounds(W.workload(3, T=16), 0.005)
    touched = 1 - (1 - 0.005) ** 16
    assert s["gate_pack"] == pytest.approx((16 * 2048 * 2 + wt + 16 * 64 * 52) / 8e12 * 1e6, abs=0.01)
    assert s["fused"] == pytest.approx((2 * 16 * 2048 * 2 + 16 * 64 * 52 + 2 * touched * wt) / 8e12 * 1e6, abs=0.01)
    assert s["dense"] == pytest.approx((2 * 16 * 2048 * 2 + 3 * wt + 2 * 16 * 8192 * 2) / 8e12 * 1e6, abs=0.01)


def test_measured_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    """A committed counter record is used only while the kernel's sources hash
    the same; otherwise the bench reports no traffic figure."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    h = bench.kernel_source_hash(bench.KERNEL_SOURCES["gate_pack"])
    (prof / "traffic_gate_pack.json").write_text(json.dumps({"source_hash": h, "bytes_per_launch": 1234}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gate_pack", h, 1.0) == 1234
    assert bench.measured_traffic("gate_pack", "0" * 16, 1.0) is None
    assert bench.measured_traffic("fused_updown", h, 1.0) is None  # no record at all
