"""Host-side checks of bench.py (no GPU): the one-GPU refusal and the
scaling of rocprofv3 byte counters by the calibration copy."""
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
