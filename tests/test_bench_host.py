"""Host-side pieces of bench.py (no GPU): the refusal of multi-GPU runs and
the ingestion of rocprofv3 counter CSVs into the kernel-keyed counter and
traffic files that the JSON line reports."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HEAD = "_ZN4attn5fwd1610fwd_kernelILi128ELi1ELi4ELb0EDF16bEEvNS0_10KernelArgsE"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _rows(kernel, counters, dispatches, dur_ns=1_000_000):
    out = []
    for i in range(dispatches):
        for name, val in counters.items():
            out.append({"Dispatch_Id": str(100 + i), "Kernel_Name": kernel, "Counter_Name": name,
                        "Counter_Value": repr(val), "Start_Timestamp": str(10_000_000 * i),
                        "End_Timestamp": str(10_000_000 * i + dur_ns)})
    return out


def test_multi_gpu_request_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_ingest_counters_and_traffic(tmp_path):
    tiles = (8192 // 32) * (8192 // 32) * 2 * 16
    cyc = 1.5e6  # per XCD, over a 1 ms launch: 1.5 GHz
    sq = {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.7 * 1024 * cyc,
          "SQ_INSTS_MFMA": 18.0 * tiles, "SQ_INSTS_VALU": 84.0 * tiles, "SQ_INSTS_LDS": 24.0 * tiles}
    _write(str(tmp_path / "a" / "p_counter_collection.csv"), _rows(HEAD, sq, 4))
    # the copy's FETCH_SIZE reads half of the copied KiB (as on the MI355X), so the calibration must
    # find a factor of 2 for reads and 1 for writes
    n = 1 << 30
    _write(str(tmp_path / "f" / "p_counter_collection.csv"), _rows(HEAD, {"FETCH_SIZE": 100_000.0}, 3))
    _write(str(tmp_path / "w" / "p_counter_collection.csv"), _rows(HEAD, {"WRITE_SIZE": 60_000.0}, 3))
    _write(str(tmp_path / "cf" / "p_counter_collection.csv"),
           _rows("__amd_rocclr_copyBuffer", {"FETCH_SIZE": n / 1024 / 2}, 3))
    _write(str(tmp_path / "cw" / "p_counter_collection.csv"),
           _rows("__amd_rocclr_copyBuffer", {"WRITE_SIZE": n / 1024}, 3))
    oc, ot = str(tmp_path / "counters.json"), str(tmp_path / "traffic.json")
    bench.ingest_pmc([str(tmp_path / x) for x in ("a", "f", "w", "cf", "cw")], out_counters=oc, out_traffic=ot,
                     commands=["cmd"])
    c = json.load(open(oc))
    assert c["kernel_sha"] == bench.kernel_sha()
    assert c["mfma_busy"] == pytest.approx(0.7)
    assert c["clock_GHz"] == pytest.approx(1.5)
    assert c["mfma_per_tile"] == pytest.approx(18.0)
    assert c["valu_per_tile"] == pytest.approx(66.0)
    assert c["lds_per_tile"] == pytest.approx(24.0)
    t = json.load(open(ot))
    assert t["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert t["bytes_per_launch"] == int(100_000 * 1024 * 2 + 60_000 * 1024)
    assert t["algorithmic_bytes_per_launch"] == bench.compulsory_bytes(2, 8192, 16, 128)


def test_counter_files_follow_the_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "c.json"
    f.write_text(json.dumps({"kernel_sha": "0" * 16, "mfma_busy": 0.5}))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.counters_entry() is None  # taken on another source
    f.write_text(json.dumps({"kernel_sha": bench.kernel_sha(), "mfma_busy": 0.5}))
    assert bench.counters_entry()["mfma_busy"] == 0.5
