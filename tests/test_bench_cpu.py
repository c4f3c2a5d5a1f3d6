"""bench.py's host-side reporting on the CPU: the HBM traffic scaling by the
1 GiB calibration copy, the engine-clock summary, the source-hash guard on
stored traffic, and the one-GPU guard.  Synthetic rocprofv3-style CSV files,
no GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(i, name, grid, counter, value, t0=0, t1=1000):
    return {"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": name, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1}


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path, capsys):
    gemm = "void moe::(anonymous namespace)::grouped_gemm_kernel<1>(unsigned short const*)"
    # the 1 GiB copy reads as 0.5 GiB of FETCH_SIZE (factor 2) and 1 GiB of WRITE_SIZE (factor 1)
    fetch = [_row(1, "__amd_rocclr_copyBuffer", 4096, "FETCH_SIZE", 524288.0),
             _row(2, gemm, 4259840, "FETCH_SIZE", 1000.0), _row(3, gemm, 4259840, "FETCH_SIZE", 3000.0)]
    write = [_row(1, "__amd_rocclr_copyBuffer", 4096, "WRITE_SIZE", 1048576.0),
             _row(2, gemm, 4259840, "WRITE_SIZE", 500.0), _row(3, gemm, 4259840, "WRITE_SIZE", 500.0)]
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    out_json = str(tmp_path / "traffic.json")
    bench.summarize_counters([str(tmp_path / "f"), str(tmp_path / "w")], out_json)
    capsys.readouterr()
    data = json.load(open(out_json))
    assert data["fetch_factor"] == pytest.approx(2.0)
    assert data["write_factor"] == pytest.approx(1.0)
    k = data["kernels"]["grouped_gemm_kernel<1>"]
    assert k["read_bytes"] == pytest.approx(2000.0 * 1024 * 2.0)   # mean 2000 KiB, scaled by 2
    assert k["write_bytes"] == pytest.approx(500.0 * 1024)
    assert k["hbm_bytes"] == pytest.approx(k["read_bytes"] + k["write_bytes"])
    assert k["sources_sha256"] == bench.sources_hash("grouped_gemm_kernel<1>")


def test_template_instances_share_their_kernels_sources(tmp_path, capsys):
    q4 = "void moe::(anonymous namespace)::skinny_q4_kernel<1, 7>(unsigned short const*)"
    _write_counters(str(tmp_path / "f"), [_row(1, "__amd_rocclr_copyBuffer", 4096, "FETCH_SIZE", 524288.0),
                                          _row(2, q4, 131072, "FETCH_SIZE", 100.0)])
    _write_counters(str(tmp_path / "w"), [_row(1, "__amd_rocclr_copyBuffer", 4096, "WRITE_SIZE", 1048576.0),
                                          _row(2, q4, 131072, "WRITE_SIZE", 10.0)])
    out_json = str(tmp_path / "traffic.json")
    bench.summarize_counters([str(tmp_path / "f"), str(tmp_path / "w")], out_json)
    capsys.readouterr()
    k = json.load(open(out_json))["kernels"]["skinny_q4_kernel<1, 7>"]
    assert k["sources_sha256"] == bench.sources_hash("skinny_q4_kernel<2, 8>") == bench.sources_hash("skinny_q4_kernel")
    assert bench.sources_hash("skinny_q4_kernel") != bench.sources_hash("skinny_kernel")
    assert bench.kernel_sources("combine_kernel<4>") is None


def test_stored_traffic_is_dropped_when_the_sources_change(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    current = bench.sources_hash("skinny_kernel<1>")
    path.write_text(json.dumps({"kernels": {"skinny_kernel<1>": {"hbm_bytes": 123.0, "sources_sha256": current}}}))
    assert bench.measured_traffic("skinny_kernel<1>") == 123.0
    path.write_text(json.dumps({"kernels": {"skinny_kernel<1>": {"hbm_bytes": 123.0, "sources_sha256": "stale"}}}))
    assert bench.measured_traffic("skinny_kernel<1>") is None
    assert bench.measured_traffic("grouped_gemm_kernel<1>") is None   # not in the file


def test_engine_clock_from_grbm_counts(tmp_path, capsys):
    gemm = "grouped_gemm_kernel<2>"
    # 1 ms dispatches; 8 XCDs x 1.7 GHz x 1 ms = 13.6e6 counts
    rows = []
    for i in range(3):
        t0 = i * 10_000_000
        rows.append(_row(i, gemm, 720896, "GRBM_COUNT", 13.6e6, t0, t0 + 1_000_000))
        rows.append(_row(i, gemm, 720896, "GRBM_GUI_ACTIVE", 13.6e6, t0, t0 + 1_000_000))
    _write_counters(str(tmp_path / "c"), rows)
    bench.summarize_clock(str(tmp_path / "c"))
    line = [l for l in capsys.readouterr().out.splitlines() if l.startswith(gemm)][0]
    assert [float(v) for v in line.split()[-2:]] == [pytest.approx(1.7), pytest.approx(1.7)]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
