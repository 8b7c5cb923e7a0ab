"""Host logic of the benchmark (no GPU): the counter records' arithmetic and
the source hash that keys them."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_record_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    gib_kib = bench.COPY_BYTES / 1024.0
    # the copy's counters read half the bytes fetched and all the bytes written
    _csv(tmp_path / "cf.csv", [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                                "Counter_Value": gib_kib / 2}])
    _csv(tmp_path / "cw.csv", [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                                "Counter_Value": gib_kib}])
    # two dispatches of the kernel (mean taken), another kernel ignored
    _csv(tmp_path / "kf.csv", [{"Kernel_Name": "void q4::k_x<1>(int)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
                               {"Kernel_Name": "void q4::k_x<1>(int)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
                               {"Kernel_Name": "void q4::k_y(int)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1e9}])
    _csv(tmp_path / "kw.csv", [{"Kernel_Name": "void q4::k_x<1>(int)", "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0}])
    e = bench.record_traffic("sweep", "k_x<1>", str(tmp_path / "kf.csv"), str(tmp_path / "kw.csv"),
                             str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"))
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["fetch_bytes"] == 200 * 1024 * 2 and e["write_bytes"] == 10 * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    table = json.load(open(tmp_path / "traffic.json"))
    assert table["sweep"]["source_hash"] == bench.kernel_source_hash("sweep")
    assert bench.counter_traffic("sweep") == e["bytes_per_launch"]


def test_counter_record_goes_stale_with_its_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    with open(tmp_path / "traffic.json", "w") as f:
        json.dump({"q8": {"source_hash": "0" * 16, "bytes_per_launch": 5}}, f)
    assert bench.counter_traffic("q8") is None
    with open(tmp_path / "traffic.json", "w") as f:
        json.dump({"q8": {"source_hash": bench.kernel_source_hash("q8"), "bytes_per_launch": 5}}, f)
    assert bench.counter_traffic("q8") == 5
    assert bench.counter_traffic("smallm_m4") is None  # no record


def test_source_hash_follows_each_workloads_kernel_files():
    # every workload names existing sources, and each workload's hash is stable
    for w in bench.KERNEL_SOURCE:
        assert bench.kernel_source_hash(w) == bench.kernel_source_hash(w)
    assert bench.kernel_source_hash("smallm_m2") == bench.kernel_source_hash("smallm_m16")
    assert bench.kernel_source_hash("q8") != bench.kernel_source_hash("sweep")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
