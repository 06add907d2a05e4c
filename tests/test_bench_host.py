"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the PMC counter
summary and its source-hash gate."""
import csv
import json
import os

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_pmc_summary_scales_by_the_copy(tmp_path):
    fused = "void basp::(anonymous namespace)::tile_kernel_staged<2, 3, true>(basp::TileDesc)"
    other = "void basp::(anonymous namespace)::tile_kernel<16, 2, 3, false>(basp::TileDesc)"
    copy = "__amd_rocclr_copyBuffer"
    cal_kib = bench.CALIB_BYTES / 1024
    # the fetch counter reads half of everything, the write counter all of it
    spin = "void at::cuda::(anonymous namespace)::spin_kernel(long)"
    # the fetch counter reads half of everything, the write counter all of it;
    # only launches between the two markers count
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(copy, 5.0), (fused, 3000.0), (spin, 0.0), (fused, 1000.0), (other, 7.0),
                     (fused, 1002.0), (fused, 998.0), (spin, 0.0), (copy, 1.5), (copy, cal_kib / 2), (copy, 9.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(fused, 5.0), (spin, 0.0), (fused, 2000.0), (spin, 0.0), (copy, cal_kib)])
    out = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"))
    assert out["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert out["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(2000.0 * 1024)
    assert out["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(2000.0 * 1024)
    assert out["traffic_bytes_per_launch"] == pytest.approx(4000.0 * 1024)
    assert out["kernel_sources_sha256"] == bench.kernel_sources_sha256()


def test_traffic_only_for_matching_sources_and_workload(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_bytes("w") is None
    path.write_text(json.dumps({"workload": "w", "kernel_sources_sha256": bench.kernel_sources_sha256(),
                                "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_bytes("w") == 123.0
    assert bench.traffic_bytes("other") is None
    path.write_text(json.dumps({"workload": "w", "kernel_sources_sha256": "0" * 64,
                                "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_bytes("w") is None
