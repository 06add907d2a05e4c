"""Host-side pieces of bench.py (no GPU): the one-GPU guard, the PMC counter
summary and its source-hash gate, and the fields of the JSON line."""
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
    assert bench.traffic_bytes("w", "basp") is None
    path.write_text(json.dumps({"workload": "w", "mode": "basp", "kernel_sources_sha256": bench.kernel_sources_sha256(),
                                "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_bytes("w", "basp") == 123.0
    assert bench.traffic_bytes("other", "basp") is None
    assert bench.traffic_bytes("w", "ulysses") is None   # counters of the other mode
    path.write_text(json.dumps({"workload": "w", "mode": "basp", "kernel_sources_sha256": "0" * 64,
                                "traffic_bytes_per_launch": 123.0}))
    assert bench.traffic_bytes("w", "basp") is None


def test_json_line_contract():
    """The bench line carries every field the benchmark contract names, with
    the roofline of the fused kernel against the 8 TB/s peak (no GPU: fake
    measurements through the same assembly code)."""
    import types
    args = bench.parse_args([])
    sb, hb = 402653184, 268435456
    r = {"value": 6300.0, "ms_per_step": 0.1065, "rotate_sets": 5, "step_bytes": sb + hb,
         "tuning": {"seq_to_head": {}, "head_to_seq": {}, "autotuned": True},
         "s2h_gbs": 6400.0, "h2s_gbs": 6370.0, "s2h_bytes": sb, "h2s_bytes": hb,
         "s2h_avg_us": 62.9, "h2s_avg_us": 42.1, "timed_launches_per_kernel": 50,
         "copy_ceiling": {str(sb): {"gbs": 6790.0}, str(hb): {"gbs": 6690.0}},
         "copy_loop": {"step_gbs": 6620.0, "s2h_bytes_gbs": 6550.0, "h2s_bytes_gbs": 6590.0, "steps": 200},
         "round_trip_bit_exact": True}
    w = types.SimpleNamespace(shape=(8, 2, 16384, 32, 8, 64), name="llama3.2-1b_s16k_b2", mode="basp")
    line = bench.make_line(args, r, w, 402657919.0)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["unit"] == "GB/s" and line["higher_is_better"] is True
    assert line["steps"] == 500 and line["warmup"] == 50 and line["vs_baseline"] is None
    assert line["config"]["workload"] == "llama3.2-1b_s16k_b2" and "model" not in line["config"]
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - 0.8) < 1e-12 and roof["traffic"] == 402657919.0
    assert line["copy_ceiling"]["in_timed_loop"]["step_frac_of_copy"] == 6300.0 / 6620.0
    json.dumps(line)   # serialisable



def test_optional_leg_records_errors(capsys):
    """A leg after the timed region that raises is recorded in the JSON line
    instead of ending the run; one that works is returned as is."""
    assert bench.optional_leg(lambda: {"x": 1}) == {"x": 1}
    out = bench.optional_leg(lambda: 1 / 0)
    assert out == {"error": "ZeroDivisionError: division by zero"}
    assert "ZeroDivisionError" in capsys.readouterr().err
    json.dumps(out)
