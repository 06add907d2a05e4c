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


SPIN = "void at::cuda::(anonymous namespace)::spin_kernel(long)"
S2H = "void basp::(anonymous namespace)::tile_kernel_staged<64, 1, 4, true, false>(basp::TileDesc)"
H2S = "void basp::(anonymous namespace)::tile_kernel<256, 16, 2, 4, false, true>(basp::TileDesc)"


def test_kernel_direction_from_its_template_arguments():
    """The direction is read from its position among the template arguments,
    not from the last one (the one-tensor flag follows it)."""
    assert bench._is_tile(S2H, True) and not bench._is_tile(S2H, False)
    assert bench._is_tile(H2S, False) and not bench._is_tile(H2S, True)
    fused_back = "void basp::(anonymous namespace)::tile_kernel<128, 16, 1, 4, false, false>(basp::TileDesc)"
    do_s2h = "void basp::(anonymous namespace)::tile_kernel_staged<256, 2, 4, true, true>(basp::TileDesc)"
    assert bench._is_tile(fused_back, False) and bench._is_tile(do_s2h, True)
    assert not bench._is_tile("basp::(anonymous namespace)::stream_copy_kernel(basp::CopyDesc)", True)
COPY = "__amd_rocclr_copyBuffer"
SCOPY = "basp::(anonymous namespace)::stream_copy_kernel(basp::(anonymous namespace)::CopyDesc)"


def test_pmc_summary_scales_by_the_copy(tmp_path):
    """Launches are taken from each mode's marked loop; the scale comes from
    the one copy between the third pair of markers (other copies, before and
    after, are ignored)."""
    cal_kib = bench.CALIB_BYTES / 1024
    # the fetch counter reads half of everything, the write counter all of it
    copies = [(SPIN, 0.0), (SCOPY, 3000.0), (SCOPY, 3000.0), (SPIN, 0.0),
              (SPIN, 0.0), (SCOPY, 2000.0), (SPIN, 0.0)]
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [(COPY, 5.0), (S2H, 3000.0), (SPIN, 0.0), (S2H, 1000.0), (H2S, 700.0),
                     (S2H, 1002.0), (H2S, 700.0), (S2H, 998.0), (SPIN, 0.0), (COPY, 9e6),
                     (SPIN, 0.0), (S2H, 2000.0), (H2S, 1400.0), (SPIN, 0.0)] + copies +
                    [(SPIN, 0.0), (COPY, cal_kib / 2), (SPIN, 0.0), (COPY, 9e9)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [(S2H, 5.0), (SPIN, 0.0), (S2H, 2000.0), (H2S, 1400.0), (SPIN, 0.0),
                     (SPIN, 0.0), (S2H, 4000.0), (H2S, 2800.0), (SPIN, 0.0)] + copies +
                    [(SPIN, 0.0), (COPY, cal_kib), (SPIN, 0.0)])
    out = bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), "w1")
    basp, uly = out["entries"]
    assert (basp["mode"], uly["mode"]) == ("basp", "ulysses") and basp["workload"] == "w1"
    f = basp["seq_to_head"]["FETCH_SIZE"]
    assert f["scale"] == pytest.approx(2.0) and f["launches"] == 3
    assert f["bytes_per_launch"] == pytest.approx(2000.0 * 1024)
    assert basp["seq_to_head"]["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(2000.0 * 1024)
    assert basp["traffic_bytes_per_launch"] == pytest.approx(4000.0 * 1024)
    assert basp["head_to_seq"]["traffic_bytes_per_launch"] == pytest.approx(2800.0 * 1024)
    assert uly["traffic_bytes_per_launch"] == pytest.approx(8000.0 * 1024)
    assert basp["kernel_sources_sha256"] == bench.kernel_sources_sha256()
    table = bench.counter_summary([str(tmp_path / "f"), str(tmp_path / "w")])
    assert table["basp seq->head"]["FETCH_SIZE"] == 1000.0 and table["ulysses head->seq"]["WRITE_SIZE"] == 2800.0
    assert table["copy at seq->head bytes"]["FETCH_SIZE"] == 3000.0
    assert table["copy at head->seq bytes"]["WRITE_SIZE"] == 2000.0


def test_trace_summary_per_mode(tmp_path):
    d = tmp_path / "t"
    os.makedirs(d)
    rows, t = [], 0
    for name, dur in [(S2H, 50), (SPIN, 1), (S2H, 100), (H2S, 60), (S2H, 102), (H2S, 62), (SPIN, 1),
                      (COPY, 5), (SPIN, 1), (S2H, 110), (H2S, 70), (SPIN, 1)]:
        rows.append({"Kernel_Name": name, "Start_Timestamp": t * 1000, "End_Timestamp": (t + dur) * 1000})
        t += dur + 1
    with open(d / "x_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    out = bench.trace_summary(str(d))
    assert out["basp"]["seq_to_head"]["avg_us"] == pytest.approx(101.0)
    assert out["basp"]["seq_to_head"]["launches"] == 2
    assert out["basp"]["head_to_seq"]["avg_us"] == pytest.approx(61.0)
    assert out["ulysses"]["seq_to_head"]["avg_us"] == pytest.approx(110.0)
    assert out["basp"]["avg_gap_us"] == pytest.approx(1.0)


def test_traffic_only_for_matching_sources_workload_mode_and_shapes(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    monkeypatch.setattr(bench, "launch_shape_key", lambda w, m: {"seq_to_head": {"stage": 2}} if m == "basp" else None)
    assert bench.traffic_bytes("w", "basp") is None
    good = {"workload": "w", "mode": "basp", "kernel_sources_sha256": bench.kernel_sources_sha256(),
            "launch_shape": {"seq_to_head": {"stage": 2}}, "traffic_bytes_per_launch": 123.0}
    uly = dict(good, mode="ulysses", launch_shape=None, traffic_bytes_per_launch=7.0)
    path.write_text(json.dumps({"entries": [good, uly]}))
    assert bench.traffic_bytes("w", "basp") == 123.0
    assert bench.traffic_bytes("w", "ulysses") == 7.0
    assert bench.traffic_bytes("other", "basp") is None
    path.write_text(json.dumps({"entries": [dict(good, launch_shape={"seq_to_head": {"stage": 1}})]}))
    assert bench.traffic_bytes("w", "basp") is None     # counters of other launch shapes
    path.write_text(json.dumps({"entries": [dict(good, kernel_sources_sha256="0" * 64)]}))
    assert bench.traffic_bytes("w", "basp") is None     # counters of other kernel sources


def _fake_run():
    sb, hb = 1342177280, 805306368

    def mode(G, P, Bl, s_us, h_us):
        return {"G": G, "P": P, "Bl": Bl, "peers_per_rank": P - 1, "ms_per_step": 0.33,
                "cross_rank_bytes_qkv": (P - 1) * (sb // 2) // P,
                "step_gbs": (sb + hb) / 0.33e-3 / 1e9, "s2h_bytes": sb, "h2s_bytes": hb,
                "s2h": {"avg_us": s_us, "median_us": s_us, "min_us": s_us, "max_us": s_us, "launches": 50},
                "h2s": {"avg_us": h_us, "median_us": h_us, "min_us": h_us, "max_us": h_us, "launches": 50},
                "s2h_gbs": sb / s_us / 1e3, "h2s_gbs": hb / h_us / 1e3, "rotate_sets": 2,
                "shape_source": "table", "tuning": {"seq_to_head": {"stage": 2, "block_size": 64},
                                                    "head_to_seq": {}}}
    return {"shape": (8, 2, 32768, 24, 8, 128), "name": "llama3.2-3b_s32k_b2",
            "modes": {"basp": mode(2, 4, 1, 203.0, 125.0), "ulysses": mode(1, 8, 2, 210.0, 126.0)},
            "copy": {"s2h_bytes_gbs": 6750.0, "h2s_bytes_gbs": 6700.0, "step_gbs": 6700.0},
            "round_trip_bit_exact": True}


def test_json_line_contract():
    """The bench line carries every field the benchmark contract names, with
    the roofline of the fused kernel against the 8 TB/s peak, and stays far
    below the few kilobytes of output a driver keeps (no GPU: fake
    measurements through the same assembly code)."""
    args = bench.parse_args(["--steps", "20", "--warmup", "5"])
    cpu = {"value": 11.0, "unit": "GB/s", "cores": 16, "kind": "oracle", "sample": "x" * 150,
           "seconds_per_step": 0.2, "cpu_model": "AMD EPYC 9575F 64-Core Processor", "one_thread_gbs": 1.2}
    line = bench.make_line(args, _fake_run(), 1342181000.0, cpu)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["unit"] == "GB/s" and line["higher_is_better"] is True
    assert line["steps"] == 20 and line["warmup"] == 5 and line["vs_baseline"] is None
    assert line["config"]["workload"] == "llama3.2-3b_s32k_b2" and "model" not in line["config"]
    # value is the fused seq->head rate of BASP mode, the roofline's achieved rate
    assert line["value"] == pytest.approx(1342177280 / 203.0 / 1e3)
    roof = line["roofline"]
    assert roof["achieved"] == line["value"] and roof["timed_launches"] >= 50
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(line["value"] / 8000.0) and roof["traffic"] == 1342181000.0
    assert set(line["basp_vs_ulysses"]) == {"basp", "ulysses"}
    assert line["basp_vs_ulysses"]["ulysses"]["P"] == 8
    # the exchange volume the two schemes differ in: (P-1)/P of the bytes read
    assert line["basp_vs_ulysses"]["basp"]["cross_rank_bytes_qkv"] == 503316480
    assert line["basp_vs_ulysses"]["ulysses"]["cross_rank_bytes_qkv"] == 587202560
    text = json.dumps(line)
    assert len(text) < 3000, len(text)
    assert "\n" not in text


def test_default_workload_is_the_largest_named_one():
    """The default workload moves the most bytes per fused call of the named
    evaluation shapes (the extra B = 16 data-parallel case is a parity and
    table case, not one of them)."""
    from sequence_re_layout_amd import workloads
    size = lambda w: w[2] * w[3] * (w[4] + 2 * w[5]) * w[6]
    assert max(workloads.ALL, key=size)[0] == bench.DEFAULT_WORKLOAD
    assert bench.parse_args([]).workload == bench.DEFAULT_WORKLOAD


def test_optional_leg_records_errors(capsys):
    """A leg after the timed region that raises is recorded in the JSON line
    instead of ending the run; one that works is returned as is."""
    assert bench.optional_leg(lambda: {"x": 1}) == {"x": 1}
    out = bench.optional_leg(lambda: 1 / 0)
    assert out == {"error": "ZeroDivisionError: division by zero"}
    assert "ZeroDivisionError" in capsys.readouterr().err
    json.dumps(out)


def test_sweep_grid_shapes_are_valid_tunings():
    """Every shape of the launch-shape sweep is a distinct tuning that the
    library accepts for both directions of the named workloads; staged shapes
    are single-pass tiles without a lane order, and the batch order varies
    only with more than one sequence."""
    from sequence_re_layout_amd import binding as b, workloads
    for B in (1, 2):
        grid = bench.sweep_grid(B)
        keys = {tuple(sorted(t.items())) for t in grid}
        assert len(keys) == len(grid)
        assert {t["batch_order"] for t in grid} == ({1} if B == 1 else {1, 2})
        for t in grid:
            if t["stage"] == 2:
                assert "tile_tokens" not in t and "lane_order" not in t
    for name, N, B, S, Hq, Hkv, d in (workloads.TINY, workloads.BY_NAME["llama3.2-1b_s8k_b1"]):
        p = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, b.BASP_MODE_BASP)
        for t in bench.sweep_grid(B):
            for direction in (b.BASP_SEQ_TO_HEAD, b.BASP_HEAD_TO_SEQ):
                b.basp_plan_set_direction_tuning(p, direction, **t)
                got = b.basp_plan_get_tuning(p, direction)
                assert all(got[k] == v for k, v in t.items())


def test_table_entries_set_every_size_dependent_field():
    """The built-in defaults of unset tuning fields depend on a call's size,
    so a table entry that left one unset could change kernels when those
    defaults change.  Every entry sets them all (lane order only matters to
    the direct kernel)."""
    from sequence_re_layout_amd import launch_shapes
    fields = ("vectors_per_thread", "block_size", "tile_heads", "tile_order", "xcd_remap")
    shapes = launch_shapes.table()["shapes"]
    assert shapes
    for name, modes in shapes.items():
        for mode, entry in modes.items():
            for direction in ("seq_to_head", "head_to_seq"):
                t = entry[direction]
                missing = [f for f in fields if not t.get(f)]
                if t.get("stage") != 2 and not t.get("lane_order"):
                    missing.append("lane_order")
                assert not missing, (name, mode, direction, missing)
