#!/usr/bin/env python3
"""Benchmark of the BASP attention-boundary re-layout on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--mode basp|ulysses]

One step is one pass of the attention-boundary re-layout of a layer: the
fused Q/K/V seq->head exchange before attention and the O head->seq exchange
after it, on the Llama-3.2-1B-shaped workload by default (N = 8 virtual
ranks, B = 2, S = 16384, Hq = 32, Hkv = 8, d = 64, bf16, BASP mode: 2 groups
of K = 4).  Inputs are seeded synthetic N(0, 1) bf16 values resident in HBM
before timing starts; R buffer sets rotate so that no step finds its bytes in
the 256 MB Infinity Cache.  Each plan's launch shapes are chosen by
basp_plan_autotune before anything is timed (--no-autotune keeps the
built-in ones).

Printed: one JSON line.  ``value`` is effective HBM GB/s of the whole step
(algorithmic bytes: every input byte read once, every output byte written
once) over wall time of K steps bracketed by device synchronisation.
``roofline`` is the fused seq->head kernel (the larger of the two) against
the 8 TB/s HBM peak, its duration taken from HIP events that its own launch
records (hipExtLaunchKernel start/stop timestamps, via basp_time_next_call)
on the stream it runs on, on every --sample-every'th step of the timed
region.  ``detail`` holds per-kernel rates of both modes, the unfused
three-pass baseline, the backward entry points, the token-major layout and
torch's device copy; ``workloads`` the fused seq->head and head->seq rates of
every named workload in both modes.  ``copy_ceiling`` is basp_stream_copy,
a plain copy with the kernels' access rules, at the same byte counts: the
rate a read-once, write-once kernel reaches on this part.  ``cpu_baseline``
is the CPU oracle doing the same step on the host, repeated for about
--cpu-seconds.

    python bench.py --pmc-summary FETCH_DIR WRITE_DIR

reads the CSV output of two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc
WRITE_SIZE`` runs of this script and writes ``profiles/pmc_traffic.json``
(HBM bytes per launch of the fused kernel, scaled by the same counters on a
plain copy of known size).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("effective HBM GB/s (and % of peak) of fused QKV seq→head re-layout, "
          "BASP vs Ulysses")
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["sequence_re_layout_amd/csrc/relayout.hip", "sequence_re_layout_amd/csrc/launch.hpp",
                  "sequence_re_layout_amd/csrc/launch.cpp", "sequence_re_layout_amd/csrc/fastdiv.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CALIB_BYTES = 256 << 20   # plain copy used to scale the PMC byte counters
MARKER_CYCLES = 1000      # torch's spin kernel, brackets the timed region


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sample-every", type=int, default=10,
                    help="time the kernels of every n-th timed step with their own events")
    ap.add_argument("--workload", default="llama3.2-1b_s16k_b2")
    ap.add_argument("--mode", choices=["basp", "ulysses"], default="basp")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: enough for > 1 GiB reuse distance)")
    ap.add_argument("--detail-iters", type=int, default=100)
    ap.add_argument("--no-autotune", action="store_true",
                    help="keep the built-in launch shapes instead of measuring them per plan")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the table of every named workload")
    ap.add_argument("--workload-steps", type=int, default=60,
                    help="least launches per HIP graph in the table of every workload")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    return ap.parse_args(argv)


# ------------------------------------------------------------------ GPU ---

class Workload:
    """Device buffers of one workload: R rotating sets of Q/K/V/out and
    O/out, filled from the same seeded host data."""

    def __init__(self, b, name, mode, rotate, autotune=True):
        import torch
        from sequence_re_layout_amd import inputs, workloads
        self.name, N, B, S, Hq, Hkv, d = workloads.BY_NAME[name]
        self.shape = (N, B, S, Hq, Hkv, d)
        self.mode = mode
        code = b.BASP_MODE_BASP if mode == "basp" else b.BASP_MODE_ULYSSES
        self.plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
        i = self.plan.info
        self.s2h_bytes = i["qkv_bytes_moved"]
        self.h2s_bytes = i["o_bytes_moved"]
        self.host = {
            "q": inputs.normal_bf16(i["q_elems"], inputs.SEED_Q),
            "k": inputs.normal_bf16(i["kv_elems"], inputs.SEED_K),
            "v": inputs.normal_bf16(i["kv_elems"], inputs.SEED_V),
            "o": inputs.normal_bf16(i["q_elems"], inputs.SEED_O),
        }
        set_bytes = self.s2h_bytes + self.h2s_bytes
        self.R = rotate or max(2, -(-(3 << 30) // set_bytes))   # > 1 GiB between reuses
        self.sets = []
        for _ in range(self.R):
            s = {n: t.cuda() for n, t in self.host.items()}
            s["qkv_out"] = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
            s["o_out"] = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
            self.sets.append(s)
        torch.cuda.synchronize()
        self.autotune_seconds = None
        if autotune:   # plan-time measurement, before anything is timed
            s = self.sets[0]
            t0 = time.perf_counter()
            b.basp_plan_autotune(self.plan, s["q"], s["k"], s["v"], s["qkv_out"], s["o"], s["o_out"])
            torch.cuda.synchronize()
            self.autotune_seconds = time.perf_counter() - t0


def make_events(n):
    """n timing events whose handles exist (torch creates them on first record)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    return ev


def time_launches(b, fn, n, rotate):
    """Durations (s) of n calls of fn(set_index), each timed from its kernels'
    own dispatch timestamps (basp_time_next_call) on the launch stream."""
    import torch
    ev = make_events(2 * n)
    for i in range(n):
        b.basp_time_next_call(ev[2 * i], ev[2 * i + 1])
        fn(i % rotate)
    torch.cuda.synchronize()
    return [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e-3 for i in range(n)]


def time_torch(fn, n, rotate):
    """Durations (s) of n calls of a torch op, bracketed by events on torch's
    current stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        fn(i % rotate)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(z) * 1e-3 for a, z in ev]


def rate(nbytes, seconds):
    return nbytes / seconds / 1e9


def run_gpu(args):
    import torch
    from sequence_re_layout_amd import binding as b

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count, "memory_bytes": props.total_memory}
    w = Workload(b, args.workload, args.mode, args.rotate, not args.no_autotune)
    plan, sets = w.plan, w.sets

    def s2h(i):
        s = sets[i]
        b.basp_seq_to_head(plan, s["q"], s["k"], s["v"], s["qkv_out"])

    def h2s(i):
        s = sets[i]
        b.basp_head_to_seq(plan, s["o"], s["o_out"])

    for i in range(args.warmup):
        s2h(i % w.R)
        h2s(i % w.R)
    torch.cuda.synchronize()

    # timed region: K steps.  Every --sample-every'th step carries start/stop
    # events recorded by its kernels' own dispatches (basp_time_next_call):
    # such a launch costs the stream about 5 us more, so timing every launch
    # would slow the step the bench reports.  A tiny marker kernel before and
    # after the region lets a profiler trace find the timed launches among
    # the plan-time measurements.
    every = max(1, args.sample_every)
    sampled = list(range(0, args.steps, every))
    ev = make_events(4 * len(sampled))
    torch.cuda._sleep(MARKER_CYCLES)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        j = i // every if i % every == 0 else -1
        if j >= 0:
            b.basp_time_next_call(ev[4 * j], ev[4 * j + 1])
        s2h(i % w.R)
        if j >= 0:
            b.basp_time_next_call(ev[4 * j + 2], ev[4 * j + 3])
        h2s(i % w.R)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    torch.cuda._sleep(MARKER_CYCLES)
    s2h_t = [ev[4 * j].elapsed_time(ev[4 * j + 1]) * 1e-3 for j in range(len(sampled))]
    h2s_t = [ev[4 * j + 2].elapsed_time(ev[4 * j + 3]) * 1e-3 for j in range(len(sampled))]

    ms_per_step = wall / args.steps * 1e3
    step_bytes = w.s2h_bytes + w.h2s_bytes
    s2h_avg = statistics.mean(s2h_t)
    res = {
        "ms_per_step": ms_per_step,
        "value": rate(step_bytes, wall / args.steps),
        "step_bytes": step_bytes,
        "rotate_sets": w.R,
        "timed_launches_per_kernel": len(sampled),
        "s2h_avg_us": s2h_avg * 1e6,
        "s2h_median_us": statistics.median(s2h_t) * 1e6,
        "s2h_min_us": min(s2h_t) * 1e6,
        "s2h_max_us": max(s2h_t) * 1e6,
        "h2s_avg_us": statistics.mean(h2s_t) * 1e6,
        "h2s_median_us": statistics.median(h2s_t) * 1e6,
        "h2s_min_us": min(h2s_t) * 1e6,
        "h2s_max_us": max(h2s_t) * 1e6,
        "s2h_bytes": w.s2h_bytes,
        "h2s_bytes": w.h2s_bytes,
        "s2h_gbs": rate(w.s2h_bytes, s2h_avg),
        "h2s_gbs": rate(w.h2s_bytes, statistics.mean(h2s_t)),
    }

    # the ceiling: basp_stream_copy (a plain read-once/write-once copy with
    # the same access rules) at the byte counts of the two kernels, timed the
    # same way on rotating buffers: each launch alone, and as the timed
    # region runs them (back to back, every --sample-every'th step sampled)
    res["copy_ceiling"] = copy_ceiling(b, (w.s2h_bytes, w.h2s_bytes), 100)
    res["copy_loop"] = copy_loop(b, w.s2h_bytes, w.h2s_bytes, 200, every)

    # device round trip of the timed buffers: head->seq of the Q part of the
    # fused output must give Q back bit for bit
    s = sets[0]
    back = torch.empty_like(s["q"])
    b.basp_seq_to_head(plan, s["q"], s["k"], s["v"], s["qkv_out"])
    b.basp_head_to_seq(plan, s["qkv_out"][: plan.info["q_elems"]], back)
    torch.cuda.synchronize()
    res["round_trip_bit_exact"] = bool(torch.equal(back.view(torch.int16), s["q"].view(torch.int16)))

    # a plain copy of known size: the PMC byte counters are scaled by it
    cal_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    cal_dst = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # the legs after the timed region are reported, not required: an error in
    # one is recorded in its place and the line is still printed
    if not args.no_detail:
        res["detail"] = optional_leg(lambda: detail(args, b, w))
    if not args.no_workloads:
        res["workloads"] = optional_leg(lambda: workload_table(b, args.workload_steps, not args.no_autotune))
    res["tuning"] = {"seq_to_head": b.basp_plan_get_tuning(plan, b.BASP_SEQ_TO_HEAD),
                     "head_to_seq": b.basp_plan_get_tuning(plan, b.BASP_HEAD_TO_SEQ),
                     "autotuned": not args.no_autotune, "autotune_seconds": w.autotune_seconds}
    res["w"] = w
    res["device"] = device
    return res


def optional_leg(fn):
    """fn(), or {"error": ...} when it raises (after reporting it on stderr)."""
    try:
        return fn()
    except Exception as e:   # noqa: BLE001 -- recorded in the JSON line
        import traceback
        traceback.print_exc()
        return {"error": "%s: %s" % (type(e).__name__, e)}


def copy_ceiling(b, moved, n):
    """Average duration and rate of basp_stream_copy moving each byte count
    in `moved` (read + write: a copy of moved/2 bytes), n timed launches each
    on buffer sets more than 1 GiB apart."""
    import torch
    out = {}
    for m in moved:
        nb = m // 2
        R = max(2, -(-(3 << 30) // m))
        src = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(R)]
        dst = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(R)]
        for i in range(R):
            b.basp_stream_copy(dst[i], src[i])
        t = time_launches(b, lambda i: b.basp_stream_copy(dst[i], src[i]), n, R)
        out[str(m)] = {"bytes_moved": m, "avg_us": statistics.mean(t) * 1e6,
                       "median_us": statistics.median(t) * 1e6, "gbs": rate(m, statistics.mean(t))}
        del src, dst
        torch.cuda.empty_cache()
    return out


def loop_rates(b, s_fn, h_fn, R, steps, every):
    """Run steps of s_fn(i) then h_fn(i) back to back on rotating sets i % R,
    as the timed region runs the kernels, with the launches of every
    `every`-th step timed by their own events.  Returns the wall seconds per
    step and the sampled launches' average seconds."""
    import torch
    for i in range(min(R, 10)):
        s_fn(i % R)
        h_fn(i % R)
    sampled = list(range(0, steps, every))
    ev = make_events(4 * len(sampled) + 2)
    ev[-2].record()
    for i in range(steps):
        if i % every == 0:
            j = i // every
            b.basp_time_next_call(ev[4 * j], ev[4 * j + 1])
            s_fn(i % R)
            b.basp_time_next_call(ev[4 * j + 2], ev[4 * j + 3])
            h_fn(i % R)
        else:
            s_fn(i % R)
            h_fn(i % R)
    ev[-1].record()
    torch.cuda.synchronize()
    wall = ev[-2].elapsed_time(ev[-1]) * 1e-3 / steps
    s_t = statistics.mean(ev[4 * j].elapsed_time(ev[4 * j + 1]) * 1e-3 for j in range(len(sampled)))
    h_t = statistics.mean(ev[4 * j + 2].elapsed_time(ev[4 * j + 3]) * 1e-3 for j in range(len(sampled)))
    return wall, s_t, h_t


def copy_loop(b, s_bytes, h_bytes, steps, every):
    """basp_stream_copy at the two kernels' byte counts run the way the timed
    region runs the kernels (loop_rates).  Returns the step rate and the
    sampled launches' average rates."""
    import torch
    R = max(2, -(-(3 << 30) // (s_bytes + h_bytes)))
    bufs = [(torch.empty(s_bytes // 2, dtype=torch.uint8, device="cuda"),
             torch.empty(s_bytes // 2, dtype=torch.uint8, device="cuda"),
             torch.empty(h_bytes // 2, dtype=torch.uint8, device="cuda"),
             torch.empty(h_bytes // 2, dtype=torch.uint8, device="cuda")) for _ in range(R)]
    wall, s_t, h_t = loop_rates(b, lambda i: b.basp_stream_copy(bufs[i][1], bufs[i][0]),
                                lambda i: b.basp_stream_copy(bufs[i][3], bufs[i][2]), R, steps, every)
    del bufs
    torch.cuda.empty_cache()
    return {"step_gbs": rate(s_bytes + h_bytes, wall), "s2h_bytes_gbs": rate(s_bytes, s_t),
            "h2s_bytes_gbs": rate(h_bytes, h_t), "steps": steps}


def graph_step(b, w, steps_per_graph=10, replays=20):
    """The same step replayed from a HIP graph: steps_per_graph steps over
    the rotating buffer sets are captured once (the entry points only launch
    kernels, so they capture), then replayed; the rate over all replays,
    between two events, against the eager loop's."""
    import torch
    plan, sets = w.plan, w.sets
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(steps_per_graph):
            s = sets[i % w.R]
            b.basp_seq_to_head(plan, s["q"], s["k"], s["v"], s["qkv_out"])
            b.basp_head_to_seq(plan, s["o"], s["o_out"])
    graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    seconds = start.elapsed_time(stop) * 1e-3 / (replays * steps_per_graph)
    del graph
    return {"steps": replays * steps_per_graph, "us_per_step": seconds * 1e6,
            "gbs": rate(w.s2h_bytes + w.h2s_bytes, seconds)}


def detail(args, b, w):
    """Per-kernel rates of both modes, the unfused baseline, the backward
    entry points, the token-major layout and a plain device copy."""
    import torch
    out = {}
    n = args.detail_iters
    med = statistics.median
    for mode in ("basp", "ulysses"):
        ww = w if mode == w.mode else Workload(b, w.name, mode, w.R, not args.no_autotune)
        p, sets = ww.plan, ww.sets
        t = time_launches(b, lambda i: b.basp_seq_to_head(p, sets[i]["q"], sets[i]["k"], sets[i]["v"],
                                                          sets[i]["qkv_out"]), n, ww.R)
        u = time_launches(b, lambda i: b.basp_head_to_seq(p, sets[i]["o"], sets[i]["o_out"]), n, ww.R)
        info = p.info
        out[mode] = {
            "G": info["G"], "P": info["P"], "Bl": info["Bl"], "peers_per_rank": info["peers_per_rank"],
            "cross_rank_bytes_qkv": info["cross_rank_bytes_q"] + 2 * info["cross_rank_bytes_kv"],
            "s2h_median_us": med(t) * 1e6,
            "s2h_gbs": rate(ww.s2h_bytes, med(t)),
            "s2h_frac_of_peak": rate(ww.s2h_bytes, med(t)) / HBM_PEAK_GBS,
            "h2s_median_us": med(u) * 1e6,
            "h2s_gbs": rate(ww.h2s_bytes, med(u)),
            "h2s_frac_of_peak": rate(ww.h2s_bytes, med(u)) / HBM_PEAK_GBS,
        }
        if mode == w.mode:
            ws = torch.empty(b.basp_unfused_workspace_bytes(p), dtype=torch.uint8, device="cuda")
            f = time_launches(b, lambda i: b.basp_seq_to_head_unfused(
                p, sets[i]["q"], sets[i]["k"], sets[i]["v"], sets[i]["qkv_out"], ws), max(10, n // 4), ww.R)
            out[mode]["s2h_unfused_median_us"] = med(f) * 1e6
            out[mode]["s2h_unfused_gbs"] = rate(ww.s2h_bytes, med(f))
            del ws
            # backward: dO seq->head (O-shaped, reuses the O buffers) and the
            # fused dQ/dK/dV head->seq (reads the fused buffer, writes q/k/v-shaped)
            grads = [{"dq": torch.empty_like(s["q"]), "dk": torch.empty_like(s["k"]),
                      "dv": torch.empty_like(s["v"])} for s in sets]
            bo = time_launches(b, lambda i: b.basp_seq_to_head_o(p, sets[i]["o"], sets[i]["o_out"]), n, ww.R)
            bq = time_launches(b, lambda i: b.basp_head_to_seq_qkv(
                p, sets[i]["qkv_out"], grads[i]["dq"], grads[i]["dk"], grads[i]["dv"]), n, ww.R)
            out[mode]["backward"] = {
                "do_s2h_gbs": rate(ww.h2s_bytes, med(bo)), "do_s2h_median_us": med(bo) * 1e6,
                "dqkv_h2s_gbs": rate(ww.s2h_bytes, med(bq)), "dqkv_h2s_median_us": med(bq) * 1e6}
            del grads
            # head shards in token-major order ([Bl][S][Hl][d])
            N, B, S, Hq, Hkv, d = ww.shape
            pt = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_BF16,
                                       b.BASP_MODE_BASP if mode == "basp" else b.BASP_MODE_ULYSSES,
                                       b.BASP_LAYOUT_TOKEN_MAJOR)
            if not args.no_autotune:
                s0 = sets[0]
                b.basp_plan_autotune(pt, s0["q"], s0["k"], s0["v"], s0["qkv_out"], s0["o"], s0["o_out"])
            tt = time_launches(b, lambda i: b.basp_seq_to_head(pt, sets[i]["q"], sets[i]["k"], sets[i]["v"],
                                                               sets[i]["qkv_out"]), n, ww.R)
            tu = time_launches(b, lambda i: b.basp_head_to_seq(pt, sets[i]["o"], sets[i]["o_out"]), n, ww.R)
            out[mode]["token_major"] = {"s2h_gbs": rate(ww.s2h_bytes, med(tt)),
                                        "h2s_gbs": rate(ww.h2s_bytes, med(tu))}
        if ww is not w:
            del ww
            torch.cuda.empty_cache()
    out["graph_step"] = graph_step(b, w)
    # plain device copy of the same byte count (read + write), and the
    # known-size copy the PMC counters are scaled by
    nb = w.s2h_bytes // 2
    src = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(4)]
    dst = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(4)]
    c = time_torch(lambda i: dst[i].copy_(src[i]), n, 4)
    out["device_copy"] = {"bytes_moved": 2 * nb, "median_us": med(c) * 1e6,
                          "gbs": rate(2 * nb, med(c))}
    del src, dst
    return out


def graph_seconds(fn, calls, reps=5):
    """Seconds per call of `calls` back-to-back calls fn(i), captured once in a
    HIP graph so that no host gap falls between the kernels (a small call runs
    for less time than a Python call takes); median over `reps` replays."""
    import torch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(calls):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    start, stop = make_events(2)
    t = []
    for _ in range(reps):
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        t.append(start.elapsed_time(stop) * 1e-3 / calls)
    del graph
    return statistics.median(t)


def workload_table(b, steps, autotune):
    """Fused seq->head and head->seq rates of every named workload in both
    modes (device-filled random bf16: the rate does not depend on values).
    Each rate is a HIP graph of back-to-back launches on rotating buffer sets
    (graph_seconds): whole steps, then each direction alone; at least `steps`
    launches per graph, more for small calls.  Once per workload, the plain
    copy pair at the same byte counts, run the same way."""
    import torch
    from sequence_re_layout_amd import workloads
    out = {}
    for (name, N, B, S, Hq, Hkv, d) in workloads.ALL + workloads.EXTRA:
        out[name] = {}
        for mode, code in (("basp", b.BASP_MODE_BASP), ("ulysses", b.BASP_MODE_ULYSSES)):
            p = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
            i = p.info
            sb, hb = i["qkv_bytes_moved"], i["o_bytes_moved"]
            R = max(2, -(-(3 << 30) // (sb + hb)))
            n = max(steps, min(10 * steps, steps * (400 << 20) // sb))
            sets = []
            for _ in range(R):
                x = torch.empty(2 * i["q_elems"] + 2 * i["kv_elems"], dtype=torch.bfloat16, device="cuda").normal_()
                sets.append({"x": x, "q": x[:i["q_elems"]], "k": x[i["q_elems"]:i["q_elems"] + i["kv_elems"]],
                             "v": x[i["q_elems"] + i["kv_elems"]:i["q_elems"] + 2 * i["kv_elems"]],
                             "o": x[i["q_elems"] + 2 * i["kv_elems"]:],
                             "out": torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda"),
                             "o_out": torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")})
            if autotune:
                b.basp_plan_autotune(p, sets[0]["q"], sets[0]["k"], sets[0]["v"], sets[0]["out"],
                                     sets[0]["o"], sets[0]["o_out"])

            def s2h(j):
                s = sets[j % R]
                b.basp_seq_to_head(p, s["q"], s["k"], s["v"], s["out"])

            def h2s(j):
                s = sets[j % R]
                b.basp_head_to_seq(p, s["o"], s["o_out"])

            wall = graph_seconds(lambda j: (s2h(j), h2s(j)), n)
            t, u = graph_seconds(s2h, n), graph_seconds(h2s, n)
            out[name][mode] = {
                "G": i["G"], "P": i["P"], "Bl": i["Bl"], "peers_per_rank": i["peers_per_rank"],
                "launches_per_graph": n, "step_gbs": rate(sb + hb, wall),
                "s2h_bytes": sb, "s2h_us": t * 1e6, "s2h_gbs": rate(sb, t), "s2h_frac": rate(sb, t) / HBM_PEAK_GBS,
                "h2s_bytes": hb, "h2s_us": u * 1e6, "h2s_gbs": rate(hb, u), "h2s_frac": rate(hb, u) / HBM_PEAK_GBS,
                "launch_shape": {"seq_to_head": b.basp_plan_get_tuning(p, b.BASP_SEQ_TO_HEAD),
                                 "head_to_seq": b.basp_plan_get_tuning(p, b.BASP_HEAD_TO_SEQ)}}
            if mode == "basp":   # both modes move the same bytes: one copy pair per workload
                qkv_b, o_b = sb // 2, hb // 2

                def cs(j):
                    b.basp_stream_copy(sets[j % R]["out"], sets[j % R]["x"], qkv_b)

                def ch(j):
                    b.basp_stream_copy(sets[j % R]["o_out"], sets[j % R]["x"], o_b)

                cw = graph_seconds(lambda j: (cs(j), ch(j)), n)
                tc, uc = graph_seconds(cs, n), graph_seconds(ch, n)
                out[name]["copy"] = {"s2h_bytes_gbs": rate(2 * qkv_b, tc), "h2s_bytes_gbs": rate(2 * o_b, uc),
                                     "step_gbs": rate(2 * (qkv_b + o_b), cw)}
            del sets
            torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ CPU ---

def cpu_baseline(args, w):
    """The oracle doing one step (fused Q/K/V seq->head, O head->seq) on the
    host bytes of the same workload, repeated for about --cpu-seconds."""
    import numpy as np

    import oracle
    from sequence_re_layout_amd import inputs
    N, B, S, Hq, Hkv, d = w.shape
    mode = oracle.BASP if w.mode == "basp" else oracle.ULYSSES
    q, k, v, o = (inputs.raw_bits(w.host[n]) for n in ("q", "k", "v", "o"))
    threads = oracle.max_threads()
    reps, spent = 0, 0.0
    while reps == 0 or spent < args.cpu_seconds:
        t0 = time.perf_counter_ns()
        oracle.seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, threads=threads)
        oracle.head_to_seq(o, mode, N, B, S, Hq, d, threads=threads)
        spent += (time.perf_counter_ns() - t0) * 1e-9
        reps += 1
    step_bytes = w.s2h_bytes + w.h2s_bytes
    # for information: the same step as one NumPy transpose per tensor
    reps_np, spent_np = 0, 0.0
    while reps_np == 0 or spent_np < args.cpu_seconds / 4:
        t0 = time.perf_counter_ns()
        np.concatenate([oracle.numpy_seq_to_head(x, mode, N, B, S, H, d)
                        for x, H in ((q, Hq), (k, Hkv), (v, Hkv))])
        oracle.numpy_head_to_seq(o, mode, N, B, S, Hq, d)
        spent_np += (time.perf_counter_ns() - t0) * 1e-9
        reps_np += 1
    # the same loop on one thread, for a shorter while
    reps1, spent1 = 0, 0.0
    while reps1 == 0 or spent1 < args.cpu_seconds / 4:
        t0 = time.perf_counter_ns()
        oracle.seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, threads=1)
        oracle.head_to_seq(o, mode, N, B, S, Hq, d, threads=1)
        spent1 += (time.perf_counter_ns() - t0) * 1e-9
        reps1 += 1
    return {"value": rate(step_bytes * reps, spent), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s) of the same workload (fused QKV seq->head + O head->seq), "
                      "%.1f s on the host, OpenMP over destination blocks" % (reps, spent),
            "seconds_per_step": spent / reps, "cpu_model": cpu_model(),
            "one_thread": {"value": rate(step_bytes * reps1, spent1), "unit": "GB/s",
                           "seconds_per_step": spent1 / reps1, "steps": reps1},
            "numpy_transpose": {"value": rate(step_bytes * reps_np, spent_np), "unit": "GB/s",
                                "seconds_per_step": spent_np / reps_np, "steps": reps_np,
                                "note": "the same step as one NumPy transpose per tensor, for information"}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------ roofline ---

def traffic_bytes(workload, mode):
    """HBM bytes per fused seq->head launch from committed PMC counters, or
    None when they are missing, were taken on other kernel sources, or on
    another workload or mode."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_sources_sha256") != kernel_sources_sha256() or t.get("workload") != workload
            or t.get("mode") != mode):
        return None
    return t.get("traffic_bytes_per_launch")


def pmc_summary(fetch_dir, write_dir):
    """Per-launch FETCH_SIZE/WRITE_SIZE of the fused kernel, scaled by the same
    counter on the known-size copy, into profiles/pmc_traffic.json."""

    def load(d, counter):
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                rows += [r for r in csv.DictReader(f) if r.get("Counter_Name") == counter]
        if not rows:
            raise SystemExit("no %s rows under %s" % (counter, d))
        return sorted(rows, key=lambda r: int(r["Dispatch_Id"]))

    out = {"workload": None, "kernel_sources_sha256": kernel_sources_sha256()}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = load(d, counter)
        # the timed launches: between the two marker kernels of the run
        marks = [i for i, r in enumerate(rows) if "spin_kernel" in r["Kernel_Name"]]
        if len(marks) < 2:
            raise SystemExit("no timed-region markers for %s" % counter)
        timed = rows[marks[0] + 1:marks[1]]
        # the fused seq->head kernel: tile_kernel<VW, VPT, POLICY, true> or
        # tile_kernel_staged<VPT, POLICY, true>
        fused = [r for r in timed if "tile_kernel" in r["Kernel_Name"] and "true>" in r["Kernel_Name"]]
        copies = [r for r in rows[marks[1]:] if "copy" in r["Kernel_Name"].lower()
                  and "stream_copy_kernel" not in r["Kernel_Name"]]
        if not fused or not copies:
            raise SystemExit("missing fused or copy dispatches for %s" % counter)
        # the calibration copy: the largest copy after the timed region (small
        # copies bring results back to the host)
        cal_row = max(copies, key=lambda r: float(r["Counter_Value"]))
        cal = float(cal_row["Counter_Value"])
        factor = (CALIB_BYTES / 1024.0) / cal
        kib = statistics.median(float(r["Counter_Value"]) for r in fused)
        out["kernel"] = fused[0]["Kernel_Name"]
        out[counter] = {"kib_per_launch_raw": kib, "kernel_name": fused[0]["Kernel_Name"],
                        "copy_kernel": cal_row["Kernel_Name"],
                        "copy_kib_raw": cal, "scale": factor,
                        "bytes_per_launch": kib * factor * 1024.0, "launches": len(fused)}
        # the head->seq kernel of the same steps, for reference
        back = [r for r in timed if "tile_kernel" in r["Kernel_Name"] and "false>" in r["Kernel_Name"]]
        if back:
            kb = statistics.median(float(r["Counter_Value"]) for r in back)
            out.setdefault("head_to_seq", {})[counter] = {
                "kib_per_launch_raw": kb, "kernel_name": back[0]["Kernel_Name"],
                "bytes_per_launch": kb * factor * 1024.0, "launches": len(back)}
    out["traffic_bytes_per_launch"] = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    if len(out.get("head_to_seq", {})) == 2:
        h = out["head_to_seq"]
        h["traffic_bytes_per_launch"] = h["FETCH_SIZE"]["bytes_per_launch"] + h["WRITE_SIZE"]["bytes_per_launch"]
    return out


# ---------------------------------------------------------------- main ---

def make_line(args, r, w, traffic):
    """The JSON line's fields from the measurements r of run_gpu and the
    workload w (its shape, name and mode); traffic is the HBM bytes per fused
    launch from the committed counters, or None."""
    N, B, S, Hq, Hkv, d = w.shape
    line = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V/O, resident in HBM, %d rotating buffer sets" % r["rotate_sets"],
        "config": {"workload": w.name, "N": N, "B": B, "S": S, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "mode": w.mode, "parallelism": "%d virtual ranks on 1 GPU" % N,
                   "step": "fused QKV seq->head + O head->seq", "step_bytes": r["step_bytes"],
                   "launch_shape": r["tuning"]},
        "roofline": {"bound": "hbm", "kernel": "fused QKV seq->head (tile_kernel)",
                     "achieved": r["s2h_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": r["s2h_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": r["s2h_bytes"], "avg_launch_us": r["s2h_avg_us"],
                     "median_launch_us": r.get("s2h_median_us"), "min_launch_us": r.get("s2h_min_us"),
                     "max_launch_us": r.get("s2h_max_us"), "timed_launches": r["timed_launches_per_kernel"]},
        "copy_ceiling": {
            "kernel": "basp_stream_copy (16-byte loads/stores, same cache policy, read once, written once)",
            "s2h_bytes_gbs": r["copy_ceiling"][str(r["s2h_bytes"])]["gbs"],
            "h2s_bytes_gbs": r["copy_ceiling"][str(r["h2s_bytes"])]["gbs"],
            "s2h_frac_of_copy": r["s2h_gbs"] / r["copy_ceiling"][str(r["s2h_bytes"])]["gbs"],
            "h2s_frac_of_copy": r["h2s_gbs"] / r["copy_ceiling"][str(r["h2s_bytes"])]["gbs"],
            "in_timed_loop": dict(r["copy_loop"],
                                  step_frac_of_copy=r["value"] / r["copy_loop"]["step_gbs"],
                                  s2h_frac_of_copy=r["s2h_gbs"] / r["copy_loop"]["s2h_bytes_gbs"],
                                  h2s_frac_of_copy=r["h2s_gbs"] / r["copy_loop"]["h2s_bytes_gbs"])},
        "head_to_seq": {"achieved": r["h2s_gbs"], "frac": r["h2s_gbs"] / HBM_PEAK_GBS,
                        "avg_launch_us": r["h2s_avg_us"], "median_launch_us": r.get("h2s_median_us"),
                        "min_launch_us": r.get("h2s_min_us"), "max_launch_us": r.get("h2s_max_us"),
                        "bytes_per_launch": r["h2s_bytes"]},
        "round_trip_bit_exact": r["round_trip_bit_exact"],
    }
    if "device" in r:
        line["device"] = r["device"]
    return line


def main(argv=None):
    args = parse_args(argv)
    if args.pmc_summary:
        res = pmc_summary(*args.pmc_summary)
        defaults = parse_args([])   # the counter runs use the default workload and mode
        res["workload"], res["mode"] = defaults.workload, defaults.mode
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the N virtual ranks of the re-layout share one "
              "device allocation, and no multi-GPU path exists (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2

    r = run_gpu(args)
    w = r.pop("w")
    line = make_line(args, r, w, traffic_bytes(w.name, w.mode))
    if "detail" in r:
        line["detail"] = r["detail"]
    if "workloads" in r:
        line["workloads"] = r["workloads"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = optional_leg(lambda: cpu_baseline(args, w))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
