#!/usr/bin/env python3
"""Benchmark of the BASP attention-boundary re-layout on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workload: by default the largest named attention shape that fits one GPU,
Llama-3.2-3B-shaped at S = 32768 (N = 8 virtual ranks, B = 2, Hq = 24,
Hkv = 8, d = 128, bf16): 1.34 GB moved per fused seq->head call.

One step is one pass of the attention-boundary re-layout of a layer: the
fused Q/K/V seq->head exchange before attention and the O head->seq exchange
after it.  Inputs are one seeded global tensor per activation (Q, K, V, O:
N(0, 1) bf16 from seeds 0-3), scattered into each mode's own rank-sharded
buffers before timing, so BASP and Ulysses re-lay the same logical tensors.
R buffer sets rotate so that no step finds its bytes in the 256 MB Infinity
Cache.  Launch shapes come from the measured table
``sequence_re_layout_amd/launch_shapes.json`` (``--autotune`` measures them
anew with ``basp_plan_autotune``).

Timing.  K steps of the headline mode (BASP) are timed by wall clock between
device synchronisations (``ms_per_step``).  The kernels of every 10th step
carry start/stop events recorded by their own dispatches
(``basp_time_next_call``, hipExtLaunchKernel timestamps on the stream they
run on); the loop goes on past the K steps, the same way, until at least
--min-launches launches of each kernel are sampled.  ``value`` and
``roofline.achieved`` are the fused seq->head call's algorithmic bytes over
its average sampled duration.  Ulysses runs the same loop on its own
buffers; ``basp_vs_ulysses`` gives both modes and both directions.

Printed: one compact JSON line (last line of stdout).  Everything else --
the per-mode detail, the unfused three-pass baseline, the backward entries,
the token-major layout, the general-G plans, torch's device copy and the
table of every named workload -- goes to --detail-out.

Other modes:

    python bench.py --tune-shapes OUT.json
        measure the launch-shape table (every named workload, both modes)
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR
        HBM bytes per launch from two rocprofv3 counter runs of this script,
        scaled by the same counters on a plain copy of known size, into
        profiles/pmc_traffic.json
    python bench.py --trace-summary TRACE_DIR
        per-mode average kernel durations of a rocprofv3 kernel trace of
        this script (the sampled loops, found by their marker kernels)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import itertools
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
MARKER_CYCLES = 1000      # torch's spin kernel: brackets each mode's sampled loop
DEFAULT_WORKLOAD = "llama3.2-3b_s32k_b2"
MODES = ("basp", "ulysses")


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sample-every", type=int, default=10,
                    help="time the kernels of every n-th step with their own events")
    ap.add_argument("--min-launches", type=int, default=50,
                    help="least sampled launches per kernel and mode (the loop continues past --steps)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: enough for > 1 GiB reuse distance)")
    ap.add_argument("--autotune", action="store_true",
                    help="measure launch shapes per plan instead of reading the table")
    ap.add_argument("--builtin-shapes", action="store_true", help="the library's built-in launch shapes")
    ap.add_argument("--detail-out", default=os.path.join("bench_out", "bench_detail.json"))
    ap.add_argument("--detail-iters", type=int, default=60)
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the table of every named workload")
    ap.add_argument("--workload-rounds", type=int, default=5,
                    help="interleaved rounds of the workload table's graph replays (median over them)")
    ap.add_argument("--workload-steps", type=int, default=60,
                    help="least launches per HIP graph in the table of every workload")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune-shapes", metavar="OUT")
    ap.add_argument("--tune-autotunes", type=int, default=3, help="autotune runs per plan for --tune-shapes")
    ap.add_argument("--tune-sweep-mib", type=int, default=128,
                    help="--tune-shapes also sweeps each direction whose call moves at most this many MiB")
    ap.add_argument("--tune-workloads", default="",
                    help="comma-separated workloads for --tune-shapes (others keep the current table's entries)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--trace-summary", metavar="TRACE_DIR")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR")
    return ap.parse_args(argv)


def rate(nbytes, seconds):
    return nbytes / seconds / 1e9


# ------------------------------------------------------------- inputs ---

def scatter_seq(x, G, P, Bl, S, H, d):
    """Sequence-sharded buffer of a global [B][S][H][d] tensor: rank (g, j)
    holds sequences [g*Bl, (g+1)*Bl) and tokens [j*St, (j+1)*St), as
    [Bl][St][H][d], ranks in order.  (Input preparation: a reshape and a
    permute of the global tensor.)"""
    return x.view(G, Bl, P, S // P, H, d).permute(0, 2, 1, 3, 4, 5).contiguous().view(-1)


def scatter_head(x, G, P, Bl, S, H, d):
    """Head-sharded (head-major) buffer of a global [B][S][H][d] tensor: rank
    (g, j) holds sequences [g*Bl, (g+1)*Bl) and heads [j*Hl, (j+1)*Hl), as
    [Bl][Hl][S][d], ranks in order."""
    return x.view(G, Bl, S, P, H // P, d).permute(0, 3, 1, 4, 2, 5).contiguous().view(-1)


class Inputs:
    """The global Q, K, V, O tensors of a workload on the host: N(0, 1)
    bf16 from seeds 0, 1, 2, 3."""

    def __init__(self, shape):
        from sequence_re_layout_amd import inputs
        N, B, S, Hq, Hkv, d = shape
        self.x = {"q": inputs.normal_bf16(B * S * Hq * d, inputs.SEED_Q).view(B, S, Hq, d),
                  "k": inputs.normal_bf16(B * S * Hkv * d, inputs.SEED_K).view(B, S, Hkv, d),
                  "v": inputs.normal_bf16(B * S * Hkv * d, inputs.SEED_V).view(B, S, Hkv, d),
                  "o": inputs.normal_bf16(B * S * Hq * d, inputs.SEED_O).view(B, S, Hq, d)}


class ModeRun:
    """Plan and R rotating device buffer sets of one mode: q, k, v
    sequence-sharded and o head-sharded, scattered from the same global
    tensors, plus the two outputs."""

    def __init__(self, b, name, shape, mode, inp, rotate, shapes):
        import torch
        from sequence_re_layout_amd import launch_shapes
        N, B, S, Hq, Hkv, d = shape
        self.name, self.shape, self.mode = name, shape, mode
        code = b.BASP_MODE_BASP if mode == "basp" else b.BASP_MODE_ULYSSES
        self.plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
        i = self.plan.info
        G, P, Bl = i["G"], i["P"], i["Bl"]
        self.s2h_bytes, self.h2s_bytes = i["qkv_bytes_moved"], i["o_bytes_moved"]
        dev = {
            "q": scatter_seq(inp.x["q"].cuda(), G, P, Bl, S, Hq, d),
            "k": scatter_seq(inp.x["k"].cuda(), G, P, Bl, S, Hkv, d),
            "v": scatter_seq(inp.x["v"].cuda(), G, P, Bl, S, Hkv, d),
            "o": scatter_head(inp.x["o"].cuda(), G, P, Bl, S, Hq, d),
        }
        self.R = rotate or max(2, -(-(3 << 30) // (self.s2h_bytes + self.h2s_bytes)))
        self.sets = []
        for r in range(self.R):
            s = {n: (t if r == 0 else t.clone()) for n, t in dev.items()}
            s["qkv_out"] = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
            s["o_out"] = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
            self.sets.append(s)
        torch.cuda.synchronize()
        self.autotune_seconds = None
        self.shape_source = "built-in"
        if shapes == "table" and launch_shapes.apply(b, self.plan, name, mode):
            self.shape_source = "table"
        elif shapes in ("table", "autotune"):
            s = self.sets[0]
            t0 = time.perf_counter()
            b.basp_plan_autotune(self.plan, s["q"], s["k"], s["v"], s["qkv_out"], s["o"], s["o_out"])
            torch.cuda.synchronize()
            self.autotune_seconds = time.perf_counter() - t0
            self.shape_source = "autotuned"
        self.tuning = {"seq_to_head": b.basp_plan_get_tuning(self.plan, b.BASP_SEQ_TO_HEAD),
                       "head_to_seq": b.basp_plan_get_tuning(self.plan, b.BASP_HEAD_TO_SEQ)}

    def s2h(self, b, i):
        s = self.sets[i % self.R]
        b.basp_seq_to_head(self.plan, s["q"], s["k"], s["v"], s["qkv_out"])

    def h2s(self, b, i):
        s = self.sets[i % self.R]
        b.basp_head_to_seq(self.plan, s["o"], s["o_out"])


# ------------------------------------------------------------- timing ---

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence, through the
    HIP runtime torch has loaded: recording it performs no system-scope cache
    writeback, so a launch that records it runs like the untimed launches
    beside it.  The bench reads its events only after a device
    synchronisation, which the fence would otherwise provide."""

    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            import torch
            torch.cuda.init()
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            lib = ctypes.CDLL(path)   # the already loaded image: the same runtime as torch's
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        h = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(h), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value   # the attribute the binding passes on

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if getattr(self, "cuda_event", None) and self._hip is not None:
            self._hip.hipEventDestroy(self.cuda_event)


def make_events(n):
    """n timing events for basp_time_next_call (see TimingEvent)."""
    import torch
    torch.cuda.synchronize()
    return [TimingEvent() for _ in range(n)]


def stats_us(t):
    return {"avg_us": statistics.mean(t) * 1e6, "median_us": statistics.median(t) * 1e6,
            "min_us": min(t) * 1e6, "max_us": max(t) * 1e6, "launches": len(t)}


def step_loop(b, s_fn, h_fn, steps, warmup, every, min_launches, marker=True):
    """Steps of s_fn(i) then h_fn(i) back to back.  The first `steps` steps
    are timed by wall clock between device synchronisations; the launches of
    every `every`-th step carry their own start/stop events; the loop goes on
    the same way past `steps` until `min_launches` launches of each are
    sampled.  A marker kernel before and after the sampled loop lets a
    profiler trace find its launches.  Returns (wall seconds of the first
    `steps` steps, sampled s_fn durations, sampled h_fn durations)."""
    import torch
    for i in range(warmup):
        s_fn(i)
        h_fn(i)
    torch.cuda.synchronize()
    every = max(1, every)
    total = max(steps, every * max(1, min_launches))
    nsamp = total // every   # steps every-1, 2*every-1, ... (at least min_launches)
    ev = make_events(4 * nsamp)
    if marker:
        torch.cuda._sleep(MARKER_CYCLES)
    torch.cuda.synchronize()
    wall = None
    t0 = time.perf_counter()
    for i in range(total):
        if i == steps:
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        # the 10th, 20th, ... step (with every = 10): the first step after a
        # short warm-up still runs in the device's ramp-up
        j = i // every if (i + 1) % every == 0 else -1
        if j >= 0:
            b.basp_time_next_call(ev[4 * j], ev[4 * j + 1])
        s_fn(i)
        if j >= 0:
            b.basp_time_next_call(ev[4 * j + 2], ev[4 * j + 3])
        h_fn(i)
    torch.cuda.synchronize()
    if wall is None:
        wall = time.perf_counter() - t0
    if marker:
        torch.cuda._sleep(MARKER_CYCLES)
        torch.cuda.synchronize()
    s_t = [ev[4 * j].elapsed_time(ev[4 * j + 1]) * 1e-3 for j in range(nsamp)]
    h_t = [ev[4 * j + 2].elapsed_time(ev[4 * j + 3]) * 1e-3 for j in range(nsamp)]
    return wall, s_t, h_t


def time_launches(b, fn, n, rotate):
    """Durations (s) of n calls of fn(i), each timed alone from its kernels'
    own dispatch timestamps (basp_time_next_call)."""
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
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t = []
    for _ in range(reps):
        start.record()
        graph.replay()
        stop.record()
        torch.cuda.synchronize()
        t.append(start.elapsed_time(stop) * 1e-3 / calls)
    del graph
    return statistics.median(t)


def copy_buffers(nbytes, R):
    import torch
    return [(torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
             torch.empty(nbytes, dtype=torch.uint8, device="cuda")) for _ in range(R)]


def copy_ceiling(b, s_bytes, h_bytes, steps, warmup, every, min_launches):
    """basp_stream_copy (a plain read-once, write-once copy with the kernels'
    access rules) at the two kernels' byte counts: each launch timed alone,
    and run the way the step loop runs the kernels."""
    import torch
    R = max(2, -(-(3 << 30) // (s_bytes + h_bytes)))
    sb, hb = copy_buffers(s_bytes // 2, R), copy_buffers(h_bytes // 2, R)
    out = {}
    for key, bufs, m in (("s2h_bytes", sb, s_bytes), ("h2s_bytes", hb, h_bytes)):
        # each leg between two marker kernels, so that profiler summaries can
        # set the copy beside the kernels
        torch.cuda.synchronize()
        torch.cuda._sleep(MARKER_CYCLES)
        t = time_launches(b, lambda i: b.basp_stream_copy(bufs[i][1], bufs[i][0]), 60, R)
        torch.cuda._sleep(MARKER_CYCLES)
        torch.cuda.synchronize()
        out[key + "_alone_gbs"] = rate(m, statistics.mean(t))
    wall, s_t, h_t = step_loop(b, lambda i: b.basp_stream_copy(sb[i % R][1], sb[i % R][0]),
                               lambda i: b.basp_stream_copy(hb[i % R][1], hb[i % R][0]),
                               steps, warmup, every, min_launches, marker=False)
    out["s2h_bytes_gbs"] = rate(s_bytes, statistics.mean(s_t))
    out["h2s_bytes_gbs"] = rate(h_bytes, statistics.mean(h_t))
    out["step_gbs"] = rate(s_bytes + h_bytes, wall / steps)
    del sb, hb
    torch.cuda.empty_cache()
    return out


# -------------------------------------------------------------- GPU run ---

def shapes_mode(args):
    return "autotune" if args.autotune else ("builtin" if args.builtin_shapes else "table")


def run_gpu(args):
    import torch
    from sequence_re_layout_amd import binding as b
    from sequence_re_layout_amd import workloads

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count, "memory_bytes": props.total_memory}
    name, *shape = workloads.BY_NAME[args.workload]
    shape = tuple(shape)
    inp = Inputs(shape)
    res = {"device": device, "modes": {}}
    runs = {}
    for mode in MODES:   # BASP first: its first `steps` steps are the timed region
        w = ModeRun(b, name, shape, mode, inp, args.rotate, shapes_mode(args))
        runs[mode] = w
        if mode == "basp":
            # host bytes of the BASP buffers for the CPU baseline (the bytes
            # the GPU consumes), copied before any marked loop
            res["host"] = {n: w.sets[0][n].cpu() for n in ("q", "k", "v", "o")}
        wall, s_t, h_t = step_loop(b, lambda i: w.s2h(b, i), lambda i: w.h2s(b, i), args.steps,
                                   args.warmup, args.sample_every, args.min_launches)
        s, h = stats_us(s_t), stats_us(h_t)
        res["modes"][mode] = {
            "G": w.plan.info["G"], "P": w.plan.info["P"], "Bl": w.plan.info["Bl"],
            "peers_per_rank": w.plan.info["peers_per_rank"],
            "cross_rank_bytes_qkv": w.plan.info["cross_rank_bytes_q"] + 2 * w.plan.info["cross_rank_bytes_kv"],
            "ms_per_step": wall / args.steps * 1e3, "step_gbs": rate(w.s2h_bytes + w.h2s_bytes, wall / args.steps),
            "s2h": s, "h2s": h, "s2h_bytes": w.s2h_bytes, "h2s_bytes": w.h2s_bytes,
            "s2h_gbs": rate(w.s2h_bytes, s["avg_us"] * 1e-6), "h2s_gbs": rate(w.h2s_bytes, h["avg_us"] * 1e-6),
            "rotate_sets": w.R, "shape_source": w.shape_source, "tuning": w.tuning,
            "autotune_seconds": w.autotune_seconds}
    # device round trip of the timed buffers: head->seq of the Q part of the
    # fused output gives Q back bit for bit, in both modes
    ok = True
    for mode, w in runs.items():
        s = w.sets[0]
        back = torch.empty_like(s["q"])
        b.basp_seq_to_head(w.plan, s["q"], s["k"], s["v"], s["qkv_out"])
        b.basp_head_to_seq(w.plan, s["qkv_out"][: w.plan.info["q_elems"]], back)
        torch.cuda.synchronize()
        ok = ok and bool(torch.equal(back.view(torch.int16), s["q"].view(torch.int16)))
        del back
    res["round_trip_bit_exact"] = ok
    basp = runs["basp"]
    res["shape"], res["name"] = shape, name
    del runs, inp
    torch.cuda.empty_cache()
    res["copy"] = copy_ceiling(b, basp.s2h_bytes, basp.h2s_bytes, args.steps, args.warmup,
                               args.sample_every, args.min_launches)
    del basp
    torch.cuda.empty_cache()
    # a plain copy of known size, between two more marker kernels: the PMC
    # byte counters are scaled by it
    cal_src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    cal_dst = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    torch.cuda._sleep(MARKER_CYCLES)
    cal_dst.copy_(cal_src)
    torch.cuda._sleep(MARKER_CYCLES)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    return res


def optional_leg(fn):
    """fn(), or {"error": ...} when it raises (after reporting it on stderr)."""
    try:
        return fn()
    except Exception as e:   # noqa: BLE001 -- recorded in the output
        import traceback
        traceback.print_exc()
        return {"error": "%s: %s" % (type(e).__name__, e)}


def detail(args, shape, name):
    """Per-mode rates of the other entry points on the bench workload: the
    unfused baseline, the backward calls, the token-major layout, the step
    replayed from a HIP graph; the general-G plans at the batch-sweep shape;
    torch's device copy."""
    import torch
    from sequence_re_layout_amd import binding as b
    N, B, S, Hq, Hkv, d = shape
    inp = Inputs(shape)
    out = {}
    n = args.detail_iters
    med = statistics.median
    for mode in MODES:
        w = ModeRun(b, name, shape, mode, inp, 2, shapes_mode(args))
        p, sets = w.plan, w.sets
        o = {}
        ws = torch.empty(b.basp_unfused_workspace_bytes(p), dtype=torch.uint8, device="cuda")
        f = time_launches(b, lambda i: b.basp_seq_to_head_unfused(
            p, sets[i]["q"], sets[i]["k"], sets[i]["v"], sets[i]["qkv_out"], ws), max(10, n // 4), w.R)
        o["s2h_unfused_gbs"] = rate(w.s2h_bytes, med(f))
        del ws
        grads = [{"dq": torch.empty_like(s["q"]), "dk": torch.empty_like(s["k"]),
                  "dv": torch.empty_like(s["v"])} for s in sets]
        bo = time_launches(b, lambda i: b.basp_seq_to_head_o(p, sets[i]["o"], sets[i]["o_out"]), n, w.R)
        bq = time_launches(b, lambda i: b.basp_head_to_seq_qkv(
            p, sets[i]["qkv_out"], grads[i]["dq"], grads[i]["dk"], grads[i]["dv"]), n, w.R)
        o["backward"] = {"do_s2h_gbs": rate(w.h2s_bytes, med(bo)), "dqkv_h2s_gbs": rate(w.s2h_bytes, med(bq))}
        del grads
        pt = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_BF16,
                                   b.BASP_MODE_BASP if mode == "basp" else b.BASP_MODE_ULYSSES,
                                   b.BASP_LAYOUT_TOKEN_MAJOR)
        s0 = sets[0]
        if not args.builtin_shapes:
            b.basp_plan_autotune(pt, s0["q"], s0["k"], s0["v"], s0["qkv_out"], s0["o"], s0["o_out"])
        tt = time_launches(b, lambda i: b.basp_seq_to_head(pt, sets[i]["q"], sets[i]["k"], sets[i]["v"],
                                                           sets[i]["qkv_out"]), n, w.R)
        tu = time_launches(b, lambda i: b.basp_head_to_seq(pt, sets[i]["o"], sets[i]["o_out"]), n, w.R)
        o["token_major"] = {"s2h_gbs": rate(w.s2h_bytes, med(tt)), "h2s_gbs": rate(w.h2s_bytes, med(tu))}
        o["graph_step_gbs"] = rate(w.s2h_bytes + w.h2s_bytes,
                                   graph_seconds(lambda i: (w.s2h(b, i), w.h2s(b, i)), 20))
        out[mode] = o
        del w, sets, p
        torch.cuda.empty_cache()
    out["groups"] = groups_rates(args)
    nb = (2 * B * S * (Hq + 2 * Hkv) * d * 2) // 2
    src = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    dst = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    c = time_torch(lambda i: dst[i].copy_(src[i]), n, 2)
    out["torch_device_copy_gbs"] = rate(2 * nb, med(c))
    del src, dst
    torch.cuda.empty_cache()
    return out


def groups_rates(args):
    """The general G-group form at the batch-sweep shape with B = 8 (N = 8,
    S = 8192, Llama-3.2-1B heads): G groups of 8/G ranks, for G = 1, 2, 4,
    8, each plan autotuned (unless --builtin-shapes), timed like the table
    of every workload (HIP graphs of back-to-back launches)."""
    import torch
    from sequence_re_layout_amd import binding as b
    from sequence_re_layout_amd import workloads
    _, N, B, S, Hq, Hkv, d = workloads.BATCH_SWEEP[-1]
    out = {}
    for G in (1, 2, 4, 8):
        p = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G)
        i = p.info
        R = max(2, -(-(3 << 30) // (i["qkv_bytes_moved"] + i["o_bytes_moved"])))
        sets = table_sets(i, R)
        if not args.builtin_shapes:
            s0 = sets[0]
            b.basp_plan_autotune(p, s0["q"], s0["k"], s0["v"], s0["out"], s0["o"], s0["o_out"])
        t = measure_pair(b, p, sets, R, args.workload_steps)
        out["G%d" % G] = dict(t, G=i["G"], P=i["P"], Bl=i["Bl"], peers_per_rank=i["peers_per_rank"],
                              cross_rank_bytes_qkv=i["cross_rank_bytes_q"] + 2 * i["cross_rank_bytes_kv"])
        del sets
        torch.cuda.empty_cache()
    return out


class GraphTimer:
    """`calls` back-to-back calls fn(i), captured once in a HIP graph (so that
    no host gap falls between the kernels) and replayed once untimed;
    seconds() replays it once more and returns the seconds per call."""

    def __init__(self, fn, calls):
        import torch
        torch.cuda.synchronize()
        self.calls = calls
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(calls):
                fn(i)
        self.graph.replay()
        torch.cuda.synchronize()
        self.start = torch.cuda.Event(enable_timing=True)
        self.stop = torch.cuda.Event(enable_timing=True)

    def seconds(self):
        import torch
        self.start.record()
        self.graph.replay()
        self.stop.record()
        torch.cuda.synchronize()
        return self.start.elapsed_time(self.stop) * 1e-3 / self.calls


def workload_table(args):
    """Fused seq->head and head->seq rates of every named workload in both
    modes (device-filled random bf16: the rate does not depend on values),
    with the launch shapes of the table, beside the plain copy at the same
    byte counts.  Per workload, each of nine items -- the copy at each
    direction's byte count and as a pair, and each mode's whole step,
    seq->head alone and head->seq alone -- is a HIP graph of back-to-back
    launches on rotating buffer sets (at least --workload-steps launches,
    more for small calls).  The nine graphs are replayed in
    --workload-rounds interleaved rounds, so that slow drift of the device
    falls on the kernels and the copy alike, and each figure is the median
    over the rounds.  Both modes' buffers have the same sizes, so they share
    one buffer set."""
    import torch
    from sequence_re_layout_amd import binding as b
    from sequence_re_layout_amd import launch_shapes, workloads
    steps = args.workload_steps
    out = {}
    for (name, N, B, S, Hq, Hkv, d) in workloads.ALL + workloads.EXTRA:
        plans, sources = {}, {}
        for mode, code in (("basp", b.BASP_MODE_BASP), ("ulysses", b.BASP_MODE_ULYSSES)):
            plans[mode] = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
        i = plans["basp"].info
        sb, hb = i["qkv_bytes_moved"], i["o_bytes_moved"]
        R = max(2, -(-(3 << 30) // (sb + hb)))
        n = max(steps, min(10 * steps, steps * (400 << 20) // sb))
        sets = table_sets(i, R)
        for mode, p in plans.items():
            sources[mode] = "built-in"
            if not args.builtin_shapes:
                if not args.autotune and launch_shapes.apply(b, p, name, mode):
                    sources[mode] = "table"
                else:
                    s0 = sets[0]
                    b.basp_plan_autotune(p, s0["q"], s0["k"], s0["v"], s0["out"], s0["o"], s0["o_out"])
                    sources[mode] = "autotuned"
        qkv_b, o_b = sb // 2, hb // 2   # bytes each copy reads (and writes)

        def cs(j):
            b.basp_stream_copy(sets[j % R]["out"], sets[j % R]["x"], qkv_b)

        def ch(j):
            b.basp_stream_copy(sets[j % R]["o_out"], sets[j % R]["x"], o_b)

        def s2h(p):
            return lambda j: b.basp_seq_to_head(p, sets[j % R]["q"], sets[j % R]["k"], sets[j % R]["v"],
                                                sets[j % R]["out"])

        def h2s(p):
            return lambda j: b.basp_head_to_seq(p, sets[j % R]["o"], sets[j % R]["o_out"])

        items = {("copy", "s2h"): cs, ("copy", "h2s"): ch, ("copy", "step"): lambda j: (cs(j), ch(j))}
        for mode, p in plans.items():
            fs, fh = s2h(p), h2s(p)
            items[(mode, "step")] = lambda j, fs=fs, fh=fh: (fs(j), fh(j))
            items[(mode, "s2h")] = fs
            items[(mode, "h2s")] = fh
        timers = {key: GraphTimer(fn, n) for key, fn in items.items()}
        times = {key: [] for key in items}
        for _ in range(args.workload_rounds):
            for key, t in timers.items():
                times[key].append(t.seconds())
        del timers
        med = {key: statistics.median(t) for key, t in times.items()}
        out[name] = {"copy": {"s2h_bytes_gbs": rate(sb, med[("copy", "s2h")]),
                              "h2s_bytes_gbs": rate(hb, med[("copy", "h2s")]),
                              "step_gbs": rate(sb + hb, med[("copy", "step")])}}
        for mode, p in plans.items():
            pi = p.info
            wall, t, u = med[(mode, "step")], med[(mode, "s2h")], med[(mode, "h2s")]
            out[name][mode] = {
                "step_us": wall * 1e6, "step_gbs": rate(sb + hb, wall), "s2h_us": t * 1e6, "s2h_gbs": rate(sb, t),
                "h2s_us": u * 1e6, "h2s_gbs": rate(hb, u), "G": pi["G"], "P": pi["P"], "Bl": pi["Bl"],
                "launches_per_graph": n, "rounds": args.workload_rounds, "shapes": sources[mode],
                "s2h_frac": rate(sb, t) / HBM_PEAK_GBS, "h2s_frac": rate(hb, u) / HBM_PEAK_GBS,
                "s2h_us_range": [min(times[(mode, "s2h")]) * 1e6, max(times[(mode, "s2h")]) * 1e6],
                "h2s_us_range": [min(times[(mode, "h2s")]) * 1e6, max(times[(mode, "h2s")]) * 1e6]}
        del sets, plans
        torch.cuda.empty_cache()
        print("workload table: %s done" % name, file=sys.stderr, flush=True)
    return out


def table_sets(i, R):
    """R rotating device sets for a plan with info i: one random buffer x
    holding q, k, v and o back to back, and the two outputs."""
    import torch
    sets = []
    for _ in range(R):
        x = torch.empty(2 * i["q_elems"] + 2 * i["kv_elems"], dtype=torch.bfloat16, device="cuda").normal_()
        nq, nkv = i["q_elems"], i["kv_elems"]
        sets.append({"x": x, "q": x[:nq], "k": x[nq:nq + nkv], "v": x[nq + nkv:nq + 2 * nkv],
                     "o": x[nq + 2 * nkv:],
                     "out": torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda"),
                     "o_out": torch.empty(nq, dtype=torch.bfloat16, device="cuda")})
    return sets


def measure_pair(b, p, sets, R, n):
    """Whole back-to-back steps, then each direction alone, from HIP graphs."""
    i = p.info
    sb, hb = i["qkv_bytes_moved"], i["o_bytes_moved"]

    def s2h(j):
        s = sets[j % R]
        b.basp_seq_to_head(p, s["q"], s["k"], s["v"], s["out"])

    def h2s(j):
        s = sets[j % R]
        b.basp_head_to_seq(p, s["o"], s["o_out"])

    wall = graph_seconds(lambda j: (s2h(j), h2s(j)), n)
    t, u = graph_seconds(s2h, n), graph_seconds(h2s, n)
    return {"step_us": wall * 1e6, "step_gbs": rate(sb + hb, wall), "s2h_us": t * 1e6, "s2h_gbs": rate(sb, t),
            "h2s_us": u * 1e6, "h2s_gbs": rate(hb, u)}


SWEEP_KEEP = 2   # shapes per swept direction that enter the pair comparison


def sweep_grid(B):
    """Launch shapes of the per-direction sweep: both kernels, every
    work-group size and tile order, 1, 2 or 4 vectors per lane, 1-8 heads per
    tile, direct tiles of one pass or of 8 or 16 tokens (several passes), both
    lane orders of the direct kernel, both XCD orders, and both batch orders
    when there is more than one sequence."""
    grid = []
    for bo, stage, block, vpt, th, tt, to, lo, xr in itertools.product(
            (1, 2) if B > 1 else (1,), (1, 2), (64, 128, 256), (1, 2, 4), (1, 2, 4, 8),
            (0, 8, 16), (1, 2, 3), (1, 2), (1, 2)):
        if stage == 2 and (tt or lo == 2):   # a staged tile is one pass; its lanes follow the layouts
            continue
        t = {"batch_order": bo, "stage": stage, "block_size": block, "vectors_per_thread": vpt,
             "tile_heads": th, "tile_order": to, "xcd_remap": xr, "cache_policy": 4}
        if tt:
            t["tile_tokens"] = tt
        if stage == 1:
            t["lane_order"] = lo
        grid.append(t)
    return grid


def sweep_direction(b, p, sets, R, direction, grid, keep=SWEEP_KEEP):
    """The best `keep` shapes of one direction, each direction timed alone
    with its launches back to back from HIP graphs on the rotating sets: every
    shape of `grid` from a short graph, then the best 16 in 3 interleaved
    rounds of longer graphs.  The plan's tuning of that direction is kept."""
    i = p.info
    if direction == b.BASP_SEQ_TO_HEAD:
        nbytes = i["qkv_bytes_moved"]

        def fn(j):
            s = sets[j % R]
            b.basp_seq_to_head(p, s["q"], s["k"], s["v"], s["out"])
    else:
        nbytes = i["o_bytes_moved"]

        def fn(j):
            s = sets[j % R]
            b.basp_head_to_seq(p, s["o"], s["o_out"])
    held = b.basp_plan_get_tuning(p, direction)
    est = 2e-6 + nbytes / 6e12                       # seconds per call, roughly
    short, long_ = max(20, min(200, int(3e-4 / est))), max(60, min(600, int(2e-3 / est)))
    coarse = []
    for t in grid:
        try:
            b.basp_plan_set_direction_tuning(p, direction, **t)
        except b.BaspError:                          # beyond the index limits
            continue
        coarse.append((graph_seconds(fn, short, reps=2), t))
    coarse.sort(key=lambda c: c[0])
    top = [t for _, t in coarse[:16]]
    times = [[] for _ in top]
    for _ in range(3):
        for c, t in enumerate(top):
            b.basp_plan_set_direction_tuning(p, direction, **t)
            times[c].append(graph_seconds(fn, long_, reps=3))
    b.basp_plan_set_direction_tuning(p, direction, **held)
    order = sorted(range(len(top)), key=lambda c: statistics.median(times[c]))
    return [top[c] for c in order[:keep]]


def tune_shapes(args):
    """The launch-shape table: for every named workload and mode,
    basp_plan_autotune runs --tune-autotunes times (each from the built-in
    shapes).  A direction whose call moves at most --tune-sweep-mib MiB is
    also swept over a wider grid (sweep_grid), timed alone from HIP graphs:
    short calls are where the autotuner's one-launch timings rank shapes
    least like back-to-back runs.  Then, per mode, the distinct pairs
    autotune kept in either mode (the two plans share their tensors' sizes;
    with B = 1 they are the same plan), the built-in pair, the pair the
    current table holds and the pairs of the swept shapes are timed as whole
    back-to-back steps from HIP graphs in 3 interleaved rounds; the pair with
    the lowest median step time is kept.  With --tune-workloads only the
    named workloads are measured; the others keep the current table's
    entries."""
    import torch
    from sequence_re_layout_amd import binding as b
    from sequence_re_layout_amd import launch_shapes, workloads
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    out = {"about": "launch shapes per named workload and mode, measured by bench.py --tune-shapes",
           "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None)},
           "kernel_sources_sha256": kernel_sources_sha256(), "shapes": {}}
    dirs = (("seq_to_head", b.BASP_SEQ_TO_HEAD), ("head_to_seq", b.BASP_HEAD_TO_SEQ))
    modes = (("basp", b.BASP_MODE_BASP), ("ulysses", b.BASP_MODE_ULYSSES))
    only = set(args.tune_workloads.split(",")) if args.tune_workloads else None
    current = launch_shapes.table().get("shapes", {})
    for (name, N, B, S, Hq, Hkv, d) in workloads.ALL + workloads.EXTRA:
        if only is not None and name not in only:
            if name in current:
                out["shapes"][name] = current[name]
            continue
        out["shapes"][name] = {}
        picks = {}
        for mode, code in modes:   # autotune's picks in each mode
            p = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
            sets = table_sets(p.info, 1)
            picks[mode] = []
            for _ in range(args.tune_autotunes):
                b.basp_plan_set_tuning(p)
                s = sets[0]
                b.basp_plan_autotune(p, s["q"], s["k"], s["v"], s["out"], s["o"], s["o_out"])
                pair = tuple({k: v for k, v in b.basp_plan_get_tuning(p, dcode).items() if v}
                             for _, dcode in dirs)
                if pair not in picks[mode]:
                    picks[mode].append(pair)
            del sets
            torch.cuda.empty_cache()
        for mode, code in modes:
            p = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, code)
            i = p.info
            R = max(2, -(-(3 << 30) // (i["qkv_bytes_moved"] + i["o_bytes_moved"])))
            n = max(args.workload_steps, min(10 * args.workload_steps,
                                             args.workload_steps * (400 << 20) // i["qkv_bytes_moved"]))
            sets = table_sets(i, R)
            cands = [({}, {})]
            held = launch_shapes.lookup(name, mode)
            other = [m for m, _ in modes if m != mode][0]
            base = ([tuple(held)] if held is not None else []) + picks[mode] + picks[other] + [({}, {})]
            for pair in base:
                if pair not in cands:
                    cands.append(pair)
            # the swept shapes of each direction, paired with each other and
            # with the first base pair's shape of the other direction
            swept = []
            for (_, dcode), nbytes in zip(dirs, (i["qkv_bytes_moved"], i["o_bytes_moved"])):
                top = []
                if nbytes <= args.tune_sweep_mib << 20:
                    b.basp_plan_set_direction_tuning(p, dcode, **base[0][dcode])
                    top = sweep_direction(b, p, sets, R, dcode, sweep_grid(B))
                swept.append(top)
            for ts in swept[0] + [base[0][0]]:
                for th in swept[1] + [base[0][1]]:
                    pair = ({k: v for k, v in ts.items() if v}, {k: v for k, v in th.items() if v})
                    if pair not in cands:
                        cands.append(pair)
            times = [[] for _ in cands]
            for _ in range(3):
                for c, (ts, th) in enumerate(cands):
                    b.basp_plan_set_direction_tuning(p, b.BASP_SEQ_TO_HEAD, **ts)
                    b.basp_plan_set_direction_tuning(p, b.BASP_HEAD_TO_SEQ, **th)
                    times[c].append(measure_pair(b, p, sets, R, n))
            med = [statistics.median(t["step_us"] for t in ts) for ts in times]
            best = min(range(len(cands)), key=lambda c: med[c])
            pick = times[best]
            out["shapes"][name][mode] = {
                "seq_to_head": cands[best][0], "head_to_seq": cands[best][1],
                "step_us": med[best], "s2h_us": statistics.median(t["s2h_us"] for t in pick),
                "h2s_us": statistics.median(t["h2s_us"] for t in pick),
                "candidates": len(cands), "candidate_step_us": med}
            print("tune-shapes: %s %s: %d candidates (%d from the sweep), step %.1f us (built-in %.1f us)"
                  % (name, mode, len(cands), sum(map(len, swept)), med[best], med[0]), file=sys.stderr,
                  flush=True)
            del sets
            torch.cuda.empty_cache()
    with open(args.tune_shapes, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    return 0


# ------------------------------------------------------------------ CPU ---

def cpu_baseline(args, shape, mode, host):
    """The oracle doing the bench step (fused Q/K/V seq->head, O head->seq) on
    the host bytes the GPU consumed, repeated for about --cpu-seconds on all
    cores OpenMP gives it, then for a quarter of that on one thread."""
    import oracle
    from sequence_re_layout_amd import inputs
    N, B, S, Hq, Hkv, d = shape
    m = oracle.BASP if mode == "basp" else oracle.ULYSSES
    q, k, v, o = (inputs.raw_bits(host[n]) for n in ("q", "k", "v", "o"))
    step_bytes = 2 * (q.nbytes + k.nbytes + v.nbytes) + 2 * o.nbytes

    def loop(threads, seconds):
        reps, spent = 0, 0.0
        while reps == 0 or spent < seconds:
            t0 = time.perf_counter_ns()
            oracle.seq_to_head_qkv(q, k, v, m, N, B, S, Hq, Hkv, d, threads=threads)
            oracle.head_to_seq(o, m, N, B, S, Hq, d, threads=threads)
            spent += (time.perf_counter_ns() - t0) * 1e-9
            reps += 1
        return reps, spent

    threads = oracle.max_threads()
    reps, spent = loop(threads, args.cpu_seconds)
    reps1, spent1 = loop(1, args.cpu_seconds / 4)
    return {"value": rate(step_bytes * reps, spent), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d full step(s) of the bench workload (fused QKV seq->head + O head->seq, %s mode), "
                      "%.1f s on the host, OpenMP over destination blocks" % (reps, mode, spent),
            "seconds_per_step": spent / reps, "cpu_model": cpu_model(),
            "one_thread_gbs": rate(step_bytes * reps1, spent1)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------- profiles ---

def _regions(rows, name_key):
    """Rows between consecutive pairs of marker kernels (torch's spin
    kernel): the sampled loop of each mode, in run order."""
    marks = [i for i, r in enumerate(rows) if "spin_kernel" in r[name_key]]
    return [rows[marks[i] + 1:marks[i + 1]] for i in range(0, len(marks) - 1, 2)]


def _is_tile(name, s2h):
    """Whether a kernel name is a tile kernel of the given direction: the
    direction is template argument 5 of tile_kernel<BS, VW, VPT, POL, S2H,
    ONE> and argument 4 of tile_kernel_staged<BS, VPT, POL, S2H, ONE>."""
    for kernel, pos in (("tile_kernel_staged<", 3), ("tile_kernel<", 4)):
        i = name.find(kernel)
        if i >= 0:
            args = [a.strip() for a in name[i + len(kernel):name.index(">", i)].split(",")]
            return len(args) > pos and args[pos] == ("true" if s2h else "false")
    return False


# marked regions of a default run, in order: the two modes' sampled loops,
# basp_stream_copy alone at seq->head's and at head->seq's byte count, the
# calibration copy
CAL_REGION = len(MODES) + 2


def _region_kernels(regions):
    """(label, rows) of the kernels each marked region of a run holds."""
    out = []
    for mode, region in zip(MODES, regions):
        out.append(("%s seq->head" % mode, [r for r in region if _is_tile(r["Kernel_Name"], True)]))
        out.append(("%s head->seq" % mode, [r for r in region if _is_tile(r["Kernel_Name"], False)]))
    for i, label in ((len(MODES), "copy at seq->head bytes"), (len(MODES) + 1, "copy at head->seq bytes")):
        if i < len(regions):
            out.append((label, [r for r in regions[i] if "stream_copy_kernel" in r["Kernel_Name"]]))
    return out


def counter_summary(dirs):
    """Median per dispatch of every counter in rocprofv3 --pmc runs of this
    script, for each kernel of the marked regions (both modes' kernels and
    the plain copy at their byte counts)."""
    out = {}
    for d in dirs:
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                rows += list(csv.DictReader(f))
        counters = sorted({r["Counter_Name"] for r in rows})
        for c in counters:
            cr = sorted((r for r in rows if r["Counter_Name"] == c), key=lambda r: int(r["Dispatch_Id"]))
            for label, k in _region_kernels(_regions(cr, "Kernel_Name")):
                if k:
                    out.setdefault(label, {"kernel": k[0]["Kernel_Name"]})[c] = statistics.median(
                        float(r["Counter_Value"]) for r in k)
    return out


def launch_shape_key(workload, mode):
    """The table's launch shapes of a workload and mode (what a default run
    times), as stored beside counters taken on them."""
    from sequence_re_layout_amd import launch_shapes
    found = launch_shapes.lookup(workload, mode)
    return None if found is None else {"seq_to_head": found[0], "head_to_seq": found[1]}


def traffic_bytes(workload, mode):
    """HBM bytes per fused seq->head launch from committed PMC counters, or
    None when there are none for this workload and mode, or they were taken
    on other kernel sources or other launch shapes."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    for e in t.get("entries", []):
        if (e.get("workload") == workload and e.get("mode") == mode
                and e.get("kernel_sources_sha256") == kernel_sources_sha256()
                and e.get("launch_shape") == launch_shape_key(workload, mode)):
            return e.get("traffic_bytes_per_launch")
    return None


def pmc_summary(fetch_dir, write_dir, workload=DEFAULT_WORKLOAD):
    """Per-launch FETCH_SIZE/WRITE_SIZE of both kernels in each mode's sampled
    loop, scaled by the same counter on the known-size copy after them."""

    def load(d, counter):
        rows = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                rows += [r for r in csv.DictReader(f) if r.get("Counter_Name") == counter]
        if not rows:
            raise SystemExit("no %s rows under %s" % (counter, d))
        return sorted(rows, key=lambda r: int(r["Dispatch_Id"]))

    entries = {m: {"workload": workload, "mode": m, "kernel_sources_sha256": kernel_sources_sha256(),
                   "launch_shape": launch_shape_key(workload, m)} for m in MODES}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = load(d, counter)
        regions = _regions(rows, "Kernel_Name")
        if len(regions) <= CAL_REGION:
            raise SystemExit("expected %d marked regions for %s, found %d"
                             % (CAL_REGION + 1, counter, len(regions)))
        # the calibration copy: the one copy between the fifth pair of markers
        # (after the two modes' loops and the two copy-ceiling legs)
        copies = [r for r in regions[CAL_REGION] if "copy" in r["Kernel_Name"].lower()]
        if len(copies) != 1:
            raise SystemExit("expected one calibration copy for %s, found %d" % (counter, len(copies)))
        cal_row = copies[0]
        cal = float(cal_row["Counter_Value"])
        factor = (CALIB_BYTES / 1024.0) / cal
        for mode, region in zip(MODES, regions):
            e = entries[mode]
            for key, s2h in (("seq_to_head", True), ("head_to_seq", False)):
                k = [r for r in region if _is_tile(r["Kernel_Name"], s2h)]
                if not k:
                    raise SystemExit("no %s launches in the %s loop" % (key, mode))
                kib = statistics.median(float(r["Counter_Value"]) for r in k)
                e.setdefault(key, {"kernel": k[0]["Kernel_Name"]})[counter] = {
                    "kib_per_launch_raw": kib, "launches": len(k), "copy_kib_raw": cal,
                    "copy_kernel": cal_row["Kernel_Name"], "scale": factor,
                    "bytes_per_launch": kib * factor * 1024.0}
    for e in entries.values():
        for key in ("seq_to_head", "head_to_seq"):
            e[key]["traffic_bytes_per_launch"] = (e[key]["FETCH_SIZE"]["bytes_per_launch"]
                                                  + e[key]["WRITE_SIZE"]["bytes_per_launch"])
        e["traffic_bytes_per_launch"] = e["seq_to_head"]["traffic_bytes_per_launch"]
    return {"entries": [entries[m] for m in MODES]}


def trace_summary(trace_dir):
    """Average durations of both kernels in each mode's sampled loop of a
    rocprofv3 --kernel-trace run of this script, and the gaps between
    back-to-back dispatches there."""
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit("no kernel trace under %s" % trace_dir)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    regions = _regions(rows, "Kernel_Name")
    for mode, region in zip(MODES, regions):
        o = {}
        for key, s2h in (("seq_to_head", True), ("head_to_seq", False)):
            k = [r for r in region if _is_tile(r["Kernel_Name"], s2h)]
            dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in k]
            o[key] = {"kernel": k[0]["Kernel_Name"] if k else None, "launches": len(k),
                      "avg_us": statistics.mean(dur) if dur else None,
                      "median_us": statistics.median(dur) if dur else None}
        gaps = [(int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) * 1e-3 for a, b in zip(region, region[1:])]
        o["avg_gap_us"] = statistics.mean(gaps) if gaps else None
        out[mode] = o
    for label, k in _region_kernels(regions)[2 * len(MODES):]:
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in k]
        out[label] = {"launches": len(k), "avg_us": statistics.mean(dur) if dur else None}
    return out


# ---------------------------------------------------------------- main ---

def make_line(args, r, traffic, cpu):
    """The compact JSON line from the measurements r of run_gpu; traffic is
    the HBM bytes per fused launch from the committed counters, or None."""
    N, B, S, Hq, Hkv, d = r["shape"]
    m = r["modes"]
    head = m["basp"]
    cp = r["copy"]

    def brief(x):
        return {"G": x["G"], "P": x["P"], "Bl": x["Bl"], "peers_per_rank": x["peers_per_rank"],
                "cross_rank_bytes_qkv": x["cross_rank_bytes_qkv"],
                "s2h_gbs": round(x["s2h_gbs"], 1), "s2h_frac": round(x["s2h_gbs"] / HBM_PEAK_GBS, 4),
                "s2h_avg_us": round(x["s2h"]["avg_us"], 2),
                "h2s_gbs": round(x["h2s_gbs"], 1), "h2s_frac": round(x["h2s_gbs"] / HBM_PEAK_GBS, 4),
                "h2s_avg_us": round(x["h2s"]["avg_us"], 2),
                "step_gbs": round(x["step_gbs"], 1), "launches": x["s2h"]["launches"]}

    line = {
        "metric": METRIC,
        "value": head["s2h_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic: one seeded N(0,1) bf16 global tensor each for Q/K/V/O, scattered into each "
                 "mode's rank-sharded buffers; resident in HBM; %d rotating sets" % head["rotate_sets"]),
        "config": {"workload": r["name"], "N": N, "B": B, "S": S, "Hq": Hq, "Hkv": Hkv, "d": d,
                   "mode": "basp", "parallelism": "%d virtual ranks on 1 GPU" % N,
                   "step": "fused QKV seq->head + O head->seq", "launch_shapes": head["shape_source"],
                   "tuning_s2h": {k: v for k, v in head["tuning"]["seq_to_head"].items() if v}},
        "roofline": {"bound": "hbm", "kernel": "tile_kernel seq->head (fused Q/K/V)",
                     "achieved": head["s2h_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["s2h_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": head["s2h_bytes"],
                     "avg_launch_us": head["s2h"]["avg_us"], "median_launch_us": head["s2h"]["median_us"],
                     "timed_launches": head["s2h"]["launches"]},
        "basp_vs_ulysses": {mode: brief(m[mode]) for mode in MODES},
        "copy_ceiling": {"s2h_bytes_gbs": round(cp["s2h_bytes_gbs"], 1), "h2s_bytes_gbs": round(cp["h2s_bytes_gbs"], 1),
                         "s2h_frac_of_copy": round(head["s2h_gbs"] / cp["s2h_bytes_gbs"], 4),
                         "h2s_frac_of_copy": round(head["h2s_gbs"] / cp["h2s_bytes_gbs"], 4)},
        "round_trip_bit_exact": r["round_trip_bit_exact"],
        "detail_file": args.detail_out,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def main(argv=None):
    args = parse_args(argv)
    if args.pmc_summary:
        res = pmc_summary(*args.pmc_summary, workload=args.workload)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res))
        return 0
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary), indent=1))
        return 0
    if args.counter_summary:
        print(json.dumps(counter_summary(args.counter_summary), indent=1))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the N virtual ranks of the re-layout share one "
              "device allocation, and no multi-GPU path exists (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.tune_shapes:
        return tune_shapes(args)

    r = run_gpu(args)
    host = r.pop("host")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = optional_leg(lambda: cpu_baseline(args, r["shape"], "basp", host))
    del host
    line = make_line(args, r, traffic_bytes(r["name"], "basp"), cpu)
    full = {"line": line, "modes": r["modes"], "copy": r["copy"], "device": r["device"]}
    if not args.no_detail:
        full["detail"] = optional_leg(lambda: detail(args, r["shape"], r["name"]))
    if not args.no_workloads:
        full["workloads"] = optional_leg(lambda: workload_table(args))
    if args.detail_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail_out)), exist_ok=True)
        with open(args.detail_out, "w") as f:
            json.dump(full, f, indent=1, default=str)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
