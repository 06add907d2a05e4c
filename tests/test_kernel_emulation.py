"""The kernels' index arithmetic and the library's launch planning, run on the
CPU and compared with the oracle (no GPU).

``tests/emu/kernel_emu.cpp`` compiles the library's own plan.cpp, launch.cpp
and launch.hpp with g++ and executes every launch on the host (see its
header).  These tests drive it over ragged shapes, all launch shapes, both
layouts, both element sizes, narrow vector widths (short rows), misaligned
views and the degenerate cases, and require (a) the oracle's result bit for
bit, with every destination written, and (b) no in-tile access outside the
kernels' buffer descriptors.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import random_cases
from sequence_re_layout_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sequence_re_layout_amd", "csrc")


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("emu") / "libbasp_emu.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-DBASP_HD=",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "launch.cpp"),
                    os.path.join(ROOT, "tests", "emu", "kernel_emu.cpp"), "-o", out], check=True)
    lib = ctypes.CDLL(out)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.basp_plan_create_ex.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32]
    lib.basp_plan_create_ex.restype = vp
    lib.basp_plan_create_groups.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32]
    lib.basp_plan_create_groups.restype = vp
    lib.basp_plan_destroy.argtypes = [vp]
    lib.basp_plan_set_tuning.argtypes = [vp, ctypes.POINTER(ctypes.c_int32 * 11)]
    lib.basp_plan_set_tuning.restype = i32
    tail = [ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_int)]
    lib.emu_seq_to_head.argtypes = [vp, vp, vp, vp, vp] + tail
    lib.emu_head_to_seq.argtypes = [vp, vp, vp] + tail
    lib.emu_seq_to_head_o.argtypes = [vp, vp, vp] + tail
    lib.emu_head_to_seq_qkv.argtypes = [vp, vp, vp, vp, vp] + tail
    lib.emu_seq_to_head_unfused.argtypes = [vp, vp, vp, vp, vp, vp] + tail
    lib.emu_last_staged.restype = ctypes.c_int
    return lib


class Run:
    """One emulated call: checks status, the descriptor bound count and
    records the vector width used."""

    def __init__(self, lib, shape, mode, layout, es, tuning=None, G=0):
        N, B, S, Hq, Hkv, d = shape
        self.lib = lib
        dtype = {2: 0, 4: 3}[es]
        if mode == oracle.GROUPS:
            self.plan = lib.basp_plan_create_groups(N, B, S, Hq, Hkv, d, dtype, G, layout)
        else:
            self.plan = lib.basp_plan_create_ex(N, B, S, Hq, Hkv, d, dtype, mode, layout)
        assert self.plan, "plan rejected"
        if tuning:
            t = (ctypes.c_int32 * 11)(*[tuning.get(k, 0) for k in (
                "vectors_per_thread", "tile_tokens", "tile_heads", "cache_policy", "max_grid",
                "lane_order", "xcd_remap", "tile_order", "stage", "block_size", "batch_order")])
            assert lib.basp_plan_set_tuning(self.plan, ctypes.byref(t)) == 0

    def __call__(self, fn, *arrays):
        bad, vw = ctypes.c_uint64(0), ctypes.c_int(0)
        ptrs = [a.ctypes.data if a is not None else None for a in arrays]
        st = getattr(self.lib, fn)(self.plan, *ptrs, ctypes.byref(bad), ctypes.byref(vw))
        assert st == 0, "%s returned status %d" % (fn, st)
        assert bad.value == 0, "%d accesses outside a descriptor" % bad.value
        return vw.value

    def __del__(self):
        self.lib.basp_plan_destroy(self.plan)


def _rand(n, es, rng):
    dt = np.uint16 if es == 2 else np.uint32
    # values below the all-ones sentinel, so an unwritten destination shows
    return rng.integers(0, np.iinfo(dt).max, size=n, dtype=dt)


def _empty(n, es, offset=0):
    """Sentinel-filled array whose data pointer sits `offset` elements past an
    allocation start (a misaligned view when offset > 0)."""
    dt = np.uint16 if es == 2 else np.uint32
    buf = np.full(n + offset + 8, np.iinfo(dt).max, dtype=dt)
    return buf[offset:offset + n]


def _shifted(a, offset):
    b = _empty(a.size, a.itemsize, offset)
    b[:] = a
    return b


def check_s2h(emu, shape, mode, layout, es, tuning=None, offset=0, seed=0, G=0):
    N, B, S, Hq, Hkv, d = shape
    rng = np.random.default_rng(seed)
    q, k, v = (_rand(B * S * H * d, es, rng) for H in (Hq, Hkv, Hkv))
    run = Run(emu, shape, mode, layout, es, tuning, G)
    out = _empty(q.size + 2 * k.size, es, offset)
    vw = run("emu_seq_to_head", _shifted(q, offset), _shifted(k, offset), _shifted(v, offset), out)
    want = oracle.seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, layout, G=G)
    assert np.array_equal(out, want)
    return vw


def check_h2s(emu, shape, mode, layout, es, tuning=None, offset=0, seed=1, G=0):
    N, B, S, Hq, Hkv, d = shape
    rng = np.random.default_rng(seed)
    o = _rand(B * S * Hq * d, es, rng)
    run = Run(emu, shape, mode, layout, es, tuning, G)
    out = _empty(o.size, es, offset)
    vw = run("emu_head_to_seq", _shifted(o, offset), out)
    assert np.array_equal(out, oracle.head_to_seq(o, mode, N, B, S, Hq, d, layout, G=G))
    return vw


RAGGED = [  # N, B, S, Hq, Hkv, d
    (6, 3, 6 * 37, 12, 6, 40),
    (4, 2, 4 * 203, 8, 4, 64),
    (8, 2, 8 * 129, 24, 8, 128),
    (3, 3, 3 * 11, 6, 3, 3),
    (2, 4, 2 * 50, 4, 2, 12),
    (8, 4, 8 * 3, 16, 8, 8),
]


@pytest.mark.parametrize("mode", [1, 0], ids=["basp", "ulysses"])
@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("es", [2, 4])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged(emu, shape, es, layout, mode):
    check_s2h(emu, shape, mode, layout, es)
    check_h2s(emu, shape, mode, layout, es)


TUNINGS = [dict(vectors_per_thread=1), dict(vectors_per_thread=2), dict(vectors_per_thread=8),
           dict(tile_tokens=1), dict(tile_tokens=3, tile_heads=2), dict(tile_tokens=100, tile_heads=3),
           dict(tile_heads=4), dict(max_grid=7), dict(max_grid=1),
           dict(vectors_per_thread=8, tile_tokens=5, tile_heads=1, cache_policy=3, max_grid=3),
           dict(lane_order=1), dict(lane_order=2), dict(lane_order=2, tile_heads=3, tile_tokens=7),
           dict(xcd_remap=2), dict(xcd_remap=2, max_grid=24), dict(xcd_remap=2, max_grid=13, lane_order=2),
           dict(xcd_remap=1, lane_order=1, vectors_per_thread=1),
           dict(tile_order=1), dict(tile_order=2), dict(tile_order=2, tile_heads=3, tile_tokens=5, max_grid=11),
           dict(tile_order=1, xcd_remap=2, lane_order=2, tile_heads=2),
           dict(stage=2), dict(stage=2, vectors_per_thread=1, tile_heads=8), dict(stage=2, vectors_per_thread=8, tile_tokens=500),
           dict(stage=2, tile_order=2, xcd_remap=2, tile_heads=3, max_grid=5),
           dict(block_size=64), dict(block_size=128, vectors_per_thread=1, stage=1),
           dict(block_size=64, stage=2, vectors_per_thread=8, tile_heads=8), dict(block_size=64, stage=1, tile_tokens=9),
           dict(cache_policy=4), dict(cache_policy=5, block_size=128, stage=2),
           dict(batch_order=2), dict(batch_order=2, tile_order=1, max_grid=5),
           dict(batch_order=2, stage=2, xcd_remap=2, block_size=64, tile_heads=2),
           dict(batch_order=1, tile_order=1, xcd_remap=2),
           dict(tile_order=3), dict(tile_order=3, tile_heads=3, tile_tokens=5, max_grid=11),
           dict(tile_order=3, stage=2, xcd_remap=2, batch_order=2, tile_heads=2),
           dict(tile_order=3, lane_order=1, vectors_per_thread=2, block_size=64, max_grid=7)]


@pytest.mark.parametrize("tuning", TUNINGS, ids=lambda t: ",".join("%s=%s" % kv for kv in t.items()))
def test_tunings(emu, tuning):
    for shape, mode in (((8, 2, 8 * 129, 24, 8, 128), 1), ((6, 3, 6 * 37, 12, 6, 40), 0)):
        for layout in (0, 1):
            check_s2h(emu, shape, mode, layout, 2, tuning)
            check_h2s(emu, shape, mode, layout, 4, tuning)


def test_staging_used_where_it_applies(emu):
    """The staged kernel runs for 16-byte vectors (and is emulated as such),
    also on views that start 2 bytes past a 16-byte boundary; rows that
    need narrower vectors fall back to the direct kernel with the same
    result."""
    shape = (8, 2, 8 * 129, 24, 8, 128)
    check_s2h(emu, shape, 1, 0, 2, dict(stage=2))
    assert emu.emu_last_staged() == 1
    check_h2s(emu, shape, 0, 1, 2, dict(stage=2, vectors_per_thread=1))
    assert emu.emu_last_staged() == 1
    check_s2h(emu, shape, 1, 0, 2, dict(stage=2), offset=1)
    assert emu.emu_last_staged() == 1
    assert check_s2h(emu, (8, 2, 8 * 33, 24, 8, 4), 1, 0, 2, dict(stage=2)) == 8
    assert emu.emu_last_staged() == 0


@pytest.mark.parametrize("d,es,offset,expect_vw", [
    (64, 2, 0, 16), (64, 2, 1, 16), (64, 2, 2, 16), (64, 2, 4, 16), (64, 4, 1, 16), (64, 4, 2, 16),
    (4, 2, 0, 8), (4, 2, 1, 8), (2, 2, 3, 4), (1, 2, 1, 2), (3, 4, 1, 4), (2, 4, 0, 8), (5, 4, 2, 4)])
def test_vector_width_follows_row_size(emu, d, es, offset, expect_vw):
    """The widest vector that divides the row, whatever the pointers'
    alignment beyond the element size (views `offset` elements past an
    allocation start)."""
    shape = (4, 2, 4 * 21, 8, 4, d)
    assert check_s2h(emu, shape, 1, 0, es, offset=offset) == expect_vw
    assert check_h2s(emu, shape, 0, 1, es, offset=offset) == expect_vw
    # the same vector width with batch indices interleaved and a capped grid
    tuning = dict(batch_order=2, max_grid=5, tile_order=1)
    assert check_s2h(emu, shape, 0, 1, es, tuning, offset=offset) == expect_vw
    assert check_h2s(emu, shape, 1, 0, es, tuning, offset=offset) == expect_vw


@pytest.mark.parametrize("shape,mode", [
    ((8, 1, 8 * 16, 8, 8, 64), 1), ((8, 8, 8 * 16, 8, 8, 64), 1), ((4, 16, 32, 8, 4, 64), 1),
    ((1, 3, 40, 4, 2, 64), 0), ((1, 3, 40, 4, 2, 64), 1), ((8, 3, 8 * 5, 8, 8, 64), 0),
    ((2, 2, 2, 2, 2, 1), 1), ((8, 2, 8, 8, 8, 2), 0),
])
def test_degenerate(emu, shape, mode):
    for layout in (0, 1):
        for es in (2, 4):
            check_s2h(emu, shape, mode, layout, es)
            check_h2s(emu, shape, mode, layout, es)
    # batch indices interleaved with the tiles
    check_s2h(emu, shape, mode, 0, 2, dict(batch_order=2))
    check_h2s(emu, shape, mode, 1, 4, dict(batch_order=2, tile_order=1))


SCALED = [(w[0], w[1], w[2], max(w[3] // 16, w[1]), w[4], w[5], w[6]) for w in workloads.ALL + workloads.EXTRA]


@pytest.mark.parametrize("mode", [1, 0], ids=["basp", "ulysses"])
@pytest.mark.parametrize("w", SCALED, ids=[w[0] + "_S/16" for w in SCALED])
def test_workloads_scaled(emu, w, mode):
    check_s2h(emu, w[1:], mode, 0, 2)
    check_h2s(emu, w[1:], mode, 0, 2)


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", SCALED, ids=[w[0] + "_S/16" for w in SCALED])
def test_workloads_scaled_table_shapes(emu, w, mode):
    """Each workload's launch shapes from the measured table (the ones the
    benchmark times), each direction with its own, at a sixteenth of S."""
    from sequence_re_layout_amd import launch_shapes
    shapes = launch_shapes.lookup(w[0], mode)
    if shapes is None:
        pytest.skip("no table entry")
    m = {"basp": 1, "ulysses": 0}[mode]
    check_s2h(emu, w[1:], m, 0, 2, shapes[0])
    check_h2s(emu, w[1:], m, 0, 2, shapes[1])


@pytest.mark.parametrize("mode", [1, 0], ids=["basp", "ulysses"])
def test_llama1b_full_size(emu, mode):
    check_s2h(emu, workloads.LLAMA_1B[1:], mode, 0, 2)
    check_h2s(emu, workloads.LLAMA_1B[1:], mode, 0, 2, dict(batch_order=2))


@pytest.mark.parametrize("mode", [1, 0], ids=["basp", "ulysses"])
@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("shape", [(8, 2, 8 * 16, 32, 8, 64), (6, 3, 6 * 37, 12, 6, 40), (3, 3, 33, 6, 3, 3)],
                         ids=["llama1b_small", "ragged", "narrow"])
def test_backward_and_unfused(emu, shape, layout, mode):
    N, B, S, Hq, Hkv, d = shape
    rng = np.random.default_rng(9)
    run = Run(emu, shape, mode, layout, 2)
    nq, nkv = B * S * Hq * d, B * S * Hkv * d
    do = _rand(nq, 2, rng)
    out = _empty(nq, 2)
    run("emu_seq_to_head_o", do, out)
    assert np.array_equal(out, oracle.seq_to_head(do, mode, N, B, S, Hq, d, layout))
    g = _rand(nq + 2 * nkv, 2, rng)
    dq, dk, dv = _empty(nq, 2), _empty(nkv, 2), _empty(nkv, 2)
    run("emu_head_to_seq_qkv", g, dq, dk, dv)
    wq, wk, wv = oracle.head_to_seq_qkv(g, mode, N, B, S, Hq, Hkv, d, layout)
    assert np.array_equal(dq, wq) and np.array_equal(dk, wk) and np.array_equal(dv, wv)
    q, k, v = (_rand(n, 2, rng) for n in (nq, nkv, nkv))
    out = _empty(nq + 2 * nkv, 2)
    ws = _empty(2 * (nq + 2 * nkv), 2)
    run("emu_seq_to_head_unfused", q, k, v, out, ws)
    assert np.array_equal(out, oracle.seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, layout))


@pytest.mark.parametrize("seed", range(random_cases.COUNT))
def test_random_shapes_and_tunings(emu, seed):
    """The GPU tests' seeded random cases: every access inside its
    descriptor and the oracle's result, both element sizes."""
    shape, mode, layout, tuning = random_cases.case(seed)
    m = 1 if mode == "basp" else 0
    for es in (2, 4):
        check_s2h(emu, shape, m, layout, es, tuning)
        check_h2s(emu, shape, m, layout, es, tuning)


GRID_LIMITS = [  # (N, B, S, Hq, Hkv, d), mode
    ((1, 65535, 3, 2, 1, 8), 1),            # data-parallel fallback: 65535 batch indices along z
    ((5, 65535, 5, 5, 5, 8), 0),            # Ulysses: z = 65535, y = 5 members
    ((4096, 1, 4096, 4096, 4096, 1), 0),    # Ulysses: 4096 members along y, 2-byte rows
]


@pytest.mark.parametrize("shape,mode", GRID_LIMITS, ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else str(x))
def test_grid_limits(emu, shape, mode):
    """The launch grid at its extents: the largest batch count the grid's z
    coordinate takes, and thousands of group members along y, with the batch
    index along z or folded into x."""
    for tuning in (None, {"batch_order": 2}):
        check_s2h(emu, shape, mode, 0, 2, tuning)
        check_h2s(emu, shape, mode, 0, 2, tuning)


# ------------------------------------------------------- general G groups --

GROUP_CASES = [  # (N, B, S, Hq, Hkv, d), G
    ((8, 8, 8 * 16, 8, 8, 64), 1), ((8, 8, 8 * 16, 8, 8, 64), 2), ((8, 8, 8 * 16, 8, 8, 64), 4),
    ((8, 8, 8 * 16, 8, 8, 64), 8),
    ((6, 4, 6 * 5, 6, 3, 40), 2),        # 3 members, 2 sequences per group, 80-byte rows
    ((12, 6, 12 * 3, 12, 4, 24), 3),     # 4 members, 2 sequences per group, 48-byte rows
    ((8, 16, 8 * 4, 8, 4, 8), 4),        # 2 members, 4 sequences per group
    ((4, 6, 4 * 7, 4, 2, 3), 2),         # 6-byte rows: 2-byte vectors
]
GROUP_TUNINGS = [None, dict(batch_order=2), dict(stage=2, tile_heads=2),
                 dict(tile_order=1, xcd_remap=2, max_grid=5), dict(batch_order=2, tile_order=1, lane_order=2)]


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: "x".join(map(str, c[0])) + "_G%d" % c[1])
def test_general_groups(emu, case, layout):
    """G groups of N/G ranks owning B/G sequences each: the oracle's result
    and every access inside its descriptor, for launch shapes that put the
    batch index along z and along x."""
    shape, G = case
    for tuning in GROUP_TUNINGS:
        for es in (2, 4):
            check_s2h(emu, shape, oracle.GROUPS, layout, es, tuning, G=G)
            check_h2s(emu, shape, oracle.GROUPS, layout, es, tuning, G=G)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_general_groups_batch_sweep_scaled(emu, G):
    """The batch-sweep shape at B = 8 (N = 8, S = 8192 / 16) for every G."""
    shape = (8, 8, 512, 32, 8, 64)
    check_s2h(emu, shape, oracle.GROUPS, 0, 2, G=G)
    check_h2s(emu, shape, oracle.GROUPS, 0, 2, G=G)


def test_general_groups_backward_and_unfused(emu):
    shape, G = (6, 4, 6 * 5, 6, 3, 40), 2
    N, B, S, Hq, Hkv, d = shape
    rng = np.random.default_rng(11)
    for layout in (0, 1):
        run = Run(emu, shape, oracle.GROUPS, layout, 2, None, G)
        nq, nkv = B * S * Hq * d, B * S * Hkv * d
        do = _rand(nq, 2, rng)
        out = _empty(nq, 2)
        run("emu_seq_to_head_o", do, out)
        assert np.array_equal(out, oracle.seq_to_head(do, oracle.GROUPS, N, B, S, Hq, d, layout, G=G))
        g = _rand(nq + 2 * nkv, 2, rng)
        dq, dk, dv = _empty(nq, 2), _empty(nkv, 2), _empty(nkv, 2)
        run("emu_head_to_seq_qkv", g, dq, dk, dv)
        wq, wk, wv = oracle.head_to_seq_qkv(g, oracle.GROUPS, N, B, S, Hq, Hkv, d, layout, G=G)
        assert np.array_equal(dq, wq) and np.array_equal(dk, wk) and np.array_equal(dv, wv)
        q, k, v = (_rand(n, 2, rng) for n in (nq, nkv, nkv))
        out = _empty(nq + 2 * nkv, 2)
        ws = _empty(2 * (nq + 2 * nkv), 2)
        run("emu_seq_to_head_unfused", q, k, v, out, ws)
        assert np.array_equal(out, oracle.seq_to_head_qkv(q, k, v, oracle.GROUPS, N, B, S, Hq, Hkv, d, layout,
                                                          G=G))


@pytest.mark.parametrize("seed", range(random_cases.GROUP_COUNT))
def test_random_general_groups(emu, seed):
    shape, G, layout, tuning = random_cases.group_case(seed)
    for es in (2, 4):
        check_s2h(emu, shape, oracle.GROUPS, layout, es, tuning, G=G)
        check_h2s(emu, shape, oracle.GROUPS, layout, es, tuning, G=G)


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("mode", [1, 0], ids=["basp", "ulysses"])
@pytest.mark.parametrize("shape", [(8, 2, 8 * 5, 24, 8, 128), (4, 2, 4 * 13, 8, 4, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_every_swept_launch_shape(emu, shape, mode, layout):
    """Each of the launch shapes the table's per-direction sweep can pick
    (bench.py sweep_grid, plus 8 vectors per lane), both directions, on small
    ragged shapes in both layouts: every access inside its descriptor and the
    oracle's result."""
    import bench
    N, B, S, Hq, Hkv, d = shape
    rng = np.random.default_rng(11)
    q, k, v, o = (_rand(B * S * H * d, 2, rng) for H in (Hq, Hkv, Hkv, Hq))
    want_qkv = oracle.seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, layout)
    want_o = oracle.head_to_seq(o, mode, N, B, S, Hq, d, layout)
    grid = bench.sweep_grid(2)
    grid += [dict(t, vectors_per_thread=8) for t in grid if t["vectors_per_thread"] == 4]
    for t in grid:
        run = Run(emu, shape, mode, layout, 2, t)
        out = _empty(want_qkv.size, 2)
        run("emu_seq_to_head", q, k, v, out)
        assert np.array_equal(out, want_qkv), ("seq->head", t)
        out = _empty(want_o.size, 2)
        run("emu_head_to_seq", o, out)
        assert np.array_equal(out, want_o), ("head->seq", t)


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
def test_every_swept_launch_shape_general_groups(emu, layout):
    """The sweep grid's launch shapes on a general G-group plan with G, P and
    Bl all above 1 (8 ranks, 4 sequences, 2 groups), both directions."""
    import bench
    N, B, S, Hq, Hkv, d, G = 8, 4, 4 * 5, 8, 4, 16, 2
    shape = (N, B, S, Hq, Hkv, d)
    rng = np.random.default_rng(12)
    q, k, v, o = (_rand(B * S * H * d, 2, rng) for H in (Hq, Hkv, Hkv, Hq))
    want_qkv = oracle.seq_to_head_qkv(q, k, v, oracle.GROUPS, N, B, S, Hq, Hkv, d, layout, G=G)
    want_o = oracle.head_to_seq(o, oracle.GROUPS, N, B, S, Hq, d, layout, G=G)
    grid = bench.sweep_grid(2)
    grid += [dict(t, vectors_per_thread=8) for t in grid if t["vectors_per_thread"] == 4]
    for t in grid:
        run = Run(emu, shape, oracle.GROUPS, layout, 2, t, G)
        out = _empty(want_qkv.size, 2)
        run("emu_seq_to_head", q, k, v, out)
        assert np.array_equal(out, want_qkv), ("seq->head", t)
        out = _empty(want_o.size, 2)
        run("emu_head_to_seq", o, out)
        assert np.array_equal(out, want_o), ("head->seq", t)
