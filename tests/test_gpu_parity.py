"""GPU parity: every entry point of libbasp against the CPU oracle, bit for
bit, on the same seeded bytes (MI355X only).

Coverage:
* every named workload at full size, both modes, seq->head (fused Q/K/V) and
  head->seq (O), compared element by element with the oracle;
* ragged shapes spanning several tiles with partial tiles at the end, odd row
  sizes (narrow vector paths), several launch shapes (tuning) and a capped
  grid (work-groups looping over tiles);
* edge cases: empty sequences, B = 1, K = 1, the data-parallel fallback
  (B > N), N = 1, unaligned (2-byte) views, all bf16 bit patterns;
* guard bands around the output and a sentinel fill (each destination written
  exactly once, nothing outside written);
* the backward entry points, the token-major layout and the unfused baseline;
* outputs beyond 4 GiB on sampled destinations, side streams and the NULL
  stream, a whole step captured in a HIP graph and replayed, autotuning;
* the plain copy the kernels are measured against (basp_stream_copy).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import random_cases
from sequence_re_layout_amd import inputs, workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sequence_re_layout_amd import binding as b
else:  # collected on a machine without a GPU: every test here is skipped
    b = None

MODE = {"basp": 1, "ulysses": 0, "groups": 2}
GUARD = 4096  # bytes of canary on each side of an output


def needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bits(t):
    return inputs.raw_bits(t.cpu())


def seq_inputs(B, S, Hq, Hkv, d, dtype):
    """Q, K, V as flat CPU tensors: N(0,1) bf16 from seeds 0/1/2, or int32 tags
    numbering the three tensors consecutively."""
    nq, nkv = B * S * Hq * d, B * S * Hkv * d
    if dtype == "int32":
        return (inputs.tags_int32(nq, 0), inputs.tags_int32(nkv, nq), inputs.tags_int32(nkv, nq + nkv))
    return (inputs.normal_bf16(nq, inputs.SEED_Q), inputs.normal_bf16(nkv, inputs.SEED_K),
            inputs.normal_bf16(nkv, inputs.SEED_V))


def guarded(numel, dtype):
    """Device buffer with GUARD bytes of canary on both sides; returns
    (whole, view).  The view is sentinel-filled: all-ones bits, a NaN for
    bf16 that N(0,1) never produces and -1 for int32, which tags never are."""
    es = torch.tensor([], dtype=dtype).element_size()
    g = GUARD // es
    whole = torch.empty(numel + 2 * g, dtype=dtype, device="cuda")
    raw = whole.view(torch.int16 if es == 2 else torch.int32)
    raw.fill_(-1)
    raw[:g] = 0x5A5A
    raw[g + numel:] = 0x5A5A
    return whole, whole[g:g + numel]


def check_guards(whole, numel):
    es = whole.element_size()
    g = GUARD // es
    raw = bits(whole)
    assert np.all(raw[:g] == 0x5A5A) and np.all(raw[g + numel:] == 0x5A5A), "guard band written"
    body = raw[g:g + numel]
    assert not np.any(body == np.iinfo(body.dtype).max), "a destination was never written"


TDT = {"bf16": (torch.bfloat16, 0), "int32": (torch.int32, 3), "fp16": (torch.float16, 1),
       "fp32": (torch.float32, 2)}


def make_plan(shape, mode, code, layout=0, G=0):
    N, B, S, Hq, Hkv, d = shape
    if mode == "groups":
        return b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, code, G, layout)
    return b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, code, MODE[mode], layout)


def run_s2h(shape, mode, dtype="bf16", layout=0, tuning=None, cpu=None, G=0):
    """Fused seq->head on the GPU and in the oracle; asserts bit equality."""
    N, B, S, Hq, Hkv, d = shape
    tdt, code = TDT[dtype]
    plan = make_plan(shape, mode, code, layout, G)
    if tuning:
        b.basp_plan_set_tuning(plan, **tuning)
    q, k, v = cpu or seq_inputs(B, S, Hq, Hkv, d, "int32" if dtype == "int32" else "bf16")
    q, k, v = (x.view(tdt) if x.element_size() == tdt.itemsize else x.to(tdt) for x in (q, k, v))
    whole, out = guarded(plan.info["qkv_elems"], tdt)
    b.basp_seq_to_head(plan, q.cuda(), k.cuda(), v.cuda(), out)
    torch.cuda.synchronize()
    check_guards(whole, plan.info["qkv_elems"])
    want = oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k), inputs.raw_bits(v),
                                  MODE[mode], N, B, S, Hq, Hkv, d, layout, G=G)
    got = bits(out)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, "first mismatches at %s" % bad[:8]
    return plan, out


def run_h2s(shape, mode, dtype="bf16", layout=0, tuning=None, G=0):
    N, B, S, Hq, Hkv, d = shape
    tdt, code = TDT[dtype]
    plan = make_plan(shape, mode, code, layout, G)
    if tuning:
        b.basp_plan_set_tuning(plan, **tuning)
    nq = plan.info["q_elems"]
    o = inputs.tags_int32(nq) if dtype == "int32" else inputs.normal_bf16(nq, inputs.SEED_O)
    o = o.view(tdt) if o.element_size() == tdt.itemsize else o.to(tdt)
    whole, out = guarded(nq, tdt)
    b.basp_head_to_seq(plan, o.cuda(), out)
    torch.cuda.synchronize()
    check_guards(whole, nq)
    want = oracle.head_to_seq(inputs.raw_bits(o), MODE[mode], N, B, S, Hq, d, layout, G=G)
    bad = np.flatnonzero(bits(out) != want)
    assert bad.size == 0, "first mismatches at %s" % bad[:8]


# ------------------------------------------------------- named workloads ---

@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", workloads.ALL + workloads.EXTRA, ids=[w[0] for w in workloads.ALL + workloads.EXTRA])
def test_workload_full_size(w, mode):
    needs_gpu()
    print("workload", w, mode, flush=True)
    shape = w[1:]
    run_s2h(shape, mode)
    run_h2s(shape, mode)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", [workloads.LLAMA_1B, workloads.LONG_CONTEXT[-1]],
                         ids=[workloads.LLAMA_1B[0], workloads.LONG_CONTEXT[-1][0]])
def test_workload_full_size_token_major(w, mode):
    """The token-major head layout ([Bl][S][Hl][d]) at full size."""
    needs_gpu()
    print("workload token-major", w, mode, flush=True)
    run_s2h(w[1:], mode, layout=1)
    run_h2s(w[1:], mode, layout=1)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
def test_tiny_int32_tagged(mode):
    needs_gpu()
    shape = workloads.TINY[1:]
    run_s2h(shape, mode, dtype="int32")
    run_h2s(shape, mode, dtype="int32")


def _pack(t, b, s, h, e):
    """(tensor, b, s, h, e) in bit fields of an int32: e bits 0-7, h 8-15,
    s 16-27, b 28, tensor 29-30 (fields wide enough for the tiny shape)."""
    return (t << 29) | (b << 28) | (s << 16) | (h << 8) | e


def _seq_tags(t, N, B, S, H, d, G, P, Bl):
    """Sequence-sharded buffer [N][Bl][St][H][d]: rank r = g*P + j holds
    sequences g*Bl + bl and tokens j*St + t."""
    St = S // P
    r, bl, tt, h, e = np.indices((N, Bl, St, H, d), dtype=np.int64)
    return _pack(t, (r // P) * Bl + bl, (r % P) * St + tt, h, e).astype(np.int32).ravel()


def _head_tags(t, N, B, S, H, d, G, P, Bl, layout):
    """Head-sharded buffer [N][Bl][Hl][S][d] (or [N][Bl][S][Hl][d]): rank
    r = g*P + j holds sequences g*Bl + bl and heads j*Hl + hl."""
    Hl = H // P
    if layout == 0:
        r, bl, hl, s, e = np.indices((N, Bl, Hl, S, d), dtype=np.int64)
    else:
        r, bl, s, hl, e = np.indices((N, Bl, S, Hl, d), dtype=np.int64)
    return _pack(t, (r // P) * Bl + bl, s, (r % P) * Hl + hl, e).astype(np.int32).ravel()


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("mode", ["basp", "ulysses"])
def test_tiny_tags_decode(mode, layout):
    """Every element of the tiny workload's Q/K/V/O carries its own (tensor,
    b, s, h, e) in bit fields; after the GPU re-layout each output position
    must hold the element the ownership rules put there (checked field by
    field from the layout definitions, independently of the oracle)."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = workloads.TINY[1:]
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_INT32, MODE[mode], layout)
    i = plan.info
    G, P, Bl = i["G"], i["P"], i["Bl"]
    ins = [torch.from_numpy(_seq_tags(t, N, B, S, H, d, G, P, Bl)).cuda()
           for t, H in ((0, Hq), (1, Hkv), (2, Hkv))]
    out = torch.full((i["qkv_elems"],), -1, dtype=torch.int32, device="cuda")
    b.basp_seq_to_head(plan, *ins, out)
    o = torch.from_numpy(_head_tags(3, N, B, S, Hq, d, G, P, Bl, layout)).cuda()
    back = torch.full((i["q_elems"],), -1, dtype=torch.int32, device="cuda")
    b.basp_head_to_seq(plan, o, back)
    torch.cuda.synchronize()
    want = np.concatenate([_head_tags(t, N, B, S, H, d, G, P, Bl, layout)
                           for t, H in ((0, Hq), (1, Hkv), (2, Hkv))])
    got = out.cpu().numpy()
    for name, shift, mask in (("tensor", 29, 3), ("b", 28, 1), ("s", 16, 0xfff), ("h", 8, 0xff), ("e", 0, 0xff)):
        bad = np.flatnonzero(((got >> shift) & mask) != ((want >> shift) & mask))
        assert bad.size == 0, "seq->head: field %s wrong at %s" % (name, bad[:8])
    want_back = _seq_tags(3, N, B, S, Hq, d, G, P, Bl)
    assert np.array_equal(back.cpu().numpy(), want_back), "head->seq: tags out of place"


# -------------------------------------------------- ragged, tunings, dtypes --

RAGGED = [  # N, B, S, Hq, Hkv, d
    (6, 3, 6 * 37, 12, 6, 40),     # St = 37 tokens, 80-byte rows (5 vectors)
    (4, 2, 4 * 203, 8, 4, 64),     # St = 203 > one tile
    (8, 2, 8 * 129, 24, 8, 128),   # Hl_q = 6 (BASP) / 3 (Ulysses)
    (3, 3, 3 * 11, 6, 3, 3),       # 6-byte rows: 2-byte vectors
    (2, 4, 2 * 50, 4, 2, 12),      # 24-byte rows: 8-byte vectors
]


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged(shape, mode):
    needs_gpu()
    for dtype in ("bf16", "int32"):
        for layout in (0, 1):
            run_s2h(shape, mode, dtype, layout)
            run_h2s(shape, mode, dtype, layout)


TUNINGS = [dict(vectors_per_thread=1), dict(vectors_per_thread=2), dict(vectors_per_thread=8),
           dict(tile_tokens=1), dict(tile_tokens=3, tile_heads=2), dict(tile_tokens=100, tile_heads=3),
           dict(cache_policy=1), dict(cache_policy=3), dict(max_grid=7),
           dict(vectors_per_thread=8, tile_tokens=5, tile_heads=1, cache_policy=3, max_grid=3),
           dict(lane_order=2, tile_heads=3, tile_tokens=7), dict(xcd_remap=2, max_grid=24),
           dict(xcd_remap=2, max_grid=13, lane_order=2),
           dict(tile_order=1), dict(tile_order=2, tile_heads=3, tile_tokens=5, max_grid=11),
           dict(stage=2), dict(stage=2, vectors_per_thread=1, tile_heads=8, cache_policy=2),
           dict(stage=2, vectors_per_thread=8, tile_tokens=500, tile_order=2, max_grid=5),
           dict(block_size=64, cache_policy=4), dict(block_size=128, stage=2, vectors_per_thread=8, cache_policy=5),
           dict(block_size=64, stage=1, tile_tokens=9, max_grid=7),
           dict(batch_order=2), dict(batch_order=2, stage=2, tile_order=1, xcd_remap=2, max_grid=9),
           dict(tile_order=3), dict(tile_order=3, tile_heads=3, tile_tokens=5, max_grid=11),
           dict(tile_order=3, stage=2, xcd_remap=2, batch_order=2, tile_heads=2)]


@pytest.mark.parametrize("tuning", TUNINGS, ids=lambda t: ",".join("%s=%s" % kv for kv in t.items()))
def test_tunings(tuning):
    needs_gpu()
    for shape, mode in (((8, 2, 8 * 129, 24, 8, 128), "basp"), ((6, 3, 6 * 37, 12, 6, 40), "ulysses")):
        for layout in (0, 1):
            run_s2h(shape, mode, "int32", layout, tuning)
            run_h2s(shape, mode, "int32", layout, tuning)


@pytest.mark.parametrize("dtype", ["fp16", "fp32"])
def test_other_dtypes(dtype):
    needs_gpu()
    run_s2h((4, 2, 4 * 33, 8, 4, 64), "basp", dtype)
    run_h2s((4, 2, 4 * 33, 8, 4, 64), "ulysses", dtype)


# ------------------------------------------------------------- edge cases --

def test_empty_sequence():
    needs_gpu()
    plan = b.basp_plan_create(8, 2, 0, 32, 8, 64)
    z = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    b.basp_seq_to_head(plan, z, z, z, z)
    b.basp_head_to_seq(plan, z, z)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape,mode", [
    ((8, 1, 8 * 16, 8, 8, 64), "basp"),       # B = 1: one group of N
    ((8, 8, 8 * 16, 8, 8, 64), "basp"),       # K = 1: purely local
    ((4, 16, 32, 8, 4, 64), "basp"),          # B > N: data-parallel fallback
    ((1, 3, 40, 4, 2, 64), "ulysses"),        # one rank
    ((1, 3, 40, 4, 2, 64), "basp"),
    ((8, 3, 8 * 5, 8, 8, 64), "ulysses"),     # Ulysses needs no N % B
])
def test_degenerate(shape, mode):
    needs_gpu()
    for layout in (0, 1):
        run_s2h(shape, mode, "int32", layout)
        run_h2s(shape, mode, "int32", layout)


@pytest.mark.parametrize("shape,mode", [
    ((1, 65535, 3, 2, 1, 8), "basp"),             # data-parallel fallback: 65535 batch indices along z
    ((5, 65535, 5, 5, 5, 8), "ulysses"),          # z = 65535, y = 5 members
    ((4096, 1, 4096, 4096, 4096, 1), "ulysses"),  # 4096 members along y, 2-byte rows
], ids=["z65535-dp", "z65535-ulysses", "y4096-ulysses"])
def test_grid_limits(shape, mode):
    """The launch grid at its extents (the largest batch count the grid's z
    coordinate takes; thousands of members along y), with the batch index
    along z or folded into x."""
    needs_gpu()
    for tuning in (None, {"batch_order": 2}):
        run_s2h(shape, mode, "bf16", 0, tuning)
        run_h2s(shape, mode, "bf16", 0, tuning)


def test_b1_basp_equals_ulysses():
    needs_gpu()
    shape = (8, 1, 8192, 32, 8, 64)
    _, a = run_s2h(shape, "basp")
    _, u = run_s2h(shape, "ulysses")
    assert torch.equal(a.view(torch.int16), u.view(torch.int16))


@pytest.mark.parametrize("shift", [1, 2, 4], ids=["2B", "4B", "8B"])
def test_unaligned_views(shift):
    """Tensors that start 2, 4 or 8 bytes past a 16-byte boundary take
    16-byte accesses at those addresses (direct and LDS-staged kernels,
    both directions) and give the same bits."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = 4, 2, 4 * 20, 8, 4, 64
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, 1)
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, "bf16")
    def shifted(t):
        buf = torch.empty(t.numel() + shift, dtype=t.dtype, device="cuda")
        buf[shift:].copy_(t.cuda())
        return buf[shift:]
    out_buf = torch.empty(plan.info["qkv_elems"] + shift, dtype=torch.bfloat16, device="cuda")
    out = out_buf[shift:]
    o_buf = torch.empty(plan.info["q_elems"] + shift, dtype=torch.bfloat16, device="cuda")
    o_out = o_buf[shift:]
    want = oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k), inputs.raw_bits(v),
                                  1, N, B, S, Hq, Hkv, d)
    o = q   # a Q-shaped head-sharded input for head->seq
    want_o = oracle.head_to_seq(inputs.raw_bits(o), 1, N, B, S, Hq, d)
    for tuning in ({}, dict(batch_order=2, max_grid=5, tile_order=1), dict(stage=2, block_size=64, tile_heads=2),
                   dict(tile_order=3, vectors_per_thread=2)):
        if tuning:
            b.basp_plan_set_tuning(plan, **tuning)
        out.fill_(0)
        o_out.fill_(0)
        b.basp_seq_to_head(plan, shifted(q), shifted(k), shifted(v), out)
        b.basp_head_to_seq(plan, shifted(o), o_out)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), want), tuning
        assert np.array_equal(bits(o_out), want_o), tuning


def test_all_bf16_patterns_round_trip():
    needs_gpu()
    pats = inputs.all_bf16_patterns()
    N, B, S, H, d = 4, 2, 16, 16, 128   # B*S*H*d = 65536
    for mode in (0, 1):
        plan = b.basp_plan_create(N, B, S, H, H, d, b.BASP_BF16, mode)
        x = pats.cuda()
        out = torch.empty(3 * x.numel(), dtype=torch.bfloat16, device="cuda")
        b.basp_seq_to_head(plan, x, x, x, out)
        back = torch.empty_like(x)
        b.basp_head_to_seq(plan, out[:x.numel()], back)
        torch.cuda.synchronize()
        assert np.array_equal(bits(back), inputs.raw_bits(pats))
        want = oracle.seq_to_head(inputs.raw_bits(pats), mode, N, B, S, H, d)
        assert np.array_equal(bits(out[2 * x.numel():]), want)


def test_device_round_trip():
    needs_gpu()
    N, B, S, Hq, Hkv, d = workloads.LLAMA_1B[1:]
    for mode in (0, 1):
        plan = b.basp_plan_create(N, B, S, Hq, Hq, d, b.BASP_BF16, mode)  # Hkv := Hq
        q = inputs.normal_bf16(plan.info["q_elems"], 11).cuda()
        out = torch.empty(plan.info["qkv_elems"], dtype=torch.bfloat16, device="cuda")
        b.basp_seq_to_head(plan, q, q, q, out)
        back = torch.empty_like(q)
        b.basp_head_to_seq(plan, out[plan.info["qkv_offset_v"]:], back)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16), q.view(torch.int16))


# ----------------------------------------- backward, layout, unfused paths --

@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [workloads.LLAMA_1B[1:], (6, 3, 6 * 37, 12, 6, 40)],
                         ids=["llama1b", "ragged"])
def test_backward_entries(shape, layout, mode):
    needs_gpu()
    N, B, S, Hq, Hkv, d = shape
    m = MODE[mode]
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_BF16, m, layout)
    i = plan.info
    # dO: seq -> head
    do = inputs.normal_bf16(i["q_elems"], 21)
    out = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
    b.basp_seq_to_head_o(plan, do.cuda(), out)
    # fused dQ/dK/dV: head -> seq
    g = inputs.normal_bf16(i["qkv_elems"], 22)
    dq = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
    dk = torch.empty(i["kv_elems"], dtype=torch.bfloat16, device="cuda")
    dv = torch.empty(i["kv_elems"], dtype=torch.bfloat16, device="cuda")
    b.basp_head_to_seq_qkv(plan, g.cuda(), dq, dk, dv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), oracle.seq_to_head(inputs.raw_bits(do), m, N, B, S, Hq, d, layout))
    wq, wk, wv = oracle.head_to_seq_qkv(inputs.raw_bits(g), m, N, B, S, Hq, Hkv, d, layout)
    assert np.array_equal(bits(dq), wq) and np.array_equal(bits(dk), wk) and np.array_equal(bits(dv), wv)


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("mode", ["basp", "ulysses"])
def test_autograd_wrappers(mode, layout):
    """sequence_re_layout_amd.autograd: the forward results are the oracle's,
    and torch.autograd's gradients through them are the oracle's inverse
    re-layouts of the upstream gradients (a permutation's adjoint is its
    inverse), bit for bit; a boundary round trip O := HEAD(Q) gives Q back
    with the upstream gradient as Q's gradient."""
    needs_gpu()
    from sequence_re_layout_amd import autograd as ag
    N, B, S, Hq, Hkv, d = (6, 3, 6 * 37, 12, 6, 40)
    m = MODE[mode]
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_BF16, m, layout)
    i = plan.info
    q = inputs.normal_bf16(i["q_elems"], 31).cuda().requires_grad_()
    k = inputs.normal_bf16(i["kv_elems"], 32).cuda().requires_grad_()
    v = inputs.normal_bf16(i["kv_elems"], 33).cuda().requires_grad_()
    qkv = ag.seq_to_head_qkv(plan, q, k, v)
    assert np.array_equal(bits(qkv.detach()), oracle.seq_to_head_qkv(
        bits(q.detach()), bits(k.detach()), bits(v.detach()), m, N, B, S, Hq, Hkv, d, layout))
    g = inputs.normal_bf16(i["qkv_elems"], 34)
    dq, dk, dv = torch.autograd.grad(qkv, (q, k, v), g.cuda())
    wq, wk, wv = oracle.head_to_seq_qkv(inputs.raw_bits(g), m, N, B, S, Hq, Hkv, d, layout)
    assert np.array_equal(bits(dq), wq) and np.array_equal(bits(dk), wk) and np.array_equal(bits(dv), wv)
    o = inputs.normal_bf16(i["q_elems"], 35).cuda().requires_grad_()
    y = ag.head_to_seq_o(plan, o)
    assert np.array_equal(bits(y.detach()), oracle.head_to_seq(bits(o.detach()), m, N, B, S, Hq, d, layout))
    go = inputs.normal_bf16(i["q_elems"], 36)
    (do,) = torch.autograd.grad(y, (o,), go.cuda())
    assert np.array_equal(bits(do), oracle.seq_to_head(inputs.raw_bits(go), m, N, B, S, Hq, d, layout))
    # round trip through both wrappers: Q back, and Q's gradient is the upstream one
    back = ag.head_to_seq_o(plan, ag.seq_to_head_qkv(plan, q, k, v)[: i["q_elems"]])
    assert torch.equal(back.detach().view(torch.int16), q.detach().view(torch.int16))
    (dq2,) = torch.autograd.grad(back, (q,), go.cuda())
    assert torch.equal(dq2.view(torch.int16), go.cuda().view(torch.int16))


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [workloads.LLAMA_1B[1:], workloads.QWEN_1_8B[1:],
                                   (6, 3, 6 * 37, 12, 6, 40), (3, 3, 3 * 11, 6, 3, 3)],
                         ids=["llama1b", "qwen", "ragged", "narrow"])
def test_unfused_matches_oracle(shape, layout, mode):
    needs_gpu()
    N, B, S, Hq, Hkv, d = shape
    m = MODE[mode]
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_BF16, m, layout)
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, "bf16")
    ws = torch.empty(b.basp_unfused_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    whole, out = guarded(plan.info["qkv_elems"], torch.bfloat16)
    b.basp_seq_to_head_unfused(plan, q.cuda(), k.cuda(), v.cuda(), out, ws)
    torch.cuda.synchronize()
    check_guards(whole, plan.info["qkv_elems"])
    want = oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k), inputs.raw_bits(v),
                                  m, N, B, S, Hq, Hkv, d, layout)
    assert np.array_equal(bits(out), want)


def test_unfused_unaligned_views():
    """The unfused baseline on views 2 bytes past a 16-byte boundary (its
    inputs, output and workspace) keeps 16-byte accesses and gives the
    oracle's bits."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = 8, 2, 8 * 16, 32, 8, 64
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, 1)
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, "bf16")
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        buf[1:].copy_(t.cuda())
        return buf[1:]
    ws_buf = torch.empty(b.basp_unfused_workspace_bytes(plan) + 2, dtype=torch.uint8, device="cuda")
    out_buf = torch.zeros(plan.info["qkv_elems"] + 1, dtype=torch.bfloat16, device="cuda")
    out = out_buf[1:]
    b.basp_seq_to_head_unfused(plan, shifted(q), shifted(k), shifted(v), out, ws_buf.data_ptr() + 2)
    torch.cuda.synchronize()
    want = oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k), inputs.raw_bits(v),
                                  1, N, B, S, Hq, Hkv, d)
    assert np.array_equal(bits(out), want)


# ------------------------------------------------------------ error paths --

def test_device_error_paths():
    needs_gpu()
    plan = b.basp_plan_create(4, 2, 64, 8, 8, 64)
    i = plan.info
    q = torch.zeros(i["q_elems"], dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.BaspError) as e:
        b.basp_seq_to_head(plan, q, q, q, out.data_ptr() + 1)
    assert e.value.status == b.BASP_ERR_ALIGN
    with pytest.raises(b.BaspError) as e:
        b.basp_seq_to_head(plan, q, q, q, q.data_ptr())
    assert e.value.status == b.BASP_ERR_ALIAS
    with pytest.raises(TypeError):
        b.basp_seq_to_head(plan, q.float(), q, q, out)
    with pytest.raises(ValueError):
        b.basp_seq_to_head(plan, q[:-1], q, q, out)
    # q, k and v may share one buffer
    b.basp_seq_to_head(plan, q, q, q, out)
    torch.cuda.synchronize()
    # the NULL stream (0) is a valid stream
    N, B, S, Hq, Hkv, d = 4, 2, 64, 8, 8, 64
    qt, kt, vt = (x.cuda() for x in seq_inputs(B, S, Hq, Hkv, d, "int32"))
    plan32 = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_INT32, b.BASP_MODE_BASP)
    out32 = torch.empty(plan32.info["qkv_elems"], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    b.basp_seq_to_head(plan32, qt, kt, vt, out32, stream=0)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out32), oracle.seq_to_head_qkv(bits(qt), bits(kt), bits(vt), 1, N, B, S, Hq, Hkv, d))


def test_single_hip_runtime_and_native_library():
    """libbasp.so is loaded from the tree and shares torch's HIP runtime: one
    libamdhip64 image in the process."""
    needs_gpu()
    maps = open("/proc/self/maps").read().splitlines()
    hip = sorted({l.split()[-1] for l in maps if "libamdhip64" in l})
    assert len(hip) == 1, hip
    basp = sorted({l.split()[-1] for l in maps if l.endswith("libbasp.so")})
    assert basp == [b.LIB_PATH], basp


def test_timed_call_records_kernel_time_and_keeps_results():
    """basp_time_next_call: the events get the kernel's start and end, the
    result is unchanged, and the request applies to one call only."""
    needs_gpu()
    shape = (8, 2, 8 * 129, 24, 8, 128)
    N, B, S, Hq, Hkv, d = shape
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, 1)
    q, k, v = (x.cuda() for x in seq_inputs(B, S, Hq, Hkv, d, "bf16"))
    ref = torch.empty(plan.info["qkv_elems"], dtype=torch.bfloat16, device="cuda")
    b.basp_seq_to_head(plan, q, k, v, ref)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    b.basp_time_next_call(ev[0], ev[1])
    b.basp_seq_to_head(plan, q, k, v, out)
    torch.cuda.synchronize()
    t = ev[0].elapsed_time(ev[1])
    assert 0 < t < 1000.0
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # the request was consumed: a second call leaves ev[2]/ev[3] as recorded
    before = ev[2].elapsed_time(ev[3])
    b.basp_seq_to_head(plan, q, k, v, out)
    torch.cuda.synchronize()
    assert ev[2].elapsed_time(ev[3]) == before
    # the unfused path: start at its first kernel, stop at its last
    ws = torch.empty(b.basp_unfused_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    b.basp_time_next_call(ev[0], ev[1])
    b.basp_seq_to_head_unfused(plan, q, k, v, out, ws)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # a call that fails its checks also consumes the request
    before = ev[2].elapsed_time(ev[3])
    b.basp_time_next_call(ev[2], ev[3])
    lib = b.library()
    assert lib.basp_seq_to_head(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                out.data_ptr() + 1, None) == b.BASP_ERR_ALIGN
    b.basp_seq_to_head(plan, q, k, v, out)
    torch.cuda.synchronize()
    assert ev[2].elapsed_time(ev[3]) == before


@pytest.mark.parametrize("shape,mode", [(workloads.LLAMA_1B[1:], 1), ((6, 3, 6 * 37, 12, 6, 40), 0)],
                         ids=["llama1b-basp", "ragged-ulysses"])
def test_autotune_keeps_results(shape, mode):
    """basp_plan_autotune stores a valid launch shape per direction and the
    re-layout stays bit-exact with it.  The Llama-3.2-1B plan's six buffers
    (670 MB) are timed on themselves; the ragged plan's are below 32 MiB, so
    its launches are timed on the temporary pool and only the final run of
    the chosen shapes writes the caller's outputs, which start sentinel-filled
    here."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = shape
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, mode)
    i = plan.info
    q, k, v = (x.cuda() for x in seq_inputs(B, S, Hq, Hkv, d, "bf16"))
    o = inputs.normal_bf16(i["q_elems"], inputs.SEED_O).cuda()
    qkv = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
    o_out = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
    qkv.view(torch.int16).fill_(-1)
    o_out.view(torch.int16).fill_(-1)
    b.basp_plan_autotune(plan, q, k, v, qkv, o, o_out)
    torch.cuda.synchronize()
    want = oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), mode, N, B, S, Hq, Hkv, d)
    want_o = oracle.head_to_seq(bits(o), mode, N, B, S, Hq, d)
    # every measured launch computes the same re-layout into the same buffers
    assert np.array_equal(bits(qkv), want)
    assert np.array_equal(bits(o_out), want_o)
    for direction in (b.BASP_SEQ_TO_HEAD, b.BASP_HEAD_TO_SEQ):
        t = b.basp_plan_get_tuning(plan, direction)
        if not any(t.values()):   # the plan's shapes on entry (built-in) won
            continue
        assert t["vectors_per_thread"] in (1, 2, 4, 8) and t["cache_policy"] == 4
        assert t["block_size"] in (64, 128, 256) and t["xcd_remap"] in (1, 2)
        assert t["stage"] in (1, 2) and t["tile_order"] in (1, 2, 3)   # a measured candidate
    qkv.fill_(0)
    o_out.fill_(0)
    b.basp_seq_to_head(plan, q, k, v, qkv)
    b.basp_head_to_seq(plan, o, o_out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(qkv), want)
    assert np.array_equal(bits(o_out), want_o)


def _sample(n, rng, extra=()):
    """Random element offsets of a tensor of n elements plus its first and last
    elements and given offsets."""
    pts = list(rng.integers(0, n, size=200000)) + [0, 1, n - 2, n - 1] + [x for x in extra if 0 <= x < n]
    return np.unique(np.array(pts, dtype=np.int64))


# ------------------------------------- full size, the shapes the bench times --

def split_tags(sizes):
    """Two passes of bf16 device tensors of the given element counts.  Element
    i of the tensors taken one after another (i counted across all of them)
    carries the low 16 bits of i in the first pass and the high 16 bits in
    the second, so the two outputs together name the source of every output
    element (fewer than 2^32 elements)."""
    total = sum(sizes)
    assert total < 2**32
    idx = torch.arange(total, dtype=torch.int64, device="cuda")
    passes = []
    for shift in (0, 16):
        t = (((idx >> shift) & 0xFFFF) - 32768).to(torch.int16).view(torch.bfloat16)
        parts, base = [], 0
        for n in sizes:
            parts.append(t[base:base + n])
            base += n
        passes.append(parts)
    del idx
    return passes


def check_s2h_full(plan, mode, shape, ins, layout=0, G=0):
    """Fused seq->head of device tensors ins = (q, k, v) against the oracle,
    every element."""
    N, B, S, Hq, Hkv, d = shape
    i = plan.info
    out = torch.empty(i["qkv_elems"], dtype=ins[0].dtype, device="cuda")
    out.view(torch.int16 if out.element_size() == 2 else torch.int32).fill_(-1)
    b.basp_seq_to_head(plan, *ins, out)
    torch.cuda.synchronize()
    want = oracle.seq_to_head_qkv(*(bits(x) for x in ins), MODE[mode], N, B, S, Hq, Hkv, d, layout, G=G)
    bad = np.flatnonzero(bits(out) != want)
    assert bad.size == 0, "seq->head: %d mismatches, first at %s" % (bad.size, bad[:8])


def check_h2s_full(plan, mode, shape, o, layout=0, G=0):
    """O head->seq of a device tensor o against the oracle, every element."""
    N, B, S, Hq, Hkv, d = shape
    out = torch.empty_like(o)
    out.view(torch.int16 if out.element_size() == 2 else torch.int32).fill_(-1)
    b.basp_head_to_seq(plan, o, out)
    torch.cuda.synchronize()
    want = oracle.head_to_seq(bits(o), MODE[mode], N, B, S, Hq, d, layout, G=G)
    bad = np.flatnonzero(bits(out) != want)
    assert bad.size == 0, "head->seq: %d mismatches, first at %s" % (bad.size, bad[:8])


def check_split_tags(plan, mode, shape, layout=0, G=0):
    """Both directions with the plan's current launch shapes, on both passes
    of split tags, every element against the oracle."""
    i = plan.info
    for q, k, v in split_tags([i["q_elems"], i["kv_elems"], i["kv_elems"]]):
        check_s2h_full(plan, mode, shape, (q, k, v), layout, G)
    for (o,) in split_tags([i["q_elems"]]):
        check_h2s_full(plan, mode, shape, o, layout, G)


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", workloads.ALL + workloads.EXTRA, ids=lambda w: w[0])
def test_workload_table_shapes_split_tags(w, mode):
    """Every named workload with the launch shapes of the measured table
    (the ones the benchmark times), at full size: both passes of split tags,
    both directions, every output element against the oracle."""
    needs_gpu()
    from sequence_re_layout_amd import launch_shapes
    name, N, B, S, Hq, Hkv, d = w
    print("table shapes", name, mode, launch_shapes.lookup(name, mode), flush=True)
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, MODE[mode])
    if not launch_shapes.apply(b, plan, name, mode):
        pytest.skip("no table entry for %s %s" % (name, mode))
    check_split_tags(plan, mode, w[1:])
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", workloads.ALL + workloads.EXTRA, ids=lambda w: w[0])
def test_workload_autotuned_full_size(w, mode):
    """Every named workload with the launch shapes autotune picks for it:
    the outputs autotune leaves behind, then fresh calls of both directions
    on both passes of split tags, every element against the oracle."""
    needs_gpu()
    name, N, B, S, Hq, Hkv, d = w
    print("autotuned", name, mode, flush=True)
    m = MODE[mode]
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, m)
    i = plan.info
    (q, k, v), = split_tags([i["q_elems"], i["kv_elems"], i["kv_elems"]])[:1]
    (o,), = split_tags([i["q_elems"]])[1:]
    qkv = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
    o_out = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
    b.basp_plan_autotune(plan, q, k, v, qkv, o, o_out)
    torch.cuda.synchronize()
    print("  picked", b.basp_plan_get_tuning(plan, b.BASP_SEQ_TO_HEAD),
          b.basp_plan_get_tuning(plan, b.BASP_HEAD_TO_SEQ), flush=True)
    want = oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), m, N, B, S, Hq, Hkv, d)
    assert np.array_equal(bits(qkv), want), "seq->head result autotune left"
    assert np.array_equal(bits(o_out), oracle.head_to_seq(bits(o), m, N, B, S, Hq, d)), \
        "head->seq result autotune left"
    del q, k, v, o, qkv, o_out, want
    check_split_tags(plan, mode, w[1:])
    torch.cuda.empty_cache()


STAGED = [dict(stage=2, block_size=64, vectors_per_thread=1, tile_heads=2),
          dict(stage=2, block_size=256, vectors_per_thread=2, tile_heads=4, tile_order=1, batch_order=2),
          dict(stage=2, block_size=128, vectors_per_thread=1, tile_heads=1, xcd_remap=2)]


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("tuning", STAGED, ids=lambda t: ",".join("%s=%s" % kv for kv in t.items()))
@pytest.mark.parametrize("w", [workloads.LONG_CONTEXT[-1], workloads.DP_FALLBACK], ids=lambda w: w[0])
def test_staged_full_size(w, tuning, mode):
    """The LDS-staged kernel at full size on the largest named workload and on
    the data-parallel fallback, both directions, both modes, split tags."""
    needs_gpu()
    name, N, B, S, Hq, Hkv, d = w
    print("staged", name, mode, tuning, flush=True)
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, MODE[mode])
    b.basp_plan_set_tuning(plan, **tuning)
    check_split_tags(plan, mode, w[1:])
    torch.cuda.empty_cache()


def _global_tags(B, S, H, d, base):
    """int32 tags of a global [B][S][H][d] tensor: base + ((b*S + s)*H + h)*d + e."""
    return torch.arange(base, base + B * S * H * d, dtype=torch.int32, device="cuda").view(B, S, H, d)


@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("w", [workloads.LLAMA_1B, workloads.LONG_CONTEXT[-1]], ids=lambda w: w[0])
def test_int32_global_tags_full_size(w, mode):
    """int32 elements tagged with their (tensor, b, s, h, e) as the linear
    index into the global [Q||K||V] tensor (below 2^31 at every named
    workload), scattered into the mode's sequence-sharded buffers by the
    ownership rules, re-laid at full size in both directions with the table's
    shapes (built-in where the table has none for int32), every element
    against the oracle."""
    needs_gpu()
    name, N, B, S, Hq, Hkv, d = w
    print("int32 global tags", name, mode, flush=True)
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_INT32, MODE[mode])
    i = plan.info
    G, P, Bl = i["G"], i["P"], i["Bl"]
    assert i["qkv_elems"] < 2**31
    nq, nkv = i["q_elems"], i["kv_elems"]
    ins = []
    for base, H in ((0, Hq), (nq, Hkv), (nq + nkv, Hkv)):
        x = _global_tags(B, S, H, d, base)
        ins.append(x.view(G, Bl, P, S // P, H, d).permute(0, 2, 1, 3, 4, 5).contiguous().view(-1))
        del x
    check_s2h_full(plan, mode, w[1:], ins)
    del ins
    x = _global_tags(B, S, Hq, d, 0)
    o = x.view(G, Bl, S, P, Hq // P, d).permute(0, 3, 1, 4, 2, 5).contiguous().view(-1)
    del x
    check_h2s_full(plan, mode, w[1:], o)
    del o
    torch.cuda.empty_cache()


# --------------------------------------------------------- general G groups --

@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_general_groups_full_size(G):
    """The batch-sweep shape at B = 8 (N = 8, S = 8192, Llama-3.2-1B heads)
    in the general form with G groups of N/G ranks: the built-in launch
    shape, the shape autotune picks, an LDS-staged shape and a shape in
    tile order 3, each on both passes of split tags in both directions,
    every element against the oracle."""
    needs_gpu()
    name, N, B, S, Hq, Hkv, d = workloads.BATCH_SWEEP[-1]
    shape = (N, B, S, Hq, Hkv, d)
    assert B == 8
    print("general groups", name, "G =", G, flush=True)
    plan = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G)
    assert (plan.info["G"], plan.info["P"], plan.info["Bl"]) == (G, N // G, B // G)
    check_split_tags(plan, "groups", shape, G=G)
    i = plan.info
    dev = lambda n: torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    q, k, v, o = dev(i["q_elems"]), dev(i["kv_elems"]), dev(i["kv_elems"]), dev(i["q_elems"])
    b.basp_plan_autotune(plan, q, k, v, torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda"), o,
                         torch.empty_like(o))
    del q, k, v, o
    print("  autotuned", b.basp_plan_get_tuning(plan, 0), b.basp_plan_get_tuning(plan, 1), flush=True)
    check_split_tags(plan, "groups", shape, G=G)
    b.basp_plan_set_tuning(plan, stage=2, block_size=64, tile_heads=2, batch_order=2)
    check_split_tags(plan, "groups", shape, G=G)
    b.basp_plan_set_tuning(plan, tile_order=3, block_size=128, tile_heads=2, lane_order=1)
    check_split_tags(plan, "groups", shape, G=G)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G", [2, 4])
def test_general_groups_full_size_token_major(G):
    needs_gpu()
    name, N, B, S, Hq, Hkv, d = workloads.BATCH_SWEEP[-1]
    print("general groups token-major", name, "G =", G, flush=True)
    plan = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G, b.BASP_LAYOUT_TOKEN_MAJOR)
    check_split_tags(plan, "groups", (N, B, S, Hq, Hkv, d), layout=1, G=G)
    torch.cuda.empty_cache()


GROUP_CASES = [  # (N, B, S, Hq, Hkv, d), G -- also run by the CPU emulation
    ((6, 4, 6 * 5, 6, 3, 40), 2), ((12, 6, 12 * 3, 12, 4, 24), 3),
    ((8, 16, 8 * 4, 8, 4, 8), 4), ((4, 6, 4 * 7, 4, 2, 3), 2),
]


@pytest.mark.parametrize("case", GROUP_CASES, ids=lambda c: "x".join(map(str, c[0])) + "_G%d" % c[1])
def test_general_groups_ragged(case):
    needs_gpu()
    shape, G = case
    for tuning in (None, dict(batch_order=2), dict(stage=2, tile_heads=2),
                   dict(tile_order=1, xcd_remap=2, max_grid=5)):
        for layout in (0, 1):
            for dtype in ("bf16", "int32"):
                run_s2h(shape, "groups", dtype, layout, tuning, G=G)
                run_h2s(shape, "groups", dtype, layout, tuning, G=G)


@pytest.mark.parametrize("seed", range(random_cases.GROUP_COUNT))
def test_random_general_groups(seed):
    """Seeded random general-G plans and launch shapes (run first by the CPU
    emulation with its bounds checks)."""
    needs_gpu()
    shape, G, layout, tuning = random_cases.group_case(seed)
    dtype = "int32" if seed % 2 else "bf16"
    print("random general-G case", seed, shape, G, layout, tuning, flush=True)
    run_s2h(shape, "groups", dtype, layout, tuning, G=G)
    run_h2s(shape, "groups", dtype, layout, tuning, G=G)


def test_general_groups_backward():
    needs_gpu()
    shape, G = (6, 4, 6 * 5, 6, 3, 40), 2
    N, B, S, Hq, Hkv, d = shape
    for layout in (0, 1):
        plan = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G, layout)
        i = plan.info
        do = inputs.normal_bf16(i["q_elems"], 31)
        out = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
        b.basp_seq_to_head_o(plan, do.cuda(), out)
        g = inputs.normal_bf16(i["qkv_elems"], 32)
        dq = torch.empty(i["q_elems"], dtype=torch.bfloat16, device="cuda")
        dk = torch.empty(i["kv_elems"], dtype=torch.bfloat16, device="cuda")
        dv = torch.empty(i["kv_elems"], dtype=torch.bfloat16, device="cuda")
        b.basp_head_to_seq_qkv(plan, g.cuda(), dq, dk, dv)
        q, k, v = seq_inputs(B, S, Hq, Hkv, d, "bf16")
        ws = torch.empty(b.basp_unfused_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
        uf = torch.empty(i["qkv_elems"], dtype=torch.bfloat16, device="cuda")
        b.basp_seq_to_head_unfused(plan, q.cuda(), k.cuda(), v.cuda(), uf, ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), oracle.seq_to_head(inputs.raw_bits(do), 2, N, B, S, Hq, d, layout, G=G))
        wq, wk, wv = oracle.head_to_seq_qkv(inputs.raw_bits(g), 2, N, B, S, Hq, Hkv, d, layout, G=G)
        assert np.array_equal(bits(dq), wq) and np.array_equal(bits(dk), wk) and np.array_equal(bits(dv), wv)
        assert np.array_equal(bits(uf), oracle.seq_to_head_qkv(inputs.raw_bits(q), inputs.raw_bits(k),
                                                                inputs.raw_bits(v), 2, N, B, S, Hq, Hkv, d,
                                                                layout, G=G))


@pytest.mark.parametrize("mode,layout", [(1, 0), (0, 0), (1, 1)], ids=["basp", "ulysses", "basp-token-major"])
def test_beyond_4gib_sampled(mode, layout):
    """Buffers larger than 2^31 and 2^32 bytes (int32, S = 98304): the fused
    output is 4.8 GB and Q 3.2 GB, so tile bases need more than 32 bits.
    Tags name each element's source; sampled outputs, including the elements
    around the 2 GiB and 4 GiB byte offsets, are checked against the oracle's
    one-element source index."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = 8, 2, 98304, 32, 8, 128
    print("beyond 4 GiB", mode, layout, flush=True)
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, b.BASP_INT32, mode, layout)
    i = plan.info
    nq, nkv = i["q_elems"], i["kv_elems"]
    assert 4 * i["qkv_elems"] > 2**32 and 4 * nq > 2**31
    q = inputs.tags_int32(nq, 0, "cuda")
    k = inputs.tags_int32(nkv, nq, "cuda")
    v = inputs.tags_int32(nkv, nq + nkv, "cuda")
    out = torch.empty(i["qkv_elems"], dtype=torch.int32, device="cuda")
    b.basp_seq_to_head(plan, q, k, v, out)
    rng = np.random.default_rng(7)
    edges = [(1 << 29) + x for x in range(-3, 3)] + [(1 << 30) + x for x in range(-3, 3)]
    for base, n, H in ((0, nq, Hq), (nq, nkv, Hkv), (nq + nkv, nkv, Hkv)):
        dst = _sample(n, rng, [e - base for e in edges])
        got = out[torch.from_numpy(dst + base).cuda()].cpu().numpy().astype(np.int64)
        want = oracle.source_index(0, dst, mode, N, B, S, H, d, layout) + base
        assert np.array_equal(got, want), "seq->head mismatch in the tensor at %d" % base
    del q, k, v, out
    o = inputs.tags_int32(nq, 0, "cuda")
    back = torch.empty_like(o)
    b.basp_head_to_seq(plan, o, back)
    dst = _sample(nq, rng, edges)
    got = back[torch.from_numpy(dst).cuda()].cpu().numpy().astype(np.int64)
    assert np.array_equal(got, oracle.source_index(1, dst, mode, N, B, S, Hq, d, layout))
    del o, back
    torch.cuda.empty_cache()


def test_side_stream():
    """The library launches on the stream it is given: torch's current stream
    (a side stream here), or an explicit handle."""
    needs_gpu()
    shape = (6, 3, 6 * 37, 12, 6, 40)
    N, B, S, Hq, Hkv, d = shape
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, 1)
    q, k, v = (x.cuda() for x in seq_inputs(B, S, Hq, Hkv, d, "bf16"))
    want = oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), 1, N, B, S, Hq, Hkv, d)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()   # default priority
    with torch.cuda.stream(side):
        out = torch.empty(plan.info["qkv_elems"], dtype=torch.bfloat16, device="cuda")
        b.basp_seq_to_head(plan, q, k, v, out)
    side.synchronize()
    assert np.array_equal(bits(out), want)
    out2 = torch.empty_like(out)
    b.basp_seq_to_head(plan, q, k, v, out2, stream=side.cuda_stream)
    side.synchronize()
    assert np.array_equal(bits(out2), want)


@pytest.mark.parametrize("shape", [workloads.LLAMA_1B[1:], (6, 3, 6 * 37, 12, 6, 40)],
                         ids=["llama1b", "ragged"])
def test_graph_capture_replays(shape):
    """Every entry point launches only kernels on its stream (no allocation,
    no memset, no synchronisation), so a whole step captures into a HIP
    graph.  Each replay runs on fresh inputs copied into the captured
    buffers, with eager work and synchronisation between replays, and is
    checked against the oracle."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = shape
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, 1)
    i = plan.info
    nq, nkv, nqkv = i["q_elems"], i["kv_elems"], i["qkv_elems"]
    dev = lambda n: torch.empty(n, dtype=torch.bfloat16, device="cuda")
    q, k, v, o, do, g = dev(nq), dev(nkv), dev(nkv), dev(nq), dev(nq), dev(nqkv)
    qkv, qkv_u, o_seq, do_head = dev(nqkv), dev(nqkv), dev(nq), dev(nq)
    dq, dk, dv = dev(nq), dev(nkv), dev(nkv)
    ws = torch.empty(b.basp_unfused_workspace_bytes(plan), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.basp_seq_to_head(plan, q, k, v, qkv)
        b.basp_head_to_seq(plan, o, o_seq)
        b.basp_seq_to_head_o(plan, do, do_head)
        b.basp_head_to_seq_qkv(plan, g, dq, dk, dv)
        b.basp_seq_to_head_unfused(plan, q, k, v, qkv_u, ws)
    torch.cuda.synchronize()

    for rep in range(3):
        seeds = [100 + 10 * rep + j for j in range(6)]
        host = [inputs.normal_bf16(n, s) for n, s in zip((nq, nkv, nkv, nq, nq, nqkv), seeds)]
        for dst, src in zip((q, k, v, o, do, g), host):
            dst.copy_(src)
        for t in (qkv, qkv_u, o_seq, do_head, dq, dk, dv):
            t.fill_(float("nan"))
        scratch = dev(nq)
        b.basp_head_to_seq(plan, o, scratch)          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hq, hk, hv, ho, hdo, hg = (inputs.raw_bits(x) for x in host)
        want = oracle.seq_to_head_qkv(hq, hk, hv, 1, N, B, S, Hq, Hkv, d)
        assert np.array_equal(bits(qkv), want), "replay %d: fused seq->head" % rep
        assert np.array_equal(bits(qkv_u), want), "replay %d: unfused seq->head" % rep
        want_o = oracle.head_to_seq(ho, 1, N, B, S, Hq, d)
        assert np.array_equal(bits(o_seq), want_o), "replay %d: head->seq" % rep
        assert np.array_equal(bits(scratch), want_o), "replay %d: eager head->seq" % rep
        assert np.array_equal(bits(do_head), oracle.seq_to_head(hdo, 1, N, B, S, Hq, d)), \
            "replay %d: dO seq->head" % rep
        wq, wk, wv = oracle.head_to_seq_qkv(hg, 1, N, B, S, Hq, Hkv, d)
        assert np.array_equal(bits(dq), wq) and np.array_equal(bits(dk), wk) and \
            np.array_equal(bits(dv), wv), "replay %d: fused dQ/dK/dV head->seq" % rep
    del graph


@pytest.mark.parametrize("nbytes", [16, 1008, 1024, 1040, (3 << 20) + 112, (4 << 30) + 1040],
                         ids=["16B", "1008B", "1KiB", "1040B", "3MiB+112", "4GiB+1040"])
def test_stream_copy(nbytes):
    """The copy the re-layout is measured against: every byte copied, nothing
    outside the destination written.  4 GiB + 1040 bytes takes offsets past
    32 bits and more chunks than the grid, so work-groups loop."""
    needs_gpu()
    gen = torch.Generator(device="cuda").manual_seed(nbytes % 1000003)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    whole = torch.full((nbytes + 2 * GUARD,), 0x5A, dtype=torch.uint8, device="cuda")
    dst = whole[GUARD:GUARD + nbytes]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()   # torch creates an event's handle when it is first recorded
    stop.record()
    torch.cuda.synchronize()
    b.basp_time_next_call(start, stop)
    b.basp_stream_copy(dst, src)
    torch.cuda.synchronize()
    assert start.elapsed_time(stop) > 0
    assert torch.equal(dst, src)
    assert bool((whole[:GUARD] == 0x5A).all()) and bool((whole[GUARD + nbytes:] == 0x5A).all())
    del src, whole, dst
    torch.cuda.empty_cache()


def test_stream_copy_errors_on_device():
    needs_gpu()
    x = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(b.BaspError):
        b.basp_stream_copy(x[16:], x, 1024)           # overlapping ranges
    with pytest.raises(b.BaspError):
        b.basp_stream_copy(x[2048:], x[1:], 1024)     # misaligned source
    b.basp_stream_copy(x[2048:], x, 0)                # zero bytes: nothing to do


def test_plan_shared_by_threads_and_streams():
    """One plan used at the same time by four host threads, each launching
    both directions on its own stream (default priority) on its own buffers;
    every result matches the oracle."""
    needs_gpu()
    import threading
    N, B, S, Hq, Hkv, d = 6, 3, 6 * 37, 12, 6, 40
    plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_INT32, 0)
    i = plan.info
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, "int32")
    o = inputs.tags_int32(i["q_elems"], 7)
    want_s = oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), 0, N, B, S, Hq, Hkv, d)
    want_h = oracle.head_to_seq(bits(o), 0, N, B, S, Hq, d)
    results, errors = {}, []
    torch.cuda.synchronize()

    def worker(t):
        try:
            torch.cuda.set_device(0)
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                qd, kd, vd, od = (x.cuda() for x in (q, k, v, o))
                out = torch.empty(i["qkv_elems"], dtype=torch.int32, device="cuda")
                back = torch.empty(i["q_elems"], dtype=torch.int32, device="cuda")
                for _ in range(20):
                    b.basp_seq_to_head(plan, qd, kd, vd, out)
                    b.basp_head_to_seq(plan, od, back)
            stream.synchronize()
            results[t] = (bits(out), bits(back))
        except Exception as e:   # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(4):
        assert np.array_equal(results[t][0], want_s) and np.array_equal(results[t][1], want_h), t


def test_autotune_in_threads():
    """Two host threads autotune plans of their own at the same time, each on
    its own stream (both small enough for the timing pool and the HIP graphs
    captured on the library's private streams), while a third thread keeps
    launching re-layouts of a third plan on its stream; every result matches
    the oracle."""
    needs_gpu()
    import threading
    cases = [((6, 3, 6 * 37, 12, 6, 40), 1, "int32"), (workloads.TINY[1:], 0, "bf16"),
             ((4, 2, 4 * 29, 8, 4, 64), 1, "int32")]
    want = []
    for (N, B, S, Hq, Hkv, d), m, dt in cases:
        q, k, v = seq_inputs(B, S, Hq, Hkv, d, dt)
        nq = B * S * Hq * d
        o = inputs.tags_int32(nq, 5) if dt == "int32" else inputs.normal_bf16(nq, inputs.SEED_O)
        want.append(((q, k, v, o), oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), m, N, B, S, Hq, Hkv, d),
                     oracle.head_to_seq(bits(o), m, N, B, S, Hq, d)))
    results, errors = {}, []
    torch.cuda.synchronize()

    def worker(t):
        try:
            (N, B, S, Hq, Hkv, d), m, dt = cases[t]
            tdt = torch.int32 if dt == "int32" else torch.bfloat16
            plan = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_INT32 if dt == "int32" else b.BASP_BF16, m)
            i = plan.info
            torch.cuda.set_device(0)
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                qd, kd, vd, od = (x.cuda() for x in want[t][0])
                out = torch.empty(i["qkv_elems"], dtype=tdt, device="cuda")
                back = torch.empty(i["q_elems"], dtype=tdt, device="cuda")
                if t < 2:
                    b.basp_plan_autotune(plan, qd, kd, vd, out, od, back)
                for _ in range(200 if t == 2 else 3):
                    b.basp_seq_to_head(plan, qd, kd, vd, out)
                    b.basp_head_to_seq(plan, od, back)
            stream.synchronize()
            results[t] = (bits(out), bits(back))
        except Exception as e:   # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(3)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(3):
        assert np.array_equal(results[t][0], want[t][1]) and np.array_equal(results[t][1], want[t][2]), t


@pytest.mark.parametrize("seed", range(random_cases.COUNT))
def test_random_shapes_and_tunings(seed):
    """Seeded random plans and launch shapes (odd row sizes, every tuning
    field), both directions, int32 tags and bf16, inside guard bands."""
    needs_gpu()
    shape, mode, layout, tuning = random_cases.case(seed)
    dtype = "int32" if seed % 2 else "bf16"
    print("random case", seed, shape, mode, layout, tuning, flush=True)
    run_s2h(shape, mode, dtype, layout, tuning)
    run_h2s(shape, mode, dtype, layout, tuning)


def _wrapped_tags(n):
    """int32 tensor whose element i holds the low 32 bits of i: distinct for
    n <= 2^32, built on the device in two ranges."""
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    half = min(n, 1 << 31)
    x[:half] = torch.arange(0, half, dtype=torch.int32, device="cuda")
    if n > half:
        x[half:] = torch.arange(-(1 << 31), -(1 << 31) + (n - half), dtype=torch.int32, device="cuda")
    return x


def test_row_index_limit_sampled():
    """Tile bases are 32-bit row indices: a tensor of 2^32 - 4 rows (the most
    a plan allows is 2^32 - 1), moved in both directions, checked on sampled
    destinations (including the last rows) against the oracle's one-element
    source index."""
    needs_gpu()
    N, B, S, H, d = 2, 1, (1 << 31) - 2, 2, 1
    print("row index limit", N, B, S, H, d, flush=True)
    plan = b.basp_plan_create(N, B, S, H, H, d, b.BASP_INT32, 0)
    n = plan.info["q_elems"]
    assert n == (1 << 32) - 4
    x = _wrapped_tags(n)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(11)
    for direction in (0, 1):
        out.fill_(-1)
        if direction == 0:
            b.basp_seq_to_head_o(plan, x, out)
        else:
            b.basp_head_to_seq(plan, x, out)
        torch.cuda.synchronize()
        dst = _sample(n, rng, [n - 1 - i for i in range(64)] + [(1 << 31) + i - 32 for i in range(64)])
        got = out[torch.from_numpy(dst).cuda()].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        want = oracle.source_index(direction, dst, 0, N, B, S, H, d) & 0xFFFFFFFF
        assert np.array_equal(got, want), "direction %d" % direction
    del x, out
    torch.cuda.empty_cache()


def swept_shapes():
    """Every launch shape the table's per-direction sweep can pick (bench.py
    sweep_grid), and the same with 8 vectors per lane, which autotune also
    measures on small calls."""
    import bench
    grid = bench.sweep_grid(2)
    return grid + [dict(t, vectors_per_thread=8) for t in grid if t["vectors_per_thread"] == 4]


@pytest.mark.parametrize("dtype", ["bf16", "int32"])
@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
@pytest.mark.parametrize("mode", ["basp", "ulysses"])
@pytest.mark.parametrize("shape", [(8, 2, 8 * 37, 24, 8, 128), (4, 2, 4 * 203, 8, 4, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_every_swept_launch_shape(shape, mode, layout, dtype):
    """Both directions with each of the 4 032 launch shapes of the sweep
    grid, on ragged shapes (partial token blocks, head counts that tiles of
    4 and 8 heads do not divide, 128- to 512-byte rows), both layouts, bf16
    values and int32 tags: every output element against the oracle, on a
    sentinel-filled output each time."""
    needs_gpu()
    N, B, S, Hq, Hkv, d = shape
    m = MODE[mode]
    code, view = (b.BASP_BF16, torch.int16) if dtype == "bf16" else (b.BASP_INT32, torch.int32)
    plan = b.basp_plan_create_ex(N, B, S, Hq, Hkv, d, code, m, layout)
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, dtype)
    nq = B * S * Hq * d
    o = inputs.normal_bf16(nq, inputs.SEED_O) if dtype == "bf16" else inputs.tags_int32(nq, 7)
    npv = np.int16 if dtype == "bf16" else np.int32
    dev = lambda a: torch.from_numpy(a.view(npv)).cuda()
    want_qkv = dev(oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), m, N, B, S, Hq, Hkv, d, layout))
    want_o = dev(oracle.head_to_seq(bits(o), m, N, B, S, Hq, d, layout))
    q, k, v, o = (t.cuda() for t in (q, k, v, o))
    qkv = torch.empty(want_qkv.numel(), dtype=q.dtype, device="cuda")
    o_out = torch.empty(want_o.numel(), dtype=q.dtype, device="cuda")
    shapes = swept_shapes()
    print("sweep grid", shape, mode, layout, dtype, len(shapes), "shapes", flush=True)
    for t in shapes:
        b.basp_plan_set_tuning(plan, **t)
        qkv.view(view).fill_(-1)
        o_out.view(view).fill_(-1)
        b.basp_seq_to_head(plan, q, k, v, qkv)
        b.basp_head_to_seq(plan, o, o_out)
        assert torch.equal(qkv.view(view), want_qkv), ("seq->head", t)
        assert torch.equal(o_out.view(view), want_o), ("head->seq", t)


@pytest.mark.parametrize("layout", [0, 1], ids=["head_major", "token_major"])
def test_every_swept_launch_shape_general_groups(layout):
    """The 4 032 launch shapes of the sweep grid on a general G-group plan in
    which G, P and Bl all exceed 1 (8 ranks, 4 sequences, 2 groups of 4
    ranks holding 2 sequences each; 37 tokens per rank), both directions:
    every output element against the oracle."""
    needs_gpu()
    N, B, S, Hq, Hkv, d, G = 8, 4, 4 * 37, 8, 4, 64, 2
    m = MODE["groups"]
    plan = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G, layout)
    q, k, v = seq_inputs(B, S, Hq, Hkv, d, "bf16")
    o = inputs.normal_bf16(B * S * Hq * d, inputs.SEED_O)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    want_qkv = dev(oracle.seq_to_head_qkv(bits(q), bits(k), bits(v), m, N, B, S, Hq, Hkv, d, layout, G=G))
    want_o = dev(oracle.head_to_seq(bits(o), m, N, B, S, Hq, d, layout, G=G))
    q, k, v, o = (t.cuda() for t in (q, k, v, o))
    qkv = torch.empty(want_qkv.numel(), dtype=torch.bfloat16, device="cuda")
    o_out = torch.empty(want_o.numel(), dtype=torch.bfloat16, device="cuda")
    shapes = swept_shapes()
    print("sweep grid, general groups", layout, len(shapes), "shapes", flush=True)
    for t in shapes:
        b.basp_plan_set_tuning(plan, **t)
        qkv.view(torch.int16).fill_(-1)
        o_out.view(torch.int16).fill_(-1)
        b.basp_seq_to_head(plan, q, k, v, qkv)
        b.basp_head_to_seq(plan, o, o_out)
        assert torch.equal(qkv.view(torch.int16), want_qkv), ("seq->head", t)
        assert torch.equal(o_out.view(torch.int16), want_o), ("head->seq", t)
