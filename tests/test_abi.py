"""The C ABI on the host (no GPU): the library loads and exports every entry
point of include/basp.h; plan creation, validation and the plan query; the
pre-launch pointer checks.  No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from sequence_re_layout_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "basp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(basp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "basp_seq_to_head" in names and "basp_head_to_seq" in names and "basp_plan_create" in names
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(b.library(), n)
        assert hasattr(b, n), "binding lacks %s" % n


MODES = {"ulysses": b.BASP_MODE_ULYSSES, "basp": b.BASP_MODE_BASP}
SHAPES = [  # N, B, S, Hq, Hkv, d
    (4, 2, 1024, 8, 8, 64), (8, 2, 16384, 32, 8, 64), (8, 2, 16384, 16, 16, 128),
    (8, 1, 8192, 32, 8, 64), (8, 4, 8192, 32, 8, 64), (8, 8, 8192, 32, 8, 64),
    (8, 2, 1024, 24, 8, 128), (8, 2, 32768, 24, 8, 128), (8, 2, 16384, 32, 8, 128),
]


@pytest.mark.parametrize("mode", ["ulysses", "basp"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_plan_info_matches_oracle(mode, shape):
    N, B, S, Hq, Hkv, d = shape
    m = MODES[mode]
    info = b.basp_plan_create(N, B, S, Hq, Hkv, d, b.BASP_BF16, m).info
    G, P, Bl = oracle.groups(m, N, B)
    assert (info["G"], info["P"], info["Bl"]) == (G, P, Bl)
    assert info["St"] == S // P and info["Hl_q"] == Hq // P and info["Hl_kv"] == Hkv // P
    assert info["tokens_per_rank"] * N == B * S
    assert info["q_elems"] == B * S * Hq * d and info["kv_elems"] == B * S * Hkv * d
    assert info["qkv_offset_k"] == info["q_elems"]
    assert info["qkv_offset_v"] == info["q_elems"] + info["kv_elems"]
    assert info["qkv_bytes_moved"] == 2 * 2 * B * S * (Hq + 2 * Hkv) * d
    assert info["o_bytes_moved"] == 2 * 2 * B * S * Hq * d
    # counts observed by the oracle on a scaled-down copy (S/P tokens -> 1 token per
    # member; traffic scales linearly in tokens and channels)
    for H, key in ((Hq, "q"), (Hkv, "kv")):
        x = np.zeros(B * P * H, dtype=np.uint16)
        _, tm = oracle.seq_to_head(x, m, N, B, P, H, 1, traffic=True)
        scale = (S // P) * d * 2
        for r in range(N):
            peers = [i for i in range(N) if i != r and tm[i, r]]
            assert len(peers) == info["peers_per_rank"]
            for i in peers:
                assert tm[i, r] * scale == info["per_peer_bytes_" + key]
        assert (tm.sum() - np.trace(tm)) * scale == info["cross_rank_bytes_" + key]


def test_b1_plans_equal_and_k1_has_no_peers():
    a = b.basp_plan_create(8, 1, 8192, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP).info
    u = b.basp_plan_create(8, 1, 8192, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_ULYSSES).info
    skip = {"mode"}
    assert {k: v for k, v in a.items() if k not in skip} == {k: v for k, v in u.items() if k not in skip}
    k1 = b.basp_plan_create(8, 8, 8192, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP).info
    assert k1["P"] == 1 and k1["peers_per_rank"] == 0 and k1["cross_rank_bytes_q"] == 0


def _create_status(*args):
    h = b.library().basp_plan_create(*args)
    st = b.basp_last_error()
    if h:
        b.library().basp_plan_destroy(h)
    return st


@pytest.mark.parametrize("args,status", [
    ((0, 1, 8, 8, 8, 8, 0, 1), b.BASP_ERR_INVALID),
    ((8, 0, 8, 8, 8, 8, 0, 1), b.BASP_ERR_INVALID),
    ((8, 2, -1, 8, 8, 8, 0, 1), b.BASP_ERR_INVALID),
    ((8, 2, 8, 0, 8, 8, 0, 1), b.BASP_ERR_INVALID),
    ((8, 2, 8, 8, 8, 0, 0, 1), b.BASP_ERR_INVALID),
    ((8, 2, 8, 8, 8, 8, 7, 1), b.BASP_ERR_INVALID),
    ((8, 2, 8, 8, 8, 8, 0, 5), b.BASP_ERR_INVALID),
    ((8, 3, 24, 24, 24, 8, 0, 1), b.BASP_ERR_INDIVISIBLE),   # N % B
    ((8, 12, 24, 24, 24, 8, 0, 1), b.BASP_ERR_INDIVISIBLE),  # B > N, B % N
    ((8, 2, 6, 8, 8, 8, 0, 1), b.BASP_ERR_INDIVISIBLE),      # S % K
    ((8, 2, 8, 6, 8, 8, 0, 1), b.BASP_ERR_INDIVISIBLE),      # Hq % K
    ((8, 2, 8, 8, 2, 8, 0, 1), b.BASP_ERR_INDIVISIBLE),      # Hkv % K (GQA, no replication)
    ((8, 2, 8, 8, 4, 8, 0, 0), b.BASP_ERR_INDIVISIBLE),      # Ulysses Hkv % N
    ((8, 2, 1 << 60, 8, 8, 8, 0, 1), b.BASP_ERR_UNSUPPORTED),
    ((8, 2, 8, 8, 8, 8, 0, 1), b.BASP_OK),
    ((8, 16, 8, 8, 8, 8, 0, 1), b.BASP_OK),                  # data-parallel fallback
    ((8, 2, 0, 8, 8, 8, 0, 1), b.BASP_OK),                   # empty
])
def test_plan_create_status(args, status):
    assert _create_status(*args) == status


def test_status_strings_and_null_plan():
    for s in range(7):
        assert b.basp_status_str(s).startswith("BASP_")
    lib = b.library()
    assert lib.basp_plan_query(None, None) == b.BASP_ERR_INVALID
    assert lib.basp_seq_to_head(None, None, None, None, None, None) == b.BASP_ERR_INVALID
    assert b.basp_last_error() == b.BASP_ERR_INVALID
    assert lib.basp_unfused_workspace_bytes(None) == 0
    lib.basp_plan_destroy(None)


def test_tuning_validation():
    p = b.basp_plan_create(8, 2, 16384, 32, 8, 64)
    b.basp_plan_set_tuning(p, vectors_per_thread=8, tile_tokens=64, tile_heads=2, cache_policy=3)
    assert b.basp_plan_get_tuning(p, b.BASP_SEQ_TO_HEAD)["tile_heads"] == 2
    assert b.basp_plan_get_tuning(p, b.BASP_HEAD_TO_SEQ)["tile_heads"] == 2
    b.basp_plan_set_direction_tuning(p, b.BASP_HEAD_TO_SEQ, tile_heads=8, tile_order=2)
    assert b.basp_plan_get_tuning(p, b.BASP_SEQ_TO_HEAD)["tile_heads"] == 2
    assert b.basp_plan_get_tuning(p, b.BASP_HEAD_TO_SEQ)["tile_order"] == 2
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_set_direction_tuning(p, 2, tile_heads=1)
    assert e.value.status == b.BASP_ERR_INVALID
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_set_tuning(p, tile_order=4)
    assert e.value.status == b.BASP_ERR_INVALID
    with pytest.raises(TypeError):
        b.basp_plan_set_tuning(p, tile_size=3)
    for bad in (dict(vectors_per_thread=3), dict(cache_policy=6), dict(tile_tokens=-1), dict(block_size=96),
                dict(batch_order=3)):
        with pytest.raises(b.BaspError) as e:
            b.basp_plan_set_tuning(p, **bad)
        assert e.value.status == b.BASP_ERR_INVALID
    # a 1-token x 1-head tile over a huge sequence exceeds the tile index range
    big = b.basp_plan_create(1, 1, 1 << 28, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_ULYSSES)
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_set_tuning(big, tile_tokens=1, tile_heads=1)
    assert e.value.status == b.BASP_ERR_UNSUPPORTED


def test_pointer_checks_before_launch():
    """Rejected before any device call: NULL, misaligned and overlapping pointers."""
    lib = b.library()
    p = b.basp_plan_create(4, 2, 64, 8, 8, 64)
    i = p.info
    qb, kb = i["q_elems"] * 2, i["kv_elems"] * 2
    base = 1 << 40  # fake addresses: never dereferenced
    q, k, v, out = base, base + qb, base + qb + kb, base + 4 * qb
    assert lib.basp_seq_to_head(p.handle, None, k, v, out, None) == b.BASP_ERR_INVALID
    assert lib.basp_seq_to_head(p.handle, q + 1, k, v, out, None) == b.BASP_ERR_ALIGN
    assert lib.basp_seq_to_head(p.handle, q, k, v, q + 64, None) == b.BASP_ERR_ALIAS
    assert lib.basp_seq_to_head(p.handle, q, k, v, v + kb - 2, None) == b.BASP_ERR_ALIAS
    assert lib.basp_head_to_seq(p.handle, q, q + qb - 2, None) == b.BASP_ERR_ALIAS
    assert lib.basp_head_to_seq_qkv(p.handle, q, out, out + qb - 2, out + 2 * qb, None) == b.BASP_ERR_ALIAS
    ws = out + 4 * qb
    assert lib.basp_seq_to_head_unfused(p.handle, q, k, v, out, out + 8, None) == b.BASP_ERR_ALIAS
    assert lib.basp_seq_to_head_unfused(p.handle, q, k, v, out, ws + 1, None) == b.BASP_ERR_ALIGN
    # autotune checks both calls' buffers before touching the device
    assert lib.basp_plan_autotune(p.handle, q, k, v, q + 64, q, out, None) == b.BASP_ERR_ALIAS
    assert lib.basp_plan_autotune(p.handle, q, k, v, out, q + 1, ws, None) == b.BASP_ERR_ALIGN
    assert lib.basp_plan_autotune(None, q, k, v, out, q, ws, None) == b.BASP_ERR_INVALID
    # the two calls run back to back, so each output is also checked against
    # the other call's buffers: o_out over q, qkv over o, o_out over qkv
    o = ws + 8 * qb
    assert lib.basp_plan_autotune(p.handle, q, k, v, out, o, q, None) == b.BASP_ERR_ALIAS
    assert lib.basp_plan_autotune(p.handle, q, k, v, out, out + 64, ws, None) == b.BASP_ERR_ALIAS
    assert lib.basp_plan_autotune(p.handle, q, k, v, out, o, out + 2 * qb, None) == b.BASP_ERR_ALIAS
    # q, k and v may alias each other (inputs only)
    e = b.basp_plan_create(4, 2, 0, 8, 8, 64)
    assert lib.basp_seq_to_head(e.handle, None, None, None, None, None) == b.BASP_OK
    assert lib.basp_head_to_seq(e.handle, None, None, None) == b.BASP_OK


def test_stream_copy_checks_before_launch():
    """The copy rejects NULL, misaligned, overlapping and oversized arguments
    before any device call; zero bytes is a no-op."""
    lib = b.library()
    base = 1 << 40  # fake addresses: never dereferenced
    n = 1 << 20
    assert lib.basp_stream_copy(None, None, 0, None) == b.BASP_OK
    assert lib.basp_stream_copy(None, base, n, None) == b.BASP_ERR_INVALID
    assert lib.basp_stream_copy(base + n, None, n, None) == b.BASP_ERR_INVALID
    assert lib.basp_stream_copy(base + n, base + 8, n, None) == b.BASP_ERR_ALIGN
    assert lib.basp_stream_copy(base + n + 4, base, n, None) == b.BASP_ERR_ALIGN
    assert lib.basp_stream_copy(base + n, base, n + 2, None) == b.BASP_ERR_ALIGN
    assert lib.basp_stream_copy(base + n - 16, base, n, None) == b.BASP_ERR_ALIAS
    assert lib.basp_stream_copy(base, base + n - 16, n, None) == b.BASP_ERR_ALIAS
    assert lib.basp_stream_copy(base, base, n, None) == b.BASP_ERR_ALIAS
    assert lib.basp_stream_copy(base, base + (1 << 58), (1 << 56) + 16, None) == b.BASP_ERR_UNSUPPORTED
    assert b.basp_last_error() == b.BASP_ERR_UNSUPPORTED


def test_binding_copy_needs_a_byte_count_for_raw_addresses():
    """With raw addresses the binding cannot infer the size: it raises
    before calling the library."""
    base = 1 << 40
    with pytest.raises(ValueError, match="nbytes"):
        b.basp_stream_copy(base + (1 << 20), base)


def test_row_count_limit():
    """Tile bases are 32-bit row indices: a tensor of 2^32 or more rows
    (B*S*max(Hq, Hkv)) is rejected at plan creation, 2^32 - 8 is not."""
    ok = b.basp_plan_create(1, 1, (1 << 29) - 1, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_ULYSSES)
    assert ok.info["q_elems"] == ((1 << 32) - 8) * 8
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_create(1, 1, 1 << 29, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_ULYSSES)
    assert e.value.status == b.BASP_ERR_UNSUPPORTED
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_create(4, 1, 1 << 30, 4, 4, 8, b.BASP_BF16, b.BASP_MODE_ULYSSES)   # 2^32 rows
    assert e.value.status == b.BASP_ERR_UNSUPPORTED
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_create(2, 2, 1 << 29, 4, 8, 8, b.BASP_BF16, b.BASP_MODE_BASP)   # Hkv > Hq
    assert e.value.status == b.BASP_ERR_UNSUPPORTED


def test_batch_fits_the_launch_grid():
    """The batch index is the launch grid's z coordinate: B above 65535 is
    rejected (here in the data-parallel fallback, N = 1), 65535 is not.  The
    group size, the y coordinate, is bounded by the row limit (H >= P and
    S >= P give P*P rows at least)."""
    ok = b.basp_plan_create(1, 65535, 1, 1, 1, 8, b.BASP_BF16, b.BASP_MODE_BASP)
    assert (ok.info["G"], ok.info["P"], ok.info["Bl"]) == (1, 1, 65535)
    with pytest.raises(b.BaspError) as e:
        b.basp_plan_create(1, 65536, 1, 1, 1, 8, b.BASP_BF16, b.BASP_MODE_BASP)
    assert e.value.status == b.BASP_ERR_UNSUPPORTED


def test_foil_tokens():
    """tokens_per_rank_foil is the token count per rank of Ulysses run over
    groups of N/B ranks that each hold the whole micro-batch: the page's
    value at its own setting, and the count the oracle observes for that
    configuration on other shapes."""
    import json
    facts = {f["id"]: f for f in json.load(open(os.path.join(ROOT, "tests", "golden", "page_facts.json")))["facts"]}
    f = facts["foil_tokens"]
    for m in MODES.values():
        info = b.basp_plan_create(f["N"], f["B"], f["S"], 32, 8, 64, b.BASP_BF16, m).info
        assert info["tokens_per_rank_foil"] == f["tokens_per_gpu_foil"]
        assert info["tokens_per_rank"] == f["tokens_per_gpu_basp"]
    for (N, B, S) in [(8, 4, 64), (8, 8, 16), (6, 3, 12), (4, 1, 8), (8, 2, 32)]:
        K = N // B
        x = np.zeros(B * S * K, dtype=np.uint16)
        _, tm = oracle.seq_to_head(x, oracle.ULYSSES, K, B, S, K, 1, traffic=True)
        observed = set(int(tm[r, :].sum()) // K for r in range(K))
        info = b.basp_plan_create(N, B, S, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_BASP).info
        assert observed == {info["tokens_per_rank_foil"]}, (N, B, S)
    # no foil where N/B is not whole: Ulysses with N % B != 0, or B > N
    assert b.basp_plan_create(8, 3, 24, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_ULYSSES).info["tokens_per_rank_foil"] == 0
    assert b.basp_plan_create(8, 16, 8, 8, 8, 8, b.BASP_BF16, b.BASP_MODE_BASP).info["tokens_per_rank_foil"] == 0


def test_noalloc_limit_checked_before_any_device_call():
    """The allocation-free entry point rejects a NULL plan and a plan whose
    workspace exceeds the library's array before touching the device (fake
    addresses, never dereferenced); an empty plan needs no device at all."""
    lib = b.library()
    base = 1 << 40
    assert lib.basp_seq_to_head_unfused_noalloc(None, base, base, base, base + (1 << 30), None) == b.BASP_ERR_INVALID
    fits = b.basp_plan_create(8, 2, 4096, 16, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP)
    assert b.basp_unfused_workspace_bytes(fits) == b.BASP_NOALLOC_SCRATCH_BYTES
    over = b.basp_plan_create(8, 2, 4104, 16, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP)
    assert lib.basp_seq_to_head_unfused_noalloc(over.handle, base, base, base, base + (1 << 30), None) \
        == b.BASP_ERR_UNSUPPORTED
    empty = b.basp_plan_create(8, 2, 0, 16, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP)
    assert lib.basp_seq_to_head_unfused_noalloc(empty.handle, None, None, None, None, None) == b.BASP_OK
    header = open(HEADER).read()
    assert "#define BASP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in header
    assert b.BASP_NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.parametrize("args,status", [
    ((8, 8, 64, 8, 8, 8, 0, 0, 0), b.BASP_ERR_INVALID),      # G = 0
    ((8, 8, 64, 8, 8, 8, 0, -2, 0), b.BASP_ERR_INVALID),
    ((8, 8, 64, 8, 8, 8, 0, 2, 3), b.BASP_ERR_INVALID),      # unknown layout
    ((8, 8, 64, 8, 8, 8, 0, 3, 0), b.BASP_ERR_INDIVISIBLE),  # N % G
    ((8, 6, 64, 8, 8, 8, 0, 4, 0), b.BASP_ERR_INDIVISIBLE),  # B % G
    ((8, 8, 6, 8, 8, 8, 0, 2, 0), b.BASP_ERR_INDIVISIBLE),   # S % (N/G)
    ((8, 8, 64, 8, 2, 8, 0, 2, 0), b.BASP_ERR_INDIVISIBLE),  # Hkv % (N/G)
    ((8, 8, 64, 8, 8, 8, 0, 16, 0), b.BASP_ERR_INDIVISIBLE), # more groups than ranks
    ((8, 8, 64, 8, 8, 8, 0, 2, 1), b.BASP_OK),
    ((8, 16, 64, 8, 8, 8, 0, 8, 0), b.BASP_OK),
])
def test_plan_create_groups_status(args, status):
    h = b.library().basp_plan_create_groups(*args)
    st = b.basp_last_error()
    if h:
        b.library().basp_plan_destroy(h)
    assert st == status


GROUP_SHAPES = [  # (N, B, S, Hq, Hkv, d), G
    ((8, 8, 8192, 32, 8, 64), 1), ((8, 8, 8192, 32, 8, 64), 2), ((8, 8, 8192, 32, 8, 64), 4),
    ((8, 8, 8192, 32, 8, 64), 8), ((6, 4, 600, 6, 3, 40), 2), ((12, 6, 36, 12, 4, 24), 3),
    ((8, 16, 8192, 32, 8, 64), 4),
]


@pytest.mark.parametrize("shape,G", GROUP_SHAPES, ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else "G%d" % x)
def test_groups_plan_info_matches_oracle(shape, G):
    """The general form's plan info against the pages' counts and the
    oracle's observed exchange matrix (scaled down in S and d, where every
    count is linear)."""
    N, B, S, Hq, Hkv, d = shape
    info = b.basp_plan_create_groups(N, B, S, Hq, Hkv, d, b.BASP_BF16, G).info
    P = N // G
    assert info["mode"] == b.BASP_MODE_GROUPS
    assert (info["G"], info["P"], info["Bl"]) == oracle.groups(oracle.GROUPS, N, B, G) == (G, P, B // G)
    assert info["tokens_per_rank"] * N == B * S
    assert info["peers_per_rank"] == P - 1
    assert info["q_elems_per_rank"] * N == B * Hq * S * d
    for H, key in ((Hq, "q"), (Hkv, "kv")):
        x = np.zeros(B * P * H, dtype=np.uint16)
        _, tm = oracle.seq_to_head(x, oracle.GROUPS, N, B, P, H, 1, traffic=True, G=G)
        scale = (S // P) * d * 2
        for r in range(N):
            peers = [i for i in range(N) if i != r and tm[i, r]]
            assert len(peers) == info["peers_per_rank"]
            for i in peers:
                assert tm[i, r] * scale == info["per_peer_bytes_" + key]
        assert (tm.sum() - np.trace(tm)) * scale == info["cross_rank_bytes_" + key]


def test_groups_special_cases_match_the_two_schemes():
    """G = 1 gives Ulysses' plan, G = B BASP's, G = N the data-parallel
    fallback's: every info field but the mode."""
    def same(a, c):
        skip = {"mode"}
        return {k: v for k, v in a.items() if k not in skip} == {k: v for k, v in c.items() if k not in skip}
    g1 = b.basp_plan_create_groups(8, 2, 16384, 32, 8, 64, b.BASP_BF16, 1).info
    assert same(g1, b.basp_plan_create(8, 2, 16384, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_ULYSSES).info)
    gb = b.basp_plan_create_groups(8, 2, 16384, 32, 8, 64, b.BASP_BF16, 2).info
    assert same(gb, b.basp_plan_create(8, 2, 16384, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP).info)
    gn = b.basp_plan_create_groups(8, 16, 8192, 32, 8, 64, b.BASP_BF16, 8).info
    assert same(gn, b.basp_plan_create(8, 16, 8192, 32, 8, 64, b.BASP_BF16, b.BASP_MODE_BASP).info)
    # create / create_ex do not take the general mode (it needs G)
    assert not b.library().basp_plan_create(8, 8, 64, 8, 8, 8, 0, b.BASP_MODE_GROUPS)
    assert b.basp_last_error() == b.BASP_ERR_INVALID


def test_autograd_module_imports_without_a_gpu():
    """The autograd wrappers load with the binding (no device needed to
    import) and only call the library's entry points."""
    from sequence_re_layout_amd import autograd
    assert callable(autograd.seq_to_head_qkv) and callable(autograd.head_to_seq_o)
    src = open(autograd.__file__).read()
    assert "oracle" not in src
