"""The CPU oracle against its pins (no GPU).  See ``oracle_pins.py`` for what
each check compares with."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import BASP, ULYSSES
from tests import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def _observed(mode, N, B, S, H=None, d=1):
    """Peers and tokens per GPU as the oracle's exchange matrix shows them."""
    G, P, Bl = oracle.groups(mode, N, B)
    H = H or P
    x = np.zeros(B * S * H * d, dtype=np.uint16)
    _, tm = oracle.seq_to_head(x, mode, N, B, S, H, d, traffic=True)
    peers = {r: sum(1 for i in range(N) if i != r and tm[i, r]) for r in range(N)}
    tokens = {r: int(tm[r, :].sum() // (H * d)) for r in range(N)}
    return peers, tokens, tm


def test_page_facts():
    facts = {f["id"]: f for f in json.load(open(GOLDEN))["facts"]}

    f = facts["peers_n8_b2"]
    pb, _, _ = _observed(BASP, f["N"], f["B"], S=f["K"])
    pu, _, _ = _observed(ULYSSES, f["N"], f["B"], S=f["N"])
    assert set(pb.values()) == {f["peers_basp"]}
    assert set(pu.values()) == {f["peers_ulysses"]}
    assert oracle.groups(BASP, f["N"], f["B"])[1] == f["K"]

    f = facts["tokens_per_gpu_16k"]
    # the token count does not depend on H or d; a reduced head count keeps it quick
    for mode in (BASP, ULYSSES):
        _, tok, _ = _observed(mode, f["N"], f["B"], f["S"], H=8, d=1)
        assert set(tok.values()) == {f["tokens_per_gpu"]}

    f = facts["batch_sweep_groups"]
    for c in f["cases"]:
        assert oracle.groups(BASP, f["N"], c["B"])[1] == c["K"]
        pb, _, _ = _observed(BASP, f["N"], c["B"], S=8, H=8)
        assert set(pb.values()) == {c["peers_basp"]}

    f = facts["b1_degenerates"]
    pb, _, tb = _observed(BASP, f["N"], f["B"], S=8)
    pu, _, tu = _observed(ULYSSES, f["N"], f["B"], S=8)
    assert set(pb.values()) == {f["peers_basp"]} and set(pu.values()) == {f["peers_ulysses"]}
    assert np.array_equal(tb, tu)

    f = facts["foil_tokens"]
    # the foil is Ulysses over a group of N/B GPUs holding the whole micro-batch
    K = f["N"] // f["B"]
    _, tok, _ = _observed(ULYSSES, K, f["B"], f["S"], H=K, d=1)
    assert set(tok.values()) == {f["tokens_per_gpu_foil"]}
    _, tok, _ = _observed(BASP, f["N"], f["B"], f["S"], H=8, d=1)
    assert set(tok.values()) == {f["tokens_per_gpu_basp"]}

    f = facts["work_equality"]
    for G in f["G_values"]:
        mode = ULYSSES if G == 1 else BASP
        assert oracle.groups(mode, f["P_total"], f["B"])[0] == G
        # received elements per GPU, scaled down in S (linear in S) to stay quick
        scale = 64
        _, _, tm = _observed(mode, f["P_total"], f["B"], f["S"] // scale, H=f["H"], d=f["d"])
        assert set(int(v) * scale for v in tm.sum(axis=0)) == {f["elements_per_gpu"]}

    f = facts["work_equality_general_G"]
    scale = 64   # received elements are linear in S: a shorter sequence keeps it quick
    for G, peers in zip(f["G_values"], f["peers"]):
        assert oracle.groups(oracle.GROUPS, f["N"], f["B"], G) == (G, f["N"] // G, f["B"] // G)
        x = np.zeros(f["B"] * (f["S"] // scale) * f["H"] * f["d"], dtype=np.uint16)
        _, tm = oracle.seq_to_head(x, oracle.GROUPS, f["N"], f["B"], f["S"] // scale, f["H"], f["d"],
                                   traffic=True, G=G)
        assert set(int(v) * scale for v in tm.sum(axis=0)) == {f["elements_per_gpu"]}
        assert {sum(1 for i in range(f["N"]) if i != r and tm[i, r]) for r in range(f["N"])} == {peers}

    f = facts["needs_n_multiple_of_b"]
    assert (oracle.groups(BASP, f["N"], f["B"]) is not None) == f["valid"]

    f = facts["heads_divide"]
    with pytest.raises(ValueError):
        oracle.seq_to_head(np.zeros(f["B"] * 8 * f["H"], np.uint16), BASP, f["N"], f["B"], 8, f["H"], 1)

    f = facts["dp_fallback"]
    pb, tok, _ = _observed(BASP, f["N"], f["B"], f["S"], H=2, d=1)
    assert set(pb.values()) == {f["peers_basp"]}
    assert set(tok.values()) == {f["tokens_per_gpu_S"]}


@pytest.mark.parametrize("mode", [ULYSSES, BASP], ids=["ulysses", "basp"])
@pytest.mark.parametrize("layout", [oracle.HEAD_MAJOR, oracle.TOKEN_MAJOR], ids=["head_major", "token_major"])
def test_numpy_transpose_forms_match_the_element_loop(mode, layout):
    """The NumPy transpose forms the benchmark times for comparison compute
    the same permutation as the element loop, both directions."""
    rng = np.random.default_rng(7)
    for (N, B, S, H, d) in [(8, 2, 32, 8, 4), (6, 3, 18, 12, 3), (4, 8, 4, 4, 2), (1, 3, 5, 2, 3),
                            (8, 1, 16, 16, 2), (2, 4, 6, 2, 5)]:
        gpb = oracle.groups(mode, N, B)
        if gpb is None or S % gpb[1] or H % gpb[1]:
            continue
        x = rng.integers(0, 1 << 16, size=B * S * H * d, dtype=np.uint16)
        assert np.array_equal(oracle.numpy_seq_to_head(x, mode, N, B, S, H, d, layout),
                              oracle.seq_to_head(x, mode, N, B, S, H, d, layout))
        assert np.array_equal(oracle.numpy_head_to_seq(x, mode, N, B, S, H, d, layout),
                              oracle.head_to_seq(x, mode, N, B, S, H, d, layout))
