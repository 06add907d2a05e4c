"""Checks that pin the CPU oracle to something other than itself.

Each check raises AssertionError on failure.  They are plain functions so that
``test_oracle_pins.py`` runs them against the oracle and
``test_oracle_mutations.py`` runs them, in a child process, against copies of
the oracle with a mistake planted in them.

What each check compares with (none re-types the oracle's formulas):

* ``check_numpy_layouts``: the two layouts written as NumPy reshapes and
  transposes of the global [B][S][H][d] tensor.  A sequence shard is a block
  of the batch and token axes; a head shard is a block of the batch and head
  axes (the ownership rules of the BASP review page, "Summary" and
  "Frequently asked questions").  NumPy's transpose is the library routine.
* ``check_tagged_brute_force``: shards assembled one rank at a time in pure
  Python from the ownership rules, with unique tags, on tiny shapes.
* ``check_round_trip``: head->seq undoes seq->head and the reverse.
* ``check_b1_is_ulysses``: BASP at B = 1 is Ulysses (the degeneracy of the
  review page, "Strengths", the paper's Fig. 8).
* ``check_groups_special_cases``: the general G-group form (review page,
  "Strengths"; the paper's Sec. IV.C) is Ulysses at G = 1, BASP at G = B and
  the data-parallel fallback at G = N, bit for bit with equal exchange
  matrices.  Its group structure itself is taken from its definition (G
  groups of N/G ranks, B/G sequences each), not from the oracle.
* ``check_k1_local_transpose``: BASP at B = N (K = 1) moves nothing between
  ranks; each rank's result is the textbook transpose [S][H][d] -> [H][S][d].
* ``check_traffic``: observed exchange matrix against the pages' counts:
  peers K-1 (BASP) vs N-1 (Ulysses), BS/N tokens per GPU, per-GPU work of the
  paper's Sec. IV.C, and the cross-rank byte closed form.
* ``check_bijection``: every destination is written once from a distinct
  source.
* ``check_bf16_patterns``: all 65536 bfloat16 bit patterns pass unchanged.
* ``check_source_index_matches_loop``: the oracle's one-element form (for
  sampled checks at large sizes) names the element the full loop copies.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle
from oracle import BASP, GROUPS, HEAD_MAJOR, TOKEN_MAJOR, ULYSSES


def structure(mode, N, B, G=0):
    """(G, P, Bl).  For the two schemes from the oracle (their group rules
    are pinned by check_traffic, check_rejects and the page facts); for the
    general form straight from its definition -- G groups of N/G
    consecutive ranks, each holding B/G sequences -- after checking that the
    oracle agrees."""
    if mode == GROUPS:
        want = (G, N // G, B // G)
        assert oracle.groups(GROUPS, N, B, G) == want, (N, B, G, oracle.groups(GROUPS, N, B, G))
        return want
    return oracle.groups(mode, N, B)


# ---------------------------------------------------------------- layouts ---

def np_seq_layout(X, G, P, Bl):
    """Sequence-sharded buffer of a global [B][S][H][d] array: rank (g, j)
    holds sequences g*Bl.. and tokens j*St.., as [Bl][St][H][d]."""
    B, S, H, d = X.shape
    return X.reshape(G, Bl, P, S // P, H, d).transpose(0, 2, 1, 3, 4, 5).reshape(-1)


def np_head_layout(X, G, P, Bl, layout=HEAD_MAJOR):
    """Head-sharded buffer: rank (g, j) holds sequences g*Bl.. and heads
    j*Hl.., as [Bl][Hl][S][d] (head-major) or [Bl][S][Hl][d] (token-major)."""
    B, S, H, d = X.shape
    Y = X.reshape(G, Bl, S, P, H // P, d)
    axes = (0, 3, 1, 4, 2, 5) if layout == HEAD_MAJOR else (0, 3, 1, 2, 4, 5)
    return Y.transpose(axes).reshape(-1)


def shapes_tiny():
    """Exhaustive grid of tiny valid cases: (mode, N, B, S, H, d, G), G the
    number of groups of the general form (0 for the two schemes)."""
    out = []
    for N in (1, 2, 3, 4, 6, 8):
        for B in (1, 2, 3, 4, 6, 8, 16):
            modes = [(ULYSSES, 0), (BASP, 0)] + [(GROUPS, G) for G in range(1, N + 1)
                                                 if N % G == 0 and B % G == 0]
            for mode, G in modes:
                g = oracle.groups(mode, N, B, G)
                if g is None:
                    continue
                P = g[1]
                for S in sorted({P, 2 * P, 3 * P}):
                    for H in sorted({P, 2 * P}):
                        for d in (1, 3):
                            out.append((mode, N, B, S, H, d, G))
    return out


def _rng_array(shape, rng, dtype=np.uint16):
    return rng.integers(0, np.iinfo(dtype).max, size=shape, dtype=dtype, endpoint=True)


def check_numpy_layouts(cases=None, seed=0):
    rng = np.random.default_rng(seed)
    cases = cases or [
        (ULYSSES, 4, 2, 8, 8, 4), (BASP, 4, 2, 8, 8, 4), (BASP, 8, 2, 16, 8, 2),
        (ULYSSES, 8, 2, 16, 8, 2), (BASP, 8, 4, 8, 6, 3), (ULYSSES, 6, 3, 12, 6, 5),
        (BASP, 6, 3, 12, 4, 2), (BASP, 4, 8, 4, 3, 2), (BASP, 8, 8, 8, 4, 2),
        (ULYSSES, 2, 1, 6, 4, 3), (BASP, 1, 1, 5, 3, 2),
        (GROUPS, 8, 8, 8, 4, 2, 2), (GROUPS, 8, 4, 8, 4, 3, 2), (GROUPS, 6, 4, 6, 3, 2, 2),
        (GROUPS, 12, 6, 12, 8, 2, 3), (GROUPS, 8, 16, 4, 2, 2, 4), (GROUPS, 4, 6, 4, 2, 3, 2),
    ]
    for c in cases:
        mode, N, B, S, H, d = c[:6]
        Gq = c[6] if len(c) > 6 else 0
        G, P, Bl = structure(mode, N, B, Gq)
        for dtype in (np.uint16, np.uint32):
            X = _rng_array((B, S, H, d), rng, dtype)
            seq = np_seq_layout(X, G, P, Bl)
            for layout in (HEAD_MAJOR, TOKEN_MAJOR):
                head = np_head_layout(X, G, P, Bl, layout)
                got = oracle.seq_to_head(seq, mode, N, B, S, H, d, layout, G=Gq)
                assert np.array_equal(got, head), ("s2h", c, layout, dtype)
                back = oracle.head_to_seq(head, mode, N, B, S, H, d, layout, G=Gq)
                assert np.array_equal(back, seq), ("h2s", c, layout, dtype)


# ------------------------------------------------------- tagged brute force --

def _brute_shards(B, S, H, d, G, P, Bl, layout):
    """Pure-Python shards from the ownership rules, element tags
    ((b*S + s)*H + h)*d + e of the global tensor."""
    St, Hl = S // P, H // P
    tag = lambda b, s, h, e: ((b * S + s) * H + h) * d + e
    seq, head = [], []
    for g in range(G):
        for j in range(P):
            mine_b = range(g * Bl, (g + 1) * Bl)
            mine_s = range(j * St, (j + 1) * St)
            mine_h = range(j * Hl, (j + 1) * Hl)
            for b in mine_b:
                for s in mine_s:
                    for h in range(H):
                        for e in range(d):
                            seq.append(tag(b, s, h, e))
            for b in mine_b:
                if layout == HEAD_MAJOR:
                    it = ((h, s) for h in mine_h for s in range(S))
                else:
                    it = ((h, s) for s in range(S) for h in mine_h)
                for h, s in it:
                    for e in range(d):
                        head.append(tag(b, s, h, e))
    return np.array(seq, dtype=np.uint32), np.array(head, dtype=np.uint32)


def check_tagged_brute_force(cases=None):
    for (mode, N, B, S, H, d, Gq) in (cases or shapes_tiny()):
        G, P, Bl = structure(mode, N, B, Gq)
        for layout in (HEAD_MAJOR, TOKEN_MAJOR):
            seq, head = _brute_shards(B, S, H, d, G, P, Bl, layout)
            got = oracle.seq_to_head(seq, mode, N, B, S, H, d, layout, G=Gq)
            assert np.array_equal(got, head), ("s2h", mode, N, B, S, H, d, Gq, layout)
            back = oracle.head_to_seq(head, mode, N, B, S, H, d, layout, G=Gq)
            assert np.array_equal(back, seq), ("h2s", mode, N, B, S, H, d, Gq, layout)


# ------------------------------------------------------------- invariants ---

def check_round_trip(seed=1):
    rng = np.random.default_rng(seed)
    for c in [(BASP, 8, 2, 32, 8, 4), (ULYSSES, 8, 2, 32, 8, 4),
                                  (BASP, 6, 2, 18, 9, 3), (BASP, 4, 8, 4, 2, 2),
                                  (ULYSSES, 3, 5, 9, 6, 2), (GROUPS, 8, 8, 16, 4, 3, 2),
                                  (GROUPS, 6, 4, 12, 6, 2, 2)]:
        mode, N, B, S, H, d = c[:6]
        x = _rng_array(B * S * H * d, rng)
        G = c[6] if len(c) > 6 else 0
        for layout in (HEAD_MAJOR, TOKEN_MAJOR):
            y = oracle.seq_to_head(x, mode, N, B, S, H, d, layout, G=G)
            assert np.array_equal(oracle.head_to_seq(y, mode, N, B, S, H, d, layout, G=G), x)
            z = oracle.head_to_seq(x, mode, N, B, S, H, d, layout, G=G)
            assert np.array_equal(oracle.seq_to_head(z, mode, N, B, S, H, d, layout, G=G), x)


def check_b1_is_ulysses(seed=2):
    rng = np.random.default_rng(seed)
    for (N, S, H, d) in [(8, 16, 8, 4), (4, 12, 4, 3), (2, 2, 2, 1)]:
        x = _rng_array(S * H * d, rng)
        for layout in (HEAD_MAJOR, TOKEN_MAJOR):
            a, ta = oracle.seq_to_head(x, BASP, N, 1, S, H, d, layout, traffic=True)
            b, tb = oracle.seq_to_head(x, ULYSSES, N, 1, S, H, d, layout, traffic=True)
            assert np.array_equal(a, b) and np.array_equal(ta, tb)
            assert np.array_equal(oracle.head_to_seq(x, BASP, N, 1, S, H, d, layout),
                                  oracle.head_to_seq(x, ULYSSES, N, 1, S, H, d, layout))


def check_k1_local_transpose(seed=3):
    """BASP with B = N: every rank transposes its own [S][H][d] sequence."""
    rng = np.random.default_rng(seed)
    for (N, S, H, d) in [(8, 8, 4, 2), (4, 6, 3, 5), (2, 3, 2, 1)]:
        B = N
        x = _rng_array((N, S, H, d), rng)
        y, tm = oracle.seq_to_head(x, BASP, N, B, S, H, d, traffic=True)
        assert np.array_equal(y.reshape(N, H, S, d), x.transpose(0, 2, 1, 3))
        assert np.count_nonzero(tm - np.diag(np.diag(tm))) == 0
        yt = oracle.seq_to_head(x, BASP, N, B, S, H, d, TOKEN_MAJOR)
        assert np.array_equal(yt.reshape(x.shape), x)  # token-major K=1 is the identity


def check_traffic():
    """Exchange matrix observed by the oracle against the pages' counts."""
    for c in [(BASP, 8, 2, 16, 8, 2), (ULYSSES, 8, 2, 16, 8, 2),
              (BASP, 8, 4, 8, 4, 3), (BASP, 8, 8, 8, 4, 1),
              (ULYSSES, 4, 2, 8, 4, 2), (BASP, 6, 2, 6, 3, 2),
              (BASP, 4, 8, 4, 2, 2), (GROUPS, 8, 8, 16, 8, 2, 2), (GROUPS, 8, 8, 16, 8, 1, 4),
              (GROUPS, 6, 4, 12, 6, 2, 2), (GROUPS, 8, 16, 4, 2, 1, 4)]:
        mode, N, B, S, H, d = c[:6]
        Gq = c[6] if len(c) > 6 else 0
        G, P, Bl = structure(mode, N, B, Gq)
        x = np.zeros(B * S * H * d, dtype=np.uint16)
        for fn in (oracle.seq_to_head, oracle.head_to_seq):
            _, tm = fn(x, mode, N, B, S, H, d, traffic=True, G=Gq)
            for r in range(N):
                peers = [i for i in range(N) if i != r and tm[i, r] > 0]
                # peers K-1 (BASP) vs N-1 (Ulysses): the group size minus one;
                # G groups of N/G ranks: N/G - 1
                if mode == GROUPS:
                    expect_peers = N // Gq - 1
                else:
                    expect_peers = (N // B - 1) if (mode == BASP and B <= N) else (
                        0 if mode == BASP else N - 1)
                assert len(peers) == expect_peers, (mode, N, B, r, peers)
                # all peers lie in r's group of contiguous ranks
                assert all(i // P == r // P for i in peers)
                # each GPU keeps B*S/N tokens (sent = its sequence shard)
                sent_tokens = tm[r, :].sum() // (H * d)
                assert sent_tokens * N == B * S, (sent_tokens, B, S, N)
                # per-GPU work (B/G) * H * (S*G/N) * d = B*H*S*d/N elements
                assert tm[:, r].sum() * N == B * H * S * d
                # each peer sends Bl*St*Hl*d elements
                for i in peers:
                    assert tm[i, r] * P * P == Bl * S * H * d
            cross = tm.sum() - np.trace(tm)
            assert cross * P == (P - 1) * B * S * H * d  # (P-1)/P of the tensor


def check_bijection(seed=4):
    rng = np.random.default_rng(seed)
    for (mode, N, B, S, H, d, G) in [(BASP, 8, 2, 16, 8, 3, 0), (ULYSSES, 8, 2, 16, 8, 3, 0),
                                     (BASP, 4, 8, 8, 4, 2, 0), (GROUPS, 8, 4, 8, 4, 3, 2)]:
        n = B * S * H * d
        x = rng.permutation(n).astype(np.uint32)
        for fn in (oracle.seq_to_head, oracle.head_to_seq):
            for layout in (HEAD_MAJOR, TOKEN_MAJOR):
                y = fn(x, mode, N, B, S, H, d, layout, G=G)
                assert np.array_equal(np.sort(y), np.arange(n, dtype=np.uint32))


def check_bf16_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(5)
    pats = rng.permutation(pats)
    for (mode, N, B, S, H, d) in [(BASP, 4, 2, 16, 16, 128), (ULYSSES, 4, 2, 16, 16, 128)]:
        y = oracle.seq_to_head(pats, mode, N, B, S, H, d)
        assert np.array_equal(np.sort(y), np.arange(65536, dtype=np.uint32).astype(np.uint16))
        assert np.array_equal(oracle.head_to_seq(y, mode, N, B, S, H, d), pats)


def check_rejects():
    """The pages' conditions: N = K*B, heads (and tokens) split evenly."""
    assert oracle.groups(BASP, 8, 3) is None          # N not a multiple of B
    assert oracle.groups(BASP, 8, 12) is None         # B > N, not whole sequences
    assert oracle.groups(BASP, 8, 16) == (8, 1, 2)    # data-parallel fallback
    # the general form needs G to divide both the ranks and the sequences
    assert oracle.groups(GROUPS, 8, 8, 3) is None     # N % G
    assert oracle.groups(GROUPS, 8, 6, 4) is None     # B % G
    assert oracle.groups(GROUPS, 8, 8, 0) is None
    assert oracle.groups(GROUPS, 8, 8, 16) is None    # more groups than ranks
    x = np.zeros(2 * 8 * 6 * 2, dtype=np.uint16)
    for args in [(BASP, 8, 2, 8, 6, 2),   # 6 heads over K = 4 members
                 (ULYSSES, 8, 2, 8, 6, 2)]:
        try:
            oracle.seq_to_head(x, *args)
        except ValueError:
            pass
        else:
            raise AssertionError("oracle accepted indivisible heads %r" % (args,))


def check_source_index_matches_loop(seed=6):
    """The one-element form names, for every destination, the element the
    full loop copies there (tags make the source readable from the output)."""
    rng = np.random.default_rng(seed)
    for (mode, N, B, S, H, d, G) in [(BASP, 8, 2, 16, 8, 3, 0), (ULYSSES, 6, 3, 12, 6, 2, 0),
                                     (BASP, 4, 8, 4, 2, 5, 0), (GROUPS, 8, 8, 8, 4, 3, 2),
                                     (GROUPS, 6, 4, 6, 3, 2, 2)]:
        n = B * S * H * d
        tags = np.arange(n, dtype=np.uint32)
        dst = rng.integers(0, n, size=500)
        for layout in (HEAD_MAJOR, TOKEN_MAJOR):
            for direction, fn in ((0, oracle.seq_to_head), (1, oracle.head_to_seq)):
                out = fn(tags, mode, N, B, S, H, d, layout, G=G)
                src = oracle.source_index(direction, dst, mode, N, B, S, H, d, layout, G=G)
                assert np.array_equal(out[dst], src.astype(np.uint32)), (mode, layout, direction)


def check_groups_special_cases(seed=7):
    """G = 1 is Ulysses, G = B (B <= N) is BASP, G = N (B > N) is the
    data-parallel fallback: equal outputs and equal exchange matrices, both
    directions and layouts."""
    rng = np.random.default_rng(seed)
    for (N, B, S, H, d) in [(8, 2, 16, 8, 2), (8, 8, 8, 8, 3), (6, 3, 12, 6, 2), (4, 8, 4, 4, 2),
                            (8, 4, 16, 8, 1), (2, 6, 6, 2, 3)]:
        x = _rng_array(B * S * H * d, rng)
        pairs = [(1, ULYSSES)]
        if B <= N and N % B == 0:
            pairs.append((B, BASP))
        if B > N and B % N == 0:
            pairs.append((N, BASP))
        for G, mode in pairs:
            for layout in (HEAD_MAJOR, TOKEN_MAJOR):
                for fn in (oracle.seq_to_head, oracle.head_to_seq):
                    a, ta = fn(x, GROUPS, N, B, S, H, d, layout, traffic=True, G=G)
                    b, tb = fn(x, mode, N, B, S, H, d, layout, traffic=True)
                    assert np.array_equal(a, b) and np.array_equal(ta, tb), (N, B, G, mode, layout)


ALL_CHECKS = [check_numpy_layouts, check_tagged_brute_force, check_round_trip,
              check_b1_is_ulysses, check_groups_special_cases, check_k1_local_transpose, check_traffic,
              check_bijection, check_bf16_patterns, check_rejects, check_source_index_matches_loop]


def run_all():
    for fn in ALL_CHECKS:
        fn()


if __name__ == "__main__":
    import sys
    names = sys.argv[1:]
    fns = [f for f in ALL_CHECKS if not names or f.__name__ in names]
    for f in fns:
        f()
    print("ok", len(fns))
