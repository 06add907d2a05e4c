"""CPU oracle for the BASP / Ulysses attention-boundary re-layout.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library under ``sequence_re_layout_amd/``, and that library never
imports it.

The arithmetic lives in ``oracle.c`` (a plain element loop over the
destination, written from the pages' definitions; see its header for the
sources and the readings).  This module only marshals NumPy arrays into it and
states the fused layout of the three-tensor calls:

* fused seq->head output = HEAD(Q) || HEAD(K) || HEAD(V), each tensor's
  head-sharded buffer in full, in that order (one output allocation for the
  three tensors; the Q part is then itself a valid head-sharded O).

Arrays are raw bit containers (``uint16`` for 2-byte types, ``uint32`` for
4-byte types); the oracle never interprets values.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

ULYSSES = 0
BASP = 1
GROUPS = 2   # the general form: G groups given explicitly (keyword G)
HEAD_MAJOR = 0
TOKEN_MAJOR = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.orc_groups.argtypes = [i32, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                   ctypes.POINTER(i64)]
        lib.orc_groups.restype = i32
        for fn in (lib.orc_seq_to_head, lib.orc_head_to_seq):
            fn.argtypes = [i32, i64, i32, i64, i64, i64, i64, i64, i64, vp, vp, vp, i32]
            fn.restype = i32
        lib.orc_source_index.argtypes = [i32, i32, i64, i32, i64, i64, i64, i64, i64, vp, vp, i64]
        lib.orc_source_index.restype = i32
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = i32
        _lib = lib
    return _lib


def _use_library(path: str) -> None:
    """Point this module at another build of the oracle (the mutation tests
    load copies with planted mistakes)."""
    global _lib
    _lib = None
    _build.LIB = path
    _load()


def max_threads() -> int:
    """Threads an OpenMP region of the oracle gets by default."""
    return int(_load().orc_max_threads())


def groups(mode: int, N: int, B: int, G: int = 0):
    """(G, P, Bl) of the scheme (G: the number of groups of mode GROUPS), or
    None when the pages' conditions fail."""
    g, P, Bl = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = _load().orc_groups(mode, G, N, B, ctypes.byref(g), ctypes.byref(P), ctypes.byref(Bl))
    if rc != 0:
        return None
    return g.value, P.value, Bl.value


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _run(fn, x, mode, layout, N, B, S, H, d, traffic, threads, G):
    x = np.ascontiguousarray(x).reshape(-1)
    if x.size != B * S * H * d:
        raise ValueError("input holds %d elements, expected B*S*H*d = %d" % (x.size, B * S * H * d))
    out = np.empty_like(x)
    tm = np.zeros((N, N), dtype=np.int64) if traffic else None
    threads = max_threads() if threads is None else threads
    rc = fn(mode, G, layout, N, B, S, H, d, x.itemsize, _ptr(x), _ptr(out),
            _ptr(tm) if traffic else None, threads)
    if rc != 0:
        raise ValueError("oracle rejected mode=%d G=%d layout=%d N=%d B=%d S=%d H=%d d=%d"
                         % (mode, G, layout, N, B, S, H, d))
    return (out, tm) if traffic else out


def seq_to_head(x, mode, N, B, S, H, d, layout=HEAD_MAJOR, traffic=False, threads=None, G=0):
    """One tensor, sequence-sharded -> head-sharded.  With ``traffic`` also
    returns the N x N matrix of elements moved from rank i to rank j.  G is
    the number of groups of mode GROUPS."""
    return _run(_load().orc_seq_to_head, x, mode, layout, N, B, S, H, d, traffic, threads, G)


def head_to_seq(x, mode, N, B, S, H, d, layout=HEAD_MAJOR, traffic=False, threads=None, G=0):
    """One tensor, head-sharded -> sequence-sharded (the inverse exchange)."""
    return _run(_load().orc_head_to_seq, x, mode, layout, N, B, S, H, d, traffic, threads, G)


def source_index(direction, dst, mode, N, B, S, H, d, layout=HEAD_MAJOR, G=0):
    """Source element offsets of the destination element offsets ``dst`` of a
    one-tensor call (direction 0: seq->head, 1: head->seq), one element at a
    time, for sampled checks at sizes the full loop does not reach."""
    dst = np.ascontiguousarray(dst, dtype=np.int64)
    src = np.empty_like(dst)
    rc = _load().orc_source_index(direction, mode, G, layout, N, B, S, H, d, _ptr(dst), _ptr(src), dst.size)
    if rc != 0:
        raise ValueError("oracle rejected the arguments or an offset")
    return src


def seq_to_head_qkv(q, k, v, mode, N, B, S, Hq, Hkv, d, layout=HEAD_MAJOR, threads=None, G=0):
    """Fused Q/K/V seq->head: HEAD(Q) || HEAD(K) || HEAD(V) in one array."""
    parts = [seq_to_head(q, mode, N, B, S, Hq, d, layout, threads=threads, G=G),
             seq_to_head(k, mode, N, B, S, Hkv, d, layout, threads=threads, G=G),
             seq_to_head(v, mode, N, B, S, Hkv, d, layout, threads=threads, G=G)]
    return np.concatenate(parts)


def head_to_seq_qkv(x, mode, N, B, S, Hq, Hkv, d, layout=HEAD_MAJOR, threads=None, G=0):
    """Fused inverse for the gradients dQ/dK/dV: splits HEAD(dQ) || HEAD(dK) ||
    HEAD(dV) and returns the three sequence-sharded arrays."""
    x = np.ascontiguousarray(x).reshape(-1)
    nq, nkv = B * S * Hq * d, B * S * Hkv * d
    if x.size != nq + 2 * nkv:
        raise ValueError("fused input holds %d elements, expected %d" % (x.size, nq + 2 * nkv))
    return (head_to_seq(x[:nq], mode, N, B, S, Hq, d, layout, threads=threads, G=G),
            head_to_seq(x[nq:nq + nkv], mode, N, B, S, Hkv, d, layout, threads=threads, G=G),
            head_to_seq(x[nq + nkv:], mode, N, B, S, Hkv, d, layout, threads=threads, G=G))


# ---------------------------------------------------------------- NumPy ---
# The same two re-layouts as one NumPy transpose each, for the benchmark's
# CPU comparison only (timing information; the element loop above is the
# oracle).  tests/test_oracle_pins.py checks them against the element loop.
#
# With G groups of P members and St = S/P, Hl = H/P (readings R1-R3 above):
#   sequence-sharded buffer  (g, js, bl, t, jh, hl, e)   shape (G, P, Bl, St, P, Hl, d)
#   head-major buffer        (g, jh, bl, hl, js, t, e)   shape (G, P, Bl, Hl, P, St, d)
#   token-major buffer       (g, jh, bl, js, t, hl, e)   shape (G, P, Bl, P, St, Hl, d)
# where member js holds tokens js*St + t and member jh holds heads jh*Hl + hl.

def _numpy_shapes(mode, N, B, S, H, d, G=0):
    gpb = groups(mode, N, B, G)
    if gpb is None or S % gpb[1] or H % gpb[1]:
        raise ValueError("the pages' conditions do not hold for mode=%d N=%d B=%d S=%d H=%d"
                         % (mode, N, B, S, H))
    G, P, Bl = gpb
    return G, P, Bl, S // P, H // P


def numpy_seq_to_head(x, mode, N, B, S, H, d, layout=HEAD_MAJOR, G=0):
    """Sequence-sharded -> head-sharded as one transpose of the rank-major buffer."""
    G, P, Bl, St, Hl = _numpy_shapes(mode, N, B, S, H, d, G)
    a = np.asarray(x).reshape(G, P, Bl, St, P, Hl, d)
    axes = (0, 4, 2, 5, 1, 3, 6) if layout == HEAD_MAJOR else (0, 4, 2, 1, 3, 5, 6)
    return np.ascontiguousarray(a.transpose(axes)).reshape(-1)


def numpy_head_to_seq(x, mode, N, B, S, H, d, layout=HEAD_MAJOR, G=0):
    """Head-sharded -> sequence-sharded, the inverse transpose."""
    G, P, Bl, St, Hl = _numpy_shapes(mode, N, B, S, H, d, G)
    if layout == HEAD_MAJOR:
        a = np.asarray(x).reshape(G, P, Bl, Hl, P, St, d)
        axes = (0, 4, 2, 5, 1, 3, 6)
    else:
        a = np.asarray(x).reshape(G, P, Bl, P, St, Hl, d)
        axes = (0, 3, 2, 4, 1, 5, 6)
    return np.ascontiguousarray(a.transpose(axes)).reshape(-1)
