"""ctypes binding of libbasp (``include/basp.h``): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
passed as device pointers (``data_ptr()``) after their dtype, device,
contiguity and element count are checked against the plan; plain ``int``
addresses are passed through unchanged.  The stream defaults to torch's
current stream on the current device.  Every step of the re-layout runs in
the HIP kernels of ``libbasp.so``; when that library is missing, importing
this module raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbasp.so")

BASP_OK = 0
BASP_ERR_INVALID = 1
BASP_ERR_INDIVISIBLE = 2
BASP_ERR_UNSUPPORTED = 3
BASP_ERR_ALIGN = 4
BASP_ERR_ALIAS = 5
BASP_ERR_HIP = 6

BASP_BF16 = 0
BASP_FP16 = 1
BASP_FP32 = 2
BASP_INT32 = 3

BASP_MODE_ULYSSES = 0
BASP_MODE_BASP = 1
BASP_MODE_GROUPS = 2

BASP_LAYOUT_HEAD_MAJOR = 0
BASP_LAYOUT_TOKEN_MAJOR = 1

BASP_SEQ_TO_HEAD = 0
BASP_HEAD_TO_SEQ = 1


class basp_plan_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("N", "B", "Hq", "Hkv", "d", "elem_size")] + [
        ("S", ctypes.c_int64)] + [(n, ctypes.c_int32) for n in ("mode", "layout", "dtype", "G", "P", "Bl")] + [
        ("St", ctypes.c_int64)] + [(n, ctypes.c_int32) for n in ("Hl_q", "Hl_kv")] + [
        ("tokens_per_rank", ctypes.c_int64), ("peers_per_rank", ctypes.c_int32)] + [
        (n, ctypes.c_int64) for n in (
            "q_elems", "kv_elems", "q_elems_per_rank", "kv_elems_per_rank", "qkv_elems",
            "qkv_offset_q", "qkv_offset_k", "qkv_offset_v", "per_peer_bytes_q",
            "per_peer_bytes_kv", "cross_rank_bytes_q", "cross_rank_bytes_kv",
            "qkv_bytes_moved", "o_bytes_moved", "tokens_per_rank_foil")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class basp_tuning(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "vectors_per_thread", "tile_tokens", "tile_heads", "cache_policy", "max_grid",
        "lane_order", "xcd_remap", "tile_order", "stage", "block_size", "batch_order")]


class BaspError(RuntimeError):
    """A libbasp call returned a status other than BASP_OK."""

    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s: %s" % (call, basp_status_str(status)))


# torch first: libbasp.so then binds to the HIP runtime torch has loaded, so
# that streams, events and allocations are shared with it (one runtime per
# process).
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError("libbasp.so is not built (expected at %s); build it with "
                      "`python -m sequence_re_layout_amd.build`" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
_plan_p = ctypes.c_void_p
_lib.basp_plan_create.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32]
_lib.basp_plan_create.restype = _plan_p
_lib.basp_plan_create_ex.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.basp_plan_create_ex.restype = _plan_p
_lib.basp_plan_create_groups.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32]
_lib.basp_plan_create_groups.restype = _plan_p
_lib.basp_plan_destroy.argtypes = [_plan_p]
_lib.basp_plan_destroy.restype = None
_lib.basp_plan_query.argtypes = [_plan_p, ctypes.POINTER(basp_plan_info)]
_lib.basp_plan_query.restype = _i32
_lib.basp_seq_to_head.argtypes = [_plan_p, _vp, _vp, _vp, _vp, _vp]
_lib.basp_seq_to_head.restype = _i32
_lib.basp_head_to_seq.argtypes = [_plan_p, _vp, _vp, _vp]
_lib.basp_head_to_seq.restype = _i32
_lib.basp_seq_to_head_o.argtypes = [_plan_p, _vp, _vp, _vp]
_lib.basp_seq_to_head_o.restype = _i32
_lib.basp_head_to_seq_qkv.argtypes = [_plan_p, _vp, _vp, _vp, _vp, _vp]
_lib.basp_head_to_seq_qkv.restype = _i32
_lib.basp_unfused_workspace_bytes.argtypes = [_plan_p]
_lib.basp_unfused_workspace_bytes.restype = ctypes.c_size_t
_lib.basp_seq_to_head_unfused.argtypes = [_plan_p, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.basp_seq_to_head_unfused.restype = _i32
_lib.basp_seq_to_head_unfused_noalloc.argtypes = [_plan_p, _vp, _vp, _vp, _vp, _vp]
_lib.basp_seq_to_head_unfused_noalloc.restype = _i32
_lib.basp_plan_set_tuning.argtypes = [_plan_p, ctypes.POINTER(basp_tuning)]
_lib.basp_plan_set_tuning.restype = _i32
_lib.basp_plan_set_direction_tuning.argtypes = [_plan_p, _i32, ctypes.POINTER(basp_tuning)]
_lib.basp_plan_set_direction_tuning.restype = _i32
_lib.basp_plan_get_tuning.argtypes = [_plan_p, _i32, ctypes.POINTER(basp_tuning)]
_lib.basp_plan_get_tuning.restype = _i32
_lib.basp_plan_autotune.argtypes = [_plan_p, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.basp_plan_autotune.restype = _i32
_lib.basp_time_next_call.argtypes = [_vp, _vp]
_lib.basp_time_next_call.restype = _i32
_lib.basp_stream_copy.argtypes = [_vp, _vp, ctypes.c_uint64, _vp]
_lib.basp_stream_copy.restype = _i32
_lib.basp_last_error.argtypes = []
_lib.basp_last_error.restype = _i32
_lib.basp_status_str.argtypes = [_i32]
_lib.basp_status_str.restype = ctypes.c_char_p


def library():
    """The loaded ``ctypes.CDLL`` of libbasp.so."""
    return _lib


class Plan:
    """Owner of a ``basp_plan*``; destroyed with the object.  ``info`` holds
    the ``basp_plan_query`` result as a dict."""

    def __init__(self, handle: int):
        self.handle = handle
        self.info = basp_plan_query(self)

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _lib is not None:   # _lib is None during interpreter shutdown
            _lib.basp_plan_destroy(h)

    @property
    def _as_parameter_(self):
        return self.handle


def _check(status: int, call: str) -> None:
    if status != BASP_OK:
        raise BaspError(status, call)


def basp_status_str(status: int) -> str:
    return _lib.basp_status_str(status).decode()


def basp_last_error() -> int:
    return _lib.basp_last_error()


def basp_plan_create(N, B, S, Hq, Hkv, d, dtype=BASP_BF16, mode=BASP_MODE_BASP) -> Plan:
    h = _lib.basp_plan_create(N, B, S, Hq, Hkv, d, dtype, mode)
    if not h:
        raise BaspError(_lib.basp_last_error(), "basp_plan_create")
    return Plan(h)


def basp_plan_create_ex(N, B, S, Hq, Hkv, d, dtype=BASP_BF16, mode=BASP_MODE_BASP,
                        layout=BASP_LAYOUT_HEAD_MAJOR) -> Plan:
    h = _lib.basp_plan_create_ex(N, B, S, Hq, Hkv, d, dtype, mode, layout)
    if not h:
        raise BaspError(_lib.basp_last_error(), "basp_plan_create_ex")
    return Plan(h)


def basp_plan_create_groups(N, B, S, Hq, Hkv, d, dtype=BASP_BF16, G=1,
                            layout=BASP_LAYOUT_HEAD_MAJOR) -> Plan:
    h = _lib.basp_plan_create_groups(N, B, S, Hq, Hkv, d, dtype, G, layout)
    if not h:
        raise BaspError(_lib.basp_last_error(), "basp_plan_create_groups")
    return Plan(h)


def basp_plan_destroy(plan: Plan) -> None:
    h, plan.handle = plan.handle, None
    _lib.basp_plan_destroy(h)


def basp_plan_query(plan: Plan) -> dict:
    info = basp_plan_info()
    _check(_lib.basp_plan_query(plan.handle, ctypes.byref(info)), "basp_plan_query")
    return info.as_dict()


_TUNING_FIELDS = ("vectors_per_thread", "tile_tokens", "tile_heads", "cache_policy", "max_grid",
                  "lane_order", "xcd_remap", "tile_order", "stage", "block_size", "batch_order")


def _tuning(fields) -> basp_tuning:
    unknown = set(fields) - set(_TUNING_FIELDS)
    if unknown:
        raise TypeError("unknown tuning fields %s" % sorted(unknown))
    return basp_tuning(*[int(fields.get(n, 0)) for n in _TUNING_FIELDS])


def basp_plan_set_tuning(plan: Plan, **fields) -> None:
    """Launch shape of both directions (fields of basp_tuning; unset = 0)."""
    t = _tuning(fields)
    _check(_lib.basp_plan_set_tuning(plan.handle, ctypes.byref(t)), "basp_plan_set_tuning")


def basp_plan_set_direction_tuning(plan: Plan, direction: int, **fields) -> None:
    t = _tuning(fields)
    _check(_lib.basp_plan_set_direction_tuning(plan.handle, direction, ctypes.byref(t)),
           "basp_plan_set_direction_tuning")


def basp_plan_get_tuning(plan: Plan, direction: int = BASP_SEQ_TO_HEAD) -> dict:
    t = basp_tuning()
    _check(_lib.basp_plan_get_tuning(plan.handle, direction, ctypes.byref(t)), "basp_plan_get_tuning")
    return {name: getattr(t, name) for name, _ in t._fields_}


def basp_plan_autotune(plan: Plan, q, k, v, qkv, o, o_out, stream=None) -> None:
    """Measure launch shapes and keep the fastest per direction: on these
    buffers, or, when the six total less than 32 MiB, on a temporary pool the
    library allocates and frees (see basp.h).  qkv and o_out end up holding
    the results of the two calls."""
    i = plan.info
    _check(_lib.basp_plan_autotune(
        plan.handle, _ptr(q, plan, i["q_elems"], "q"), _ptr(k, plan, i["kv_elems"], "k"),
        _ptr(v, plan, i["kv_elems"], "v"), _ptr(qkv, plan, i["qkv_elems"], "qkv"),
        _ptr(o, plan, i["q_elems"], "o"), _ptr(o_out, plan, i["q_elems"], "o_out"),
        _stream(stream)), "basp_plan_autotune")


def basp_time_next_call(start_event, stop_event) -> None:
    """Time the next call of this thread from its kernels' own dispatch
    timestamps.  Takes torch.cuda.Event objects (already recorded once, so
    that their handles exist) or raw hipEvent_t addresses."""
    def handle(e):
        if e is None or isinstance(e, int):
            return e
        return e.cuda_event
    _check(_lib.basp_time_next_call(handle(start_event), handle(stop_event)), "basp_time_next_call")


def basp_unfused_workspace_bytes(plan: Plan) -> int:
    return int(_lib.basp_unfused_workspace_bytes(plan.handle))


# ------------------------------------------------------------ marshalling --

def _torch_dtype(code):
    import torch
    return {BASP_BF16: torch.bfloat16, BASP_FP16: torch.float16,
            BASP_FP32: torch.float32, BASP_INT32: torch.int32}[code]


def _check_device(x, name: str) -> None:
    """The library launches on the current device: a tensor elsewhere is an
    error, not a cross-device access."""
    import torch
    if x.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s, the current device is cuda:%d"
                         % (name, x.device, torch.cuda.current_device()))


def _ptr(x, plan: Plan, numel: int, name: str):
    """Device address of a tensor checked against the plan, or an int as is."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if x.dtype != _torch_dtype(plan.info["dtype"]):
        raise TypeError("%s: dtype %s does not match the plan" % (name, x.dtype))
    if not x.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    _check_device(x, name)
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.numel() != numel:
        raise ValueError("%s holds %d elements, the plan needs %d" % (name, x.numel(), numel))
    return x.data_ptr() if numel else None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def basp_seq_to_head(plan: Plan, q, k, v, out, stream=None) -> None:
    i = plan.info
    _check(_lib.basp_seq_to_head(
        plan.handle, _ptr(q, plan, i["q_elems"], "q"), _ptr(k, plan, i["kv_elems"], "k"),
        _ptr(v, plan, i["kv_elems"], "v"), _ptr(out, plan, i["qkv_elems"], "out"),
        _stream(stream)), "basp_seq_to_head")


def basp_head_to_seq(plan: Plan, o, out, stream=None) -> None:
    i = plan.info
    _check(_lib.basp_head_to_seq(
        plan.handle, _ptr(o, plan, i["q_elems"], "o"), _ptr(out, plan, i["q_elems"], "out"),
        _stream(stream)), "basp_head_to_seq")


def basp_seq_to_head_o(plan: Plan, dout, out, stream=None) -> None:
    i = plan.info
    _check(_lib.basp_seq_to_head_o(
        plan.handle, _ptr(dout, plan, i["q_elems"], "dout"), _ptr(out, plan, i["q_elems"], "out"),
        _stream(stream)), "basp_seq_to_head_o")


def basp_head_to_seq_qkv(plan: Plan, inp, dq, dk, dv, stream=None) -> None:
    i = plan.info
    _check(_lib.basp_head_to_seq_qkv(
        plan.handle, _ptr(inp, plan, i["qkv_elems"], "in"), _ptr(dq, plan, i["q_elems"], "dq"),
        _ptr(dk, plan, i["kv_elems"], "dk"), _ptr(dv, plan, i["kv_elems"], "dv"),
        _stream(stream)), "basp_head_to_seq_qkv")


def basp_seq_to_head_unfused(plan: Plan, q, k, v, out, ws, stream=None) -> None:
    i = plan.info
    if ws is not None and not isinstance(ws, int):
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous device tensor")
        _check_device(ws, "ws")
        if ws.numel() * ws.element_size() < basp_unfused_workspace_bytes(plan):
            raise ValueError("ws holds %d bytes, the plan needs %d"
                             % (ws.numel() * ws.element_size(), basp_unfused_workspace_bytes(plan)))
        ws = ws.data_ptr()
    _check(_lib.basp_seq_to_head_unfused(
        plan.handle, _ptr(q, plan, i["q_elems"], "q"), _ptr(k, plan, i["kv_elems"], "k"),
        _ptr(v, plan, i["kv_elems"], "v"), _ptr(out, plan, i["qkv_elems"], "out"), ws,
        _stream(stream)), "basp_seq_to_head_unfused")


BASP_NOALLOC_SCRATCH_BYTES = 64 << 20


def basp_seq_to_head_unfused_noalloc(plan: Plan, q, k, v, out, stream=None) -> None:
    i = plan.info
    _check(_lib.basp_seq_to_head_unfused_noalloc(
        plan.handle, _ptr(q, plan, i["q_elems"], "q"), _ptr(k, plan, i["kv_elems"], "k"),
        _ptr(v, plan, i["kv_elems"], "v"), _ptr(out, plan, i["qkv_elems"], "out"),
        _stream(stream)), "basp_seq_to_head_unfused_noalloc")


def basp_stream_copy(dst, src, nbytes=None, stream=None) -> None:
    """Plain device copy of nbytes bytes (default: all of src) with the
    re-layout kernels' access rules; dst and src are device tensors or raw
    addresses."""
    def addr(x, name):
        if isinstance(x, int) or x is None:
            return x
        if not x.is_cuda or not x.is_contiguous():
            raise ValueError("%s must be a contiguous device tensor" % name)
        _check_device(x, name)
        return x.data_ptr()

    if nbytes is None:
        if isinstance(src, int) or src is None:
            raise ValueError("nbytes is needed when src is a raw address")
        nbytes = src.numel() * src.element_size()
    for x, name in ((dst, "dst"), (src, "src")):
        if not isinstance(x, int) and x is not None and x.numel() * x.element_size() < nbytes:
            raise ValueError("%s holds fewer than %d bytes" % (name, nbytes))
    _check(_lib.basp_stream_copy(addr(dst, "dst"), addr(src, "src"), nbytes, _stream(stream)),
           "basp_stream_copy")
