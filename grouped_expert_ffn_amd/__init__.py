"""Python binding of the MI355X MoE token-dispatch library (libmoe_dispatch.so).

Argument marshalling only: each function checks the torch tensors it is
given (device, dtype, shape, contiguity), passes their device pointers and
torch's current HIP stream to the C entry point of the same name, and raises
``MoeError`` on a non-zero status. All arithmetic runs in the library's HIP
kernels; torch provides device memory and streams. There is no fallback:
importing this package fails loudly when the library has not been built.

The layer: y_t = sum over e in TopK(h_t W_r, k) of g_{t,e} f_e(h_t)
("How Does Mixture-of-Experts Routing Affect LLM Repeatability?", token-choice
layer formula), staged as route -> permute -> grouped FFN -> unpermute/combine.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_dispatch.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
GATES = {"softmax": 0, "softmax_topk_renorm": 1, "sigmoid_topk_renorm": 2}
ACTS = {"relu": 0, "swiglu": 1}
FLAG_ROW_OVERFLOW, FLAG_BAD_EXPERT_ID, FLAG_NONFINITE_LOGIT, FLAG_DROPPED = 1, 2, 4, 8

EXPORTED = ("moe_capacity_from_factor", "moe_workspace_size", "moe_route",
            "moe_topk_from_logits", "moe_permute", "moe_grouped_ffn",
            "moe_permute_no_workspace",
            "moe_grouped_ffn_gather", "moe_grouped_ffn_slots", "moe_pack_dedup",
            "moe_unpermute_combine", "moe_combine_slots",
            "moe_layer_forward", "moe_status_str")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_str(status)}")


class LayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("act", ctypes.c_int32), ("ep_size", ctypes.c_int32),
                ("ep_rank", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("max_rows", ctypes.c_int64)]


class LayerBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "logits", "topk_idx", "topk_gate", "counts", "offsets", "dest", "src_token",
        "src_slot", "send_splits", "send_displs", "x_perm", "y_perm", "flags")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python grouped_expert_ffn_amd/build.py` "
            "(no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(LayerDesc)
    sig = {
        "moe_capacity_from_factor": (I64, [ctypes.c_double, I64, I32, I32]),
        "moe_workspace_size": (I32, [D, ctypes.POINTER(SZ)]),
        "moe_route": (I32, [D, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_topk_from_logits": (I32, [D, P, P, P, P, P]),
        "moe_permute": (I32, [D, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_permute_no_workspace": (I32, [D, P, P, P, P, P, P, P, P, P, P, P, P]),
        "moe_grouped_ffn": (I32, [D, P, P, P, P, P, P, P, SZ, P]),
        "moe_grouped_ffn_gather": (I32, [D, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_pack_dedup": (I32, [D, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_grouped_ffn_slots": (I32, [D, P, P, P, P, P, P, P, P, P, SZ, P]),
        "moe_combine_slots": (I32, [D, P, P, P, P, P, P]),
        "moe_unpermute_combine": (I32, [D, P, P, P, P, P, P]),
        "moe_layer_forward": (I32, [D, P, P, P, P, P, P, ctypes.POINTER(LayerBuffers), P, SZ, P]),
        "moe_status_str": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


_lib = _load()


def status_str(status: int) -> str:
    return _lib.moe_status_str(status).decode()


def capacity_from_factor(cf, T: int, k: int, E: int) -> int:
    """floor(cf*T*k/E), or -1 (dropless) when cf is None."""
    return int(_lib.moe_capacity_from_factor(-1.0 if cf is None else float(cf), T, k, E))


def make_desc(T, d, E, k, d_ff, dtype, gate, act, *, ep_size=1, ep_rank=0, capacity=-1,
              max_rows=None) -> LayerDesc:
    if isinstance(dtype, torch.dtype):
        dtype = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}[dtype]
    elif isinstance(dtype, str):
        dtype = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}[dtype]
    return LayerDesc(T=T, d=d, E=E, k=k, d_ff=d_ff, dtype=dtype,
                     gate=GATES[gate] if isinstance(gate, str) else gate,
                     act=ACTS[act] if isinstance(act, str) else act,
                     ep_size=ep_size, ep_rank=ep_rank, reserved=0,
                     capacity=-1 if capacity is None else capacity,
                     max_rows=T * k if max_rows is None else max_rows)


def torch_dtype(desc: LayerDesc) -> torch.dtype:
    return torch.bfloat16 if desc.dtype == DTYPE_BF16 else torch.float32


def workspace_size(desc: LayerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def alloc_workspace(desc: LayerDesc, device="cuda") -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks
    return torch.empty(max(1, workspace_size(desc)), dtype=torch.uint8, device=device)


def _check(status, where):
    if status != 0:
        raise MoeError(status, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws):
    return _ptr(ws, "ws", torch.uint8), ctypes.c_size_t(ws.numel())


def _flags(flags):
    return _ptr(flags, "flags", torch.int32, (1,), optional=True)


@dataclass
class LayerBuffersT:
    """Device tensors of the fused call's outputs and intermediates. Only
    y_perm is required; a field left None is kept in the workspace (and
    x_perm None also means the first expert GEMM gathers rows from h)."""
    logits: Optional[torch.Tensor]
    topk_idx: Optional[torch.Tensor]
    topk_gate: Optional[torch.Tensor]
    counts: Optional[torch.Tensor]
    offsets: Optional[torch.Tensor]
    dest: Optional[torch.Tensor]
    src_token: Optional[torch.Tensor]
    src_slot: Optional[torch.Tensor]
    send_splits: Optional[torch.Tensor]
    send_displs: Optional[torch.Tensor]
    x_perm: Optional[torch.Tensor]
    y_perm: torch.Tensor
    flags: Optional[torch.Tensor]


def alloc_buffers(desc: LayerDesc, device="cuda", x_perm=True, outputs=True) -> LayerBuffersT:
    """Buffers of the fused call. x_perm=False leaves out the expert-ordered
    copy of the rows (the first expert GEMM then gathers them); outputs=False
    leaves out every optional output (logits, routing, plan, splits, flags),
    which the call then keeps in its workspace."""
    T, E, k, d, R = desc.T, desc.E, desc.k, desc.d, desc.max_rows
    dt = torch_dtype(desc)
    i32, f32 = torch.int32, torch.float32

    def opt(make):
        return make() if outputs else None

    return LayerBuffersT(
        logits=opt(lambda: torch.empty((T, E), dtype=f32, device=device)),
        topk_idx=opt(lambda: torch.empty((T, k), dtype=i32, device=device)),
        topk_gate=opt(lambda: torch.empty((T, k), dtype=f32, device=device)),
        counts=opt(lambda: torch.empty((E,), dtype=i32, device=device)),
        offsets=opt(lambda: torch.empty((E + 1,), dtype=i32, device=device)),
        dest=opt(lambda: torch.empty((T, k), dtype=i32, device=device)),
        src_token=opt(lambda: torch.full((max(R, 1),), -1, dtype=i32, device=device)[:R]),
        src_slot=opt(lambda: torch.full((max(R, 1),), -1, dtype=i32, device=device)[:R]),
        send_splits=opt(lambda: torch.empty((desc.ep_size,), dtype=torch.int64, device=device)),
        send_displs=opt(lambda: torch.empty((desc.ep_size,), dtype=torch.int64, device=device)),
        x_perm=torch.empty((R, d), dtype=dt, device=device) if x_perm else None,
        y_perm=torch.empty((R, d), dtype=dt, device=device),
        flags=opt(lambda: torch.zeros((1,), dtype=torch.int32, device=device)),
    )


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI, without the moe_ prefix)

def route(desc, h, w_router, bias, logits, topk_idx, topk_gate, flags, ws, stream=None):
    dt = torch_dtype(desc)
    T, d, E, k = desc.T, desc.d, desc.E, desc.k
    wsp, wsn = _ws(ws)
    _check(_lib.moe_route(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)), _ptr(w_router, "w_router", dt, (d, E)),
        _ptr(bias, "router_bias", torch.float32, (E,), optional=True),
        _ptr(logits, "logits", torch.float32, (T, E)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_gate, "topk_gate", torch.float32, (T, k)),
        _ptr(flags, "flags", torch.int32, (1,)), wsp, wsn, _stream(stream)), "moe_route")


def topk_from_logits(desc, logits, topk_idx, topk_gate, flags, stream=None):
    T, E, k = desc.T, desc.E, desc.k
    _check(_lib.moe_topk_from_logits(
        ctypes.byref(desc), _ptr(logits, "logits", torch.float32, (T, E)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_gate, "topk_gate", torch.float32, (T, k)),
        _ptr(flags, "flags", torch.int32, (1,)), _stream(stream)), "moe_topk_from_logits")


def permute(desc, h, topk_idx, x_perm, counts, offsets, dest, src_token, src_slot,
            send_splits, send_displs, flags, ws, stream=None):
    dt = torch_dtype(desc)
    T, d, E, k, R = desc.T, desc.d, desc.E, desc.k, desc.max_rows
    wsp, wsn = _ws(ws)
    _check(_lib.moe_permute(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(x_perm, "x_perm", dt, (R, d), optional=True),
        _ptr(counts, "counts", torch.int32, (E,)),
        _ptr(offsets, "offsets", torch.int32, (E + 1,)),
        _ptr(dest, "dest", torch.int32, (T, k)),
        _ptr(src_token, "src_token", torch.int32, (R,)),
        _ptr(src_slot, "src_slot", torch.int32, (R,)),
        _ptr(send_splits, "send_splits", torch.int64, (desc.ep_size,)),
        _ptr(send_displs, "send_displs", torch.int64, (desc.ep_size,)),
        _ptr(flags, "flags", torch.int32, (1,)), wsp, wsn, _stream(stream)), "moe_permute")


def permute_no_workspace(desc, h, topk_idx, x_perm, counts, offsets, dest, src_token,
                         src_slot, send_splits, send_displs, flags, stream=None):
    """permute without a workspace: the plan's scratch is the library's fixed
    per-GPU array (calls that overlap on one GPU race)."""
    dt = torch_dtype(desc)
    T, d, E, k, R = desc.T, desc.d, desc.E, desc.k, desc.max_rows
    _check(_lib.moe_permute_no_workspace(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(x_perm, "x_perm", dt, (R, d), optional=True),
        _ptr(counts, "counts", torch.int32, (E,)),
        _ptr(offsets, "offsets", torch.int32, (E + 1,)),
        _ptr(dest, "dest", torch.int32, (T, k)),
        _ptr(src_token, "src_token", torch.int32, (R,)),
        _ptr(src_slot, "src_slot", torch.int32, (R,)),
        _ptr(send_splits, "send_splits", torch.int64, (desc.ep_size,)),
        _ptr(send_displs, "send_displs", torch.int64, (desc.ep_size,)),
        _ptr(flags, "flags", torch.int32, (1,)), _stream(stream)), "moe_permute_no_workspace")


def _w_shapes(desc):
    el = desc.E // desc.ep_size
    rows = 2 * desc.d_ff if desc.act == ACTS["swiglu"] else desc.d_ff
    return (el, rows, desc.d), (el, desc.d, desc.d_ff)


def grouped_ffn(desc, x_perm, offsets, w1, w2, y_perm, ws, stream=None, flags=None):
    """flags: optional [1] int32 word, OR-ed with FLAG_ROW_OVERFLOW when local
    rows lie past max_rows (the C argument before ws)."""
    dt = torch_dtype(desc)
    s1, s2 = _w_shapes(desc)
    R, d = desc.max_rows, desc.d
    wsp, wsn = _ws(ws)
    _check(_lib.moe_grouped_ffn(
        ctypes.byref(desc), _ptr(x_perm, "x_perm", dt, (R, d)),
        _ptr(offsets, "offsets", torch.int32, (desc.E + 1,)),
        _ptr(w1, "w1", dt, s1), _ptr(w2, "w2", dt, s2), _ptr(y_perm, "y_perm", dt, (R, d)),
        _flags(flags), wsp, wsn, _stream(stream)), "moe_grouped_ffn")


def grouped_ffn_gather(desc, h, src_token, offsets, w1, w2, y_perm, ws, stream=None,
                       flags=None):
    """h: the token rows [T, d], or a deduplicated send buffer [max_pairs, d]
    (then src_token is the recv_rows of moe_pack_dedup). flags as for
    grouped_ffn."""
    dt = torch_dtype(desc)
    s1, s2 = _w_shapes(desc)
    T, R, d = desc.T, desc.max_rows, desc.d
    if h is not None and h.shape[0] not in (T, max_pairs(desc)):
        raise ValueError(f"h must have {T} or {max_pairs(desc)} rows")
    wsp, wsn = _ws(ws)
    _check(_lib.moe_grouped_ffn_gather(
        ctypes.byref(desc), _ptr(h, "h", dt, (h.shape[0] if h is not None else T, d)),
        _ptr(src_token, "src_token", torch.int32, (R,)),
        _ptr(offsets, "offsets", torch.int32, (desc.E + 1,)),
        _ptr(w1, "w1", dt, s1), _ptr(w2, "w2", dt, s2), _ptr(y_perm, "y_perm", dt, (R, d)),
        _flags(flags), wsp, wsn, _stream(stream)), "moe_grouped_ffn_gather")


def grouped_ffn_slots(desc, h, src_token, src_slot, offsets, w1, w2, y_slots, ws, stream=None,
                      flags=None):
    """Gathered first GEMM; the second writes each grouped row to its
    (token, slot) row of y_slots [T*k, d]. flags as for grouped_ffn."""
    dt = torch_dtype(desc)
    s1, s2 = _w_shapes(desc)
    T, R, d, k = desc.T, desc.max_rows, desc.d, desc.k
    wsp, wsn = _ws(ws)
    _check(_lib.moe_grouped_ffn_slots(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)),
        _ptr(src_token, "src_token", torch.int32, (R,)),
        _ptr(src_slot, "src_slot", torch.int32, (R,)),
        _ptr(offsets, "offsets", torch.int32, (desc.E + 1,)),
        _ptr(w1, "w1", dt, s1), _ptr(w2, "w2", dt, s2), _ptr(y_slots, "y_slots", dt, (T * k, d)),
        _flags(flags), wsp, wsn, _stream(stream)), "moe_grouped_ffn_slots")


def max_pairs(desc) -> int:
    """Rows of a deduplicated send buffer: T * min(k, ep_size)."""
    return desc.T * min(desc.k, desc.ep_size)


def pack_dedup(desc, h, topk_idx, dest, src_token, src_slot, offsets, send_buf, pair_dest,
               pair_token, pair_splits, pair_displs, recv_rows, ws, stream=None):
    dt = torch_dtype(desc)
    T, d, k, R, P = desc.T, desc.d, desc.k, desc.max_rows, max_pairs(desc)
    wsp, wsn = _ws(ws)
    _check(_lib.moe_pack_dedup(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)), _ptr(dest, "dest", torch.int32, (T, k)),
        _ptr(src_token, "src_token", torch.int32, (R,)),
        _ptr(src_slot, "src_slot", torch.int32, (R,)),
        _ptr(offsets, "offsets", torch.int32, (desc.E + 1,)),
        _ptr(send_buf, "send_buf", dt, (P, d)),
        _ptr(pair_dest, "pair_dest", torch.int32, (T, k)),
        _ptr(pair_token, "pair_token", torch.int32, (P,)),
        _ptr(pair_splits, "pair_splits", torch.int64, (desc.ep_size,)),
        _ptr(pair_displs, "pair_displs", torch.int64, (desc.ep_size,)),
        _ptr(recv_rows, "recv_rows", torch.int32, (R,)), wsp, wsn, _stream(stream)),
        "moe_pack_dedup")


def unpermute_combine(desc, y_perm, topk_idx, topk_gate, dest, y, stream=None):
    dt = torch_dtype(desc)
    T, d, k, R = desc.T, desc.d, desc.k, desc.max_rows
    _check(_lib.moe_unpermute_combine(
        ctypes.byref(desc), _ptr(y_perm, "y_perm", dt, (R, d)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_gate, "topk_gate", torch.float32, (T, k)),
        _ptr(dest, "dest", torch.int32, (T, k)), _ptr(y, "y", dt, (T, d)),
        _stream(stream)), "moe_unpermute_combine")


def combine_slots(desc, y_slots, topk_idx, topk_gate, dest, y, stream=None):
    dt = torch_dtype(desc)
    T, d, k = desc.T, desc.d, desc.k
    _check(_lib.moe_combine_slots(
        ctypes.byref(desc), _ptr(y_slots, "y_slots", dt, (T * k, d)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_gate, "topk_gate", torch.float32, (T, k)),
        _ptr(dest, "dest", torch.int32, (T, k)), _ptr(y, "y", dt, (T, d)),
        _stream(stream)), "moe_combine_slots")


def layer_forward(desc, h, w_router, bias, w1, w2, y, bufs: LayerBuffersT, ws, stream=None):
    dt = torch_dtype(desc)
    T, d, E, k, R = desc.T, desc.d, desc.E, desc.k, desc.max_rows
    s1, s2 = _w_shapes(desc)

    def o(t, name, dtype, shape):
        p = _ptr(t, name, dtype, shape, optional=True)
        return None if p is None else p.value

    b = LayerBuffers(
        logits=o(bufs.logits, "logits", torch.float32, (T, E)),
        topk_idx=o(bufs.topk_idx, "topk_idx", torch.int32, (T, k)),
        topk_gate=o(bufs.topk_gate, "topk_gate", torch.float32, (T, k)),
        counts=o(bufs.counts, "counts", torch.int32, (E,)),
        offsets=o(bufs.offsets, "offsets", torch.int32, (E + 1,)),
        dest=o(bufs.dest, "dest", torch.int32, (T, k)),
        src_token=o(bufs.src_token, "src_token", torch.int32, (R,)),
        src_slot=o(bufs.src_slot, "src_slot", torch.int32, (R,)),
        send_splits=o(bufs.send_splits, "send_splits", torch.int64, (desc.ep_size,)),
        send_displs=o(bufs.send_displs, "send_displs", torch.int64, (desc.ep_size,)),
        x_perm=o(bufs.x_perm, "x_perm", dt, (R, d)),
        y_perm=_ptr(bufs.y_perm, "y_perm", dt, (R, d)).value,
        flags=o(bufs.flags, "flags", torch.int32, (1,)))
    wsp, wsn = _ws(ws)
    _check(_lib.moe_layer_forward(
        ctypes.byref(desc), _ptr(h, "h", dt, (T, d)), _ptr(w_router, "w_router", dt, (d, E)),
        _ptr(bias, "router_bias", torch.float32, (E,), optional=True),
        _ptr(w1, "w1", dt, s1), _ptr(w2, "w2", dt, s2), _ptr(y, "y", dt, (T, d)),
        ctypes.byref(b), wsp, wsn, _stream(stream)), "moe_layer_forward")
