"""Thin Python binding of ``libmoe_fused.so`` (the C ABI in include/moe_fused.h).

The functions with the C names marshal arguments and call the library; every
step of the layer runs in the HIP kernels.  ``fused_forward`` is a torch
convenience on top: it derives the dims from tensor shapes, checks dtypes, keeps
a workspace tensor per (device, stream) and passes ``data_ptr()`` values and the
current stream.  There is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_fused.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe_fused.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_SCRATCH = 5
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_MODE_F32ACT = 0
MOE_MODE_BF16 = 1
MOE_MODE_FP8 = 2
MOE_MODE_MXFP8 = 3
MOE_MODE_INT8 = 4

MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_PACKED = 1

MOE_ACT_SWIGLU = 0
MOE_ACT_SWIGLU_CLAMPED = 1

MOE_LAUNCH_MULTI = 0
MOE_LAUNCH_SINGLE = 1
MOE_SYNC_BYTES = 265216
# int32 word of the synchronisation block counting single-launch waits that ran out
SYNC_TIMEOUTS_WORD = 64


class moe_dims(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("num_tokens", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_hidden", ctypes.c_int32), ("d_expert", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("activation", ctypes.c_int32), ("launch", ctypes.c_int32)]


class moe_scales(ctypes.Structure):
    _fields_ = [("x_scale", ctypes.c_void_p), ("w1_scale", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


class moe_route_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("counts", "offsets", "padded_offsets", "pos", "sorted_p", "ppos",
                                                "row_src", "tile_expert", "tile_row0", "stats")]


class moe_ws_layout(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_size_t) for n in ("counts", "offsets", "padded_offsets", "pos", "sorted_p", "ppos",
                                                 "row_src", "row_w", "tile_expert", "tile_row0", "stats", "tasks1",
                                                 "tasks2",
                                                 "h", "h_scale", "y", "zero", "x_bf16", "sync", "total")]
                + [(n, ctypes.c_int64) for n in ("n_pad_cap", "tile_cap", "task1_cap", "task2_cap")]
                + [(n, ctypes.c_int32) for n in ("block_n1", "block_n2", "max_row_blocks")])


class MoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where} failed: {moe_error_string(code)} (code {code})")
        self.code = code


_lib = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m skew_aware_grouped_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    L.moe_workspace_bytes.restype = ctypes.c_size_t
    L.moe_workspace_bytes.argtypes = [P(moe_dims)]
    L.moe_fused_forward.restype = ctypes.c_int
    L.moe_fused_forward.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, P(moe_scales), vp, vp, ctypes.c_size_t, vp]
    L.moe_fused_forward_profiled.restype = ctypes.c_int
    L.moe_fused_forward_profiled.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, P(moe_scales), vp, vp,
                                             ctypes.c_size_t, vp, P(vp)]
    L.moe_fused_forward_noalloc.restype = ctypes.c_int
    L.moe_fused_forward_noalloc.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, P(moe_scales), vp, vp]
    L.moe_backward_workspace_bytes.restype = ctypes.c_size_t
    L.moe_backward_workspace_bytes.argtypes = [P(moe_dims)]
    L.moe_fused_backward.restype = ctypes.c_int
    L.moe_fused_backward.argtypes = [P(moe_dims), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.moe_workspace_init.restype = ctypes.c_int
    L.moe_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    L.moe_pack_weights.restype = ctypes.c_int
    L.moe_pack_weights.argtypes = [P(moe_dims), vp, vp, vp, vp, vp]
    L.moe_block_m.restype = ctypes.c_int32
    L.moe_block_m.argtypes = []
    L.moe_route_caps.restype = ctypes.c_int
    L.moe_route_caps.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int64),
                                 P(ctypes.c_int64)]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, P(moe_route_out), vp]
    L.moe_workspace_layout.restype = ctypes.c_int
    L.moe_workspace_layout.argtypes = [P(moe_dims), P(moe_ws_layout)]
    L.moe_error_string.restype = ctypes.c_char_p
    L.moe_error_string.argtypes = [ctypes.c_int]
    _lib = L
    return L


def header_symbols() -> list:
    """Names of the entry points the public header declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


# ------------------------------------------------------------- C entry points
def moe_workspace_bytes(dims: moe_dims) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(dims)))


def moe_fused_forward(dims, x, topk_ids, topk_w, w1, w2, scales, out, workspace, workspace_bytes, stream) -> int:
    return int(lib().moe_fused_forward(ctypes.byref(dims) if dims is not None else None, x, topk_ids, topk_w, w1,
                                       w2, ctypes.byref(scales) if scales is not None else None, out, workspace,
                                       workspace_bytes, stream))


def moe_fused_forward_noalloc(dims, x, topk_ids, topk_w, w1, w2, scales, out, stream) -> int:
    return int(lib().moe_fused_forward_noalloc(ctypes.byref(dims) if dims is not None else None, x, topk_ids, topk_w,
                                               w1, w2, ctypes.byref(scales) if scales is not None else None, out,
                                               stream))


def moe_fused_forward_profiled(dims, x, topk_ids, topk_w, w1, w2, scales, out, workspace, workspace_bytes, stream,
                               events) -> int:
    ev = (ctypes.c_void_p * 8)(*events) if events is not None else None
    return int(lib().moe_fused_forward_profiled(ctypes.byref(dims), x, topk_ids, topk_w, w1, w2,
                                                ctypes.byref(scales) if scales is not None else None, out,
                                                workspace, workspace_bytes, stream, ev))


def moe_backward_workspace_bytes(dims: moe_dims) -> int:
    return int(lib().moe_backward_workspace_bytes(ctypes.byref(dims)))


def moe_fused_backward(dims, x, topk_ids, topk_w, w1, w2, dout, dx, dw1, dw2, dtopk_w, workspace, workspace_bytes,
                       stream) -> int:
    return int(lib().moe_fused_backward(ctypes.byref(dims) if dims is not None else None, x, topk_ids, topk_w, w1, w2,
                                        dout, dx, dw1, dw2, dtopk_w, workspace, workspace_bytes, stream))


def moe_workspace_init(workspace, workspace_bytes, stream) -> int:
    return int(lib().moe_workspace_init(workspace, workspace_bytes, stream))


def moe_pack_weights(dims, w1, w2, w1_packed, w2_packed, stream) -> int:
    return int(lib().moe_pack_weights(ctypes.byref(dims) if dims is not None else None, w1, w2, w1_packed,
                                      w2_packed, stream))


def moe_block_m() -> int:
    return int(lib().moe_block_m())


def moe_route_caps(num_tokens: int, top_k: int, num_experts: int):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().moe_route_caps(num_tokens, top_k, num_experts, ctypes.byref(a), ctypes.byref(b))
    if rc:
        raise MoEError(rc, "moe_route_caps")
    return a.value, b.value


def moe_route(num_tokens, top_k, num_experts, topk_ids, out: moe_route_out, stream) -> int:
    return int(lib().moe_route(num_tokens, top_k, num_experts, topk_ids, ctypes.byref(out), stream))


def moe_workspace_layout(dims: moe_dims) -> moe_ws_layout:
    L = moe_ws_layout()
    rc = lib().moe_workspace_layout(ctypes.byref(dims), ctypes.byref(L))
    if rc:
        raise MoEError(rc, "moe_workspace_layout")
    return L


def moe_error_string(code: int) -> str:
    return lib().moe_error_string(code).decode()


# ------------------------------------------------------------ torch helpers
def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _mode_of(x, w1, x_scale=None):
    """e4m3 weights: MXFP8 when the scales are E8M0 bytes (uint8), else FP8;
    int8 tokens: INT8."""
    import torch
    if x.dtype == torch.int8:
        return MOE_MODE_INT8
    if w1.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MOE_MODE_MXFP8 if x_scale is not None and x_scale.dtype == torch.uint8 else MOE_MODE_FP8
    if x.dtype == torch.float32:
        return MOE_MODE_F32ACT
    return MOE_MODE_BF16


_workspaces = {}


def workspace_for(dims: moe_dims, device, stream=None):
    """A cached uint8 workspace tensor large enough for ``dims``, one per
    (device, stream): calls that share a workspace must be ordered on one
    stream (the routing counters, task queues and intermediates in it are
    rewritten by every call), so two streams never get the same buffer.  The
    tensor is allocated on that stream, so torch's allocator does not reuse
    its memory while work queued there may still read it.  It starts zeroed,
    which the single launch needs of its synchronisation block."""
    import torch
    need = moe_workspace_bytes(dims)
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    key = (str(dev), int(s.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        with torch.cuda.stream(s):
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def make_dims(x, topk_ids, w1, mode: Optional[int] = None, weight_layout: int = MOE_WEIGHTS_ROW_MAJOR,
              x_scale=None, activation: int = MOE_ACT_SWIGLU, launch: int = MOE_LAUNCH_MULTI) -> moe_dims:
    T, d_h = x.shape
    E, two_de, d_h2 = w1.shape
    assert d_h2 == d_h and two_de % 2 == 0, "w1 must be [E, 2*d_expert, d_hidden]"
    return moe_dims(mode=_mode_of(x, w1, x_scale) if mode is None else mode, num_tokens=T, num_experts=E,
                    top_k=topk_ids.shape[1], d_hidden=d_h, d_expert=two_de // 2, weight_layout=weight_layout,
                    activation=activation, launch=launch)


def pack_weights(w1, w2, stream=None):
    """``moe_pack_weights`` on torch device tensors: new tensors of the same
    shapes and dtypes holding W1 and W2 in the packed tile order (pass them
    to ``fused_forward`` with ``weight_layout=MOE_WEIGHTS_PACKED``)."""
    import torch
    E, two_de, d_h = w1.shape
    mode = MOE_MODE_FP8 if w1.dtype in (torch.float8_e4m3fn, torch.uint8) else MOE_MODE_BF16
    for name, t in (("w1", w1), ("w2", w2)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(w2.shape) != (E, d_h, two_de // 2):
        raise ValueError("w2 must be [E, d_hidden, d_expert]")
    dims = moe_dims(mode=mode, num_tokens=0, num_experts=E, top_k=1, d_hidden=d_h, d_expert=two_de // 2)
    p1, p2 = torch.empty_like(w1), torch.empty_like(w2)
    rc = moe_pack_weights(dims, w1.data_ptr(), w2.data_ptr(), p1.data_ptr(), p2.data_ptr(), _stream_ptr(stream))
    if rc:
        raise MoEError(rc, "moe_pack_weights")
    return p1, p2


def fused_forward(x, topk_ids, topk_w, w1, w2, out=None, x_scale=None, w1_scale=None, w2_scale=None,
                  workspace=None, stream=None, events=None, weight_layout=MOE_WEIGHTS_ROW_MAJOR,
                  activation=MOE_ACT_SWIGLU, launch=MOE_LAUNCH_MULTI):
    """Run ``moe_fused_forward`` on torch device tensors; returns ``out``.  With
    ``events`` (8 torch.cuda.Event objects: start and end of the routing, GEMM-1,
    GEMM-2 and combine kernels) the kernel-timing variant is used.  With
    ``weight_layout=MOE_WEIGHTS_PACKED``, w1 and w2 are ``pack_weights`` outputs.
    e4m3 weights take fp32 block scales (FP8 mode) or uint8 E8M0 scales per 32
    values (MXFP8 mode); the dtype of ``x_scale`` selects the mode.  int8 ``x``
    (INT8 mode) takes bf16 weights and one fp32 ``x_scale`` per token.
    ``launch=MOE_LAUNCH_SINGLE`` runs the layer as one kernel; a workspace
    passed in must then have had its synchronisation block zeroed once
    (``moe_workspace_init``; the cached workspaces are allocated zeroed)."""
    import torch
    dims = make_dims(x, topk_ids, w1, weight_layout=weight_layout, x_scale=x_scale, activation=activation,
                     launch=launch)
    if out is None:
        odt = torch.float32 if dims.mode == MOE_MODE_F32ACT else torch.bfloat16
        out = torch.empty(x.shape[0], x.shape[1], dtype=odt, device=x.device)
    for name, t in (("x", x), ("topk_ids", topk_ids), ("topk_w", topk_w), ("w1", w1), ("w2", w2), ("out", out)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if topk_ids.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("topk_ids must be int32 and topk_w float32")
    scales = None
    if dims.mode == MOE_MODE_INT8:
        if x_scale is None or not (x_scale.is_cuda and x_scale.is_contiguous()) or x_scale.dtype != torch.float32 \
                or x_scale.numel() != x.shape[0]:
            raise ValueError("x_scale must be a contiguous float32 device tensor with one scale per token")
        scales = moe_scales(x_scale.data_ptr(), None, None)
    elif dims.mode in (MOE_MODE_FP8, MOE_MODE_MXFP8):
        sdt = torch.uint8 if dims.mode == MOE_MODE_MXFP8 else torch.float32
        for name, t in (("x_scale", x_scale), ("w1_scale", w1_scale), ("w2_scale", w2_scale)):
            if t is None or not (t.is_cuda and t.is_contiguous()) or t.dtype != sdt:
                raise ValueError(f"{name} must be a contiguous {sdt} device tensor")
        scales = moe_scales(x_scale.data_ptr(), w1_scale.data_ptr(), w2_scale.data_ptr())
    ws = workspace if workspace is not None else workspace_for(dims, x.device, stream)
    args = (dims, x.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), w1.data_ptr(), w2.data_ptr(), scales,
            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    if events is None:
        rc = moe_fused_forward(*args)
    else:
        for e in events:
            if not e.cuda_event:  # torch creates its event lazily, on first record
                e.record(stream if stream is not None else torch.cuda.current_stream())
        rc = moe_fused_forward_profiled(*args, [e.cuda_event for e in events])
    if rc:
        raise MoEError(rc, "moe_fused_forward")
    return out


def fused_backward(x, topk_ids, topk_w, w1, w2, dout, workspace=None, stream=None):
    """``moe_fused_backward`` on torch device tensors (bf16 x, w1, w2, dout; int32
    ids; float32 weights): returns (dx, dw1, dw2, dtopk_w), float32."""
    import torch
    dims = make_dims(x, topk_ids, w1)
    if dims.mode != MOE_MODE_BF16:
        raise ValueError("the backward takes bf16 x and weights")
    for name, t in (("x", x), ("topk_ids", topk_ids), ("topk_w", topk_w), ("w1", w1), ("w2", w2), ("dout", dout)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if dout.dtype != torch.bfloat16 or tuple(dout.shape) != tuple(x.shape):
        raise ValueError("dout must be bf16 with the shape of x")
    T, d_h = x.shape
    E, two_de, _ = w1.shape
    dx = torch.empty(T, d_h, dtype=torch.float32, device=x.device)
    dw1 = torch.empty(E, two_de, d_h, dtype=torch.float32, device=x.device)
    dw2 = torch.empty(E, d_h, two_de // 2, dtype=torch.float32, device=x.device)
    dtw = torch.empty(topk_w.shape, dtype=torch.float32, device=x.device)
    need = moe_backward_workspace_bytes(dims)
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    rc = moe_fused_backward(dims, x.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                            dout.data_ptr(), dx.data_ptr(), dw1.data_ptr(), dw2.data_ptr(), dtw.data_ptr(),
                            ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    if rc:
        raise MoEError(rc, "moe_fused_backward")
    return dx, dw1, dw2, dtw
