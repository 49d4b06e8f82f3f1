"""ctypes wrapper around the plain C oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports this
module and this module imports nothing from the product package.

Every function here marshals numpy arrays and calls the C code; the arithmetic
lives in ``moe_oracle.c`` (see its header for what it follows on the pages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

MODE_F32ACT = 0
MODE_BF16 = 1
MODE_FP8 = 2
MODE_MXFP8 = 3
MODE_INT8 = 4
MIRROR_H = 1
ACC64 = 2
ACT_CLAMPED = 4  # clamped activation (GPT-OSS variant of SwiGLU)
ACT_SWIGLU, ACT_SWIGLU_CLAMPED = 0, 1  # values of a workload's ``activation``

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MOE_ORACLE_LIB points the wrapper at a deliberately broken build of the
    # oracle; the mutation test uses it to show that the pins catch mistakes.
    path = os.environ.get("MOE_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_bf16_encode.restype = ctypes.c_uint16
    lib.oracle_bf16_encode.argtypes = [ctypes.c_float]
    lib.oracle_bf16_decode.restype = ctypes.c_float
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_requant_chunk.restype = None
    lib.oracle_requant_chunk.argtypes = [vp, i64, i32]
    lib.oracle_e8m0_decode.restype = ctypes.c_double
    lib.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_mx_requant_block.restype = None
    lib.oracle_mx_requant_block.argtypes = [vp, i64, vp]
    lib.moe_oracle_forward.restype = i32
    lib.moe_oracle_forward.argtypes = [i32, i64, i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                       vp, i64, vp, vp]
    lib.moe_oracle_backward.restype = i32
    lib.moe_oracle_backward.argtypes = [i32, i64, i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.moe_oracle_route.restype = i32
    lib.moe_oracle_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, i64, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- codecs
def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def e4m3_encode(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float64)
    return np.array([lib.oracle_e4m3_encode(float(a)) for a in v.ravel()], dtype=np.uint8).reshape(v.shape)


def bf16_encode(values) -> np.ndarray:
    lib = _load()
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib.oracle_bf16_encode(float(a)) for a in v.ravel()], dtype=np.uint16).reshape(v.shape)


def bf16_decode(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_decode(int(a)) for a in b.ravel()], dtype=np.float32).reshape(b.shape)


def requant_chunk(values, acc64: bool = False) -> np.ndarray:
    """FP8 requantisation of one chunk of the intermediate (returns dequantised values)."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(values, dtype=np.float64).copy())
    lib.oracle_requant_chunk(_ptr(a), a.size, 1 if acc64 else 0)
    return a


def e8m0_decode(scales) -> np.ndarray:
    lib = _load()
    s = np.asarray(scales, dtype=np.uint8)
    return np.array([lib.oracle_e8m0_decode(int(v)) for v in s.ravel()], dtype=np.float64).reshape(s.shape)


def mx_requant_block(values):
    """MX requantisation of one block of the intermediate: (dequantised values, E8M0 scale byte)."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(values, dtype=np.float64).copy())
    sc = np.zeros(1, np.uint8)
    lib.oracle_mx_requant_block(_ptr(a), a.size, _ptr(sc))
    return a, int(sc[0])


# ----------------------------------------------------------------- routing
def route(ids, num_experts: int, bm: int) -> dict:
    """Routing metadata for flat assignment ids (see moe_oracle_route)."""
    lib = _load()
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
    n = ids.size
    E = int(num_experts)
    n_pad_cap = n + min(E, n) * (bm - 1)
    tile_cap = max(1, n_pad_cap // bm)
    out = {
        "counts": np.zeros(E, np.int32),
        "offsets": np.zeros(E + 1, np.int32),
        "padded_offsets": np.zeros(E + 1, np.int32),
        "pos": np.zeros(n, np.int32),
        "sorted_p": np.zeros(n, np.int32),
        "ppos": np.zeros(n, np.int32),
        "row_src": np.zeros(max(1, n_pad_cap), np.int32),
        "tile_expert": np.zeros(tile_cap, np.int32),
        "tile_row0": np.zeros(tile_cap, np.int32),
    }
    stats = np.zeros(2, np.int64)
    rc = lib.moe_oracle_route(_ptr(ids), n, E, int(bm), _ptr(out["counts"]), _ptr(out["offsets"]),
                              _ptr(out["padded_offsets"]), _ptr(out["pos"]), _ptr(out["sorted_p"]),
                              _ptr(out["ppos"]), _ptr(out["row_src"]), out["row_src"].size,
                              _ptr(out["tile_expert"]), _ptr(out["tile_row0"]), tile_cap, _ptr(stats))
    if rc != 0:
        raise ValueError(f"moe_oracle_route failed with code {rc}")
    out["dropped"] = int(stats[0])
    out["ntiles"] = int(stats[1])
    out["n_pad"] = int(out["padded_offsets"][E])
    return out


# ----------------------------------------------------------------- forward
def forward(inp, rows=None, mirror: bool = True, acc64: bool = False):
    """Layer output for the tokens in ``rows`` (all tokens when None).

    ``inp`` is a workload object with fields mode, T, E, k, d_h, d_e, x, x_scale,
    topk_ids, topk_w, w1, w1_scale, w2, w2_scale (numpy, see the input generator).
    Returns (acc, out): acc float64 [R, d_h] is the top-k sum before the final
    cast, out is that sum in the mode's output dtype (float32, or bf16 bits as uint16).
    """
    lib = _load()
    mode = int(inp.mode)
    rows_arr = None
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).ravel())
        nrows = rows_arr.size
    else:
        nrows = int(inp.T)
    acc = np.zeros((nrows, inp.d_h), np.float64)
    out = np.zeros((nrows, inp.d_h), np.float32 if mode == MODE_F32ACT else np.uint16)

    def c(a, dt):
        return None if a is None else np.ascontiguousarray(a, dtype=dt)

    xdt = {MODE_F32ACT: np.float32, MODE_BF16: np.uint16, MODE_FP8: np.uint8, MODE_MXFP8: np.uint8,
           MODE_INT8: np.int8}[mode]
    wdt = np.uint8 if mode in (MODE_FP8, MODE_MXFP8) else np.uint16
    sdt = np.uint8 if mode == MODE_MXFP8 else np.float32  # E8M0 bytes or fp32 scales (per token in INT8 mode)
    x = c(inp.x, xdt)
    xs = c(inp.x_scale, sdt)
    ids = c(inp.topk_ids, np.int32)
    tw = c(inp.topk_w, np.float32)
    w1 = c(inp.w1, wdt)
    w1s = c(inp.w1_scale, sdt)
    w2 = c(inp.w2, wdt)
    w2s = c(inp.w2_scale, sdt)
    flags = (MIRROR_H if mirror else 0) | (ACC64 if acc64 else 0)
    if getattr(inp, "activation", ACT_SWIGLU) == ACT_SWIGLU_CLAMPED:
        flags |= ACT_CLAMPED
    rc = lib.moe_oracle_forward(mode, int(inp.T), int(inp.E), int(inp.k), int(inp.d_h), int(inp.d_e),
                                _ptr(x), _ptr(xs), _ptr(ids), _ptr(tw), _ptr(w1), _ptr(w1s), _ptr(w2), _ptr(w2s),
                                flags, _ptr(rows_arr), nrows, _ptr(acc), _ptr(out))
    if rc != 0:
        raise ValueError(f"moe_oracle_forward failed with code {rc}")
    return acc, out


# ---------------------------------------------------------------- backward
def backward(inp, dout_bits, mirror: bool = True, acc64: bool = False):
    """Gradients of the layer (BF16 mode) for the output gradient ``dout_bits``
    (bf16 bits [T, d_h]): returns dx [T, d_h], dw1 [E, 2 d_e, d_h],
    dw2 [E, d_h, d_e], dtopk_w [T, k], all float32 (see moe_oracle_backward)."""
    lib = _load()
    if int(inp.mode) != MODE_BF16:
        raise ValueError("the backward oracle takes BF16 mode")
    T, E, k, d_h, d_e = int(inp.T), int(inp.E), int(inp.k), int(inp.d_h), int(inp.d_e)
    x = np.ascontiguousarray(inp.x, dtype=np.uint16)
    ids = np.ascontiguousarray(inp.topk_ids, dtype=np.int32)
    tw = np.ascontiguousarray(inp.topk_w, dtype=np.float32)
    w1 = np.ascontiguousarray(inp.w1, dtype=np.uint16)
    w2 = np.ascontiguousarray(inp.w2, dtype=np.uint16)
    dout = np.ascontiguousarray(dout_bits, dtype=np.uint16)
    dx = np.zeros((T, d_h), np.float32)
    dw1 = np.zeros((E, 2 * d_e, d_h), np.float32)
    dw2 = np.zeros((E, d_h, d_e), np.float32)
    dtw = np.zeros((T, k), np.float32)
    flags = (MIRROR_H if mirror else 0) | (ACC64 if acc64 else 0)
    rc = lib.moe_oracle_backward(MODE_BF16, T, E, k, d_h, d_e, _ptr(x), _ptr(ids), _ptr(tw), _ptr(w1), _ptr(w2),
                                 _ptr(dout), flags, _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(dtw))
    if rc != 0:
        raise ValueError(f"moe_oracle_backward failed with code {rc}")
    return dx, dw1, dw2, dtw
