"""Seeded synthetic inputs for the fused MoE layer.

This module only draws inputs; it holds none of the layer's arithmetic.  Both
the HIP path and the CPU oracle are fed from it, so it imports neither.

The pages measure on the authors' own per-expert token counts (the
tilelang.dataflow README, section 0 "Fused MoE vs MegaMoE", takes them from a
table that is not published).  The recipes below stand in for them with the
same model shapes (32 experts, top-2, DeepSeek 7168/2048 and Qwen 2048/768)
and skewed routing with hot and empty experts:

* ``tiny``       64 tokens, 8 experts, 256/128, fp32 x, bf16 weights, k distinct
                 uniform experts per token.
* ``qwen_bf16``  128 tokens, 2048/768, bf16; Zipf(1.1) over a seeded expert
                 permutation, k distinct experts drawn one after another.
* ``qwen_fp8``   1024 tokens, 2048/768, FP8 e4m3 with fp32 block scales;
                 Zipf(1.2) over 28 experts, the last 4 of the permutation empty.
* ``ds_fp8_<T>`` T in {128, 256, 512, 1024}, 7168/2048, FP8; exact counts: one
                 expert gets 40% of the assignments, 3 experts none, the other
                 28 share the rest by Zipf(1.0) (largest remainder, at least 1).
* ``ds_fp8_8192`` 8192 tokens, 7168/2048, FP8; two experts get 30% each, 16
                 experts none, 14 share the rest by Zipf(1.0).
* ``qwen_int8``, ``ds_int8_1024``: the Qwen-FP8 and 1024-token DeepSeek recipes
                 with tokens quantised to int8 (one fp32 scale per token,
                 s = amax/127, codes rounded to nearest even) and bf16 weights:
                 the token quantisation of the CUCo page's DeepSeek-V3 MoE
                 workload (its section 4, steps (1) and (3)).
* ``qwen_mxfp8``, ``ds_mxfp8_<T>`` (T in {1024, 8192}): the same recipes in MXFP8
                 (the MX variant the pages name for the MoE kernels of PipeLink
                 section 5.3): e4m3 codes with one E8M0 scale per 32 values along
                 the reduction dimension.

Weights are N(0, 1/fan_in); activations N(0, 1).  FP8 tensors are e4m3 codes
(OCP E4M3FN) with fp32 scales s = amax/448 per 128x128 weight block and per
token per 128 activation columns; the cast to e4m3 is torch's.  Combine
weights are the softmax of N(0,1) logits over the k chosen experts.  MXFP8
tensors: per 32 values along the reduction dimension, shared exponent
X = floor(log2(amax)) - 8, scale byte X + 127, codes = e4m3(v / 2^X) with the
quotient clamped to +-448 before torch's cast.
Randomness: ``numpy.random.default_rng([1000 + config_index, stream])`` with
streams 0 (x), 1 (W1), 2 (W2), 3 (routing), 4 (logits).
"""
from __future__ import annotations

import functools
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MODE_F32ACT = 0
MODE_BF16 = 1
MODE_FP8 = 2
MODE_MXFP8 = 3
MODE_INT8 = 4
ACT_SWIGLU = 0          # silu(gate) * up
ACT_SWIGLU_CLAMPED = 1  # clamped gate/up, gate * sigmoid(1.702 gate) * (up + 1)
QBLK = 128
MXBLK = 32

STREAM_X, STREAM_W1, STREAM_W2, STREAM_ROUTE, STREAM_LOGITS = range(5)


@dataclass
class MoEWorkload:
    name: str
    mode: int
    T: int
    E: int
    k: int
    d_h: int
    d_e: int
    x: np.ndarray
    topk_ids: np.ndarray
    topk_w: np.ndarray
    w1: np.ndarray
    w2: np.ndarray
    x_scale: Optional[np.ndarray] = None
    w1_scale: Optional[np.ndarray] = None
    w2_scale: Optional[np.ndarray] = None
    activation: int = 0  # ACT_SWIGLU or ACT_SWIGLU_CLAMPED
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.T * self.k

    def active_experts(self) -> int:
        ids = self.topk_ids.ravel()
        ids = ids[(ids >= 0) & (ids < self.E)]
        return int(np.unique(ids).size)

    def valid_assignments(self) -> int:
        ids = self.topk_ids.ravel()
        return int(((ids >= 0) & (ids < self.E)).sum())


def _rng(index: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([1000 + index, stream])


# ------------------------------------------------------------------ casts
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_rows(a: np.ndarray):
    """[R, C] float -> e4m3 codes [R, C], scales [R, C/128] (per row per 128 columns)."""
    R, C = a.shape
    blk = a.reshape(R, C // QBLK, QBLK)
    amax = np.abs(blk).max(axis=2).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = _to_e4m3_codes((blk / s[:, :, None]).reshape(R, C))
    return q, s


def quantize_blocks(a: np.ndarray):
    """[R, C] float -> e4m3 codes [R, C], scales [R/128, C/128] (per 128x128 block)."""
    R, C = a.shape
    blk = a.reshape(R // QBLK, QBLK, C // QBLK, QBLK)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = _to_e4m3_codes((blk / s[:, None, :, None]).reshape(R, C))
    return q, s


def quantize_mx(a: np.ndarray):
    """[R, C] float -> e4m3 codes [R, C], E8M0 scale bytes [R, C/32] (per row per 32 columns)."""
    R, C = a.shape
    blk = a.reshape(R, C // MXBLK, MXBLK).astype(np.float64)
    amax = np.abs(blk).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = f 2^ex, f in [0.5, 1)
    b = np.where(amax > 0, np.clip(ex - 1 - 8 + 127, 0, 254), 127).astype(np.int64)
    q = np.clip(blk / np.ldexp(1.0, b - 127)[:, :, None], -448.0, 448.0)
    return _to_e4m3_codes(q.reshape(R, C).astype(np.float32)), b.astype(np.uint8)


def quantize_int8_rows(a: np.ndarray):
    """[R, C] float -> int8 codes [R, C], fp32 scales [R] (one per row): s = amax/127
    (1 for an all-zero row), codes = x/s rounded to nearest even, clamped to +-127."""
    a = np.asarray(a, np.float32)
    amax = np.abs(a).max(axis=1).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(a / s[:, None]), -127, 127).astype(np.int8)
    return q, s


# ---------------------------------------------------------------- routing
def route_uniform(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def route_zipf(rng, T, E, k, s, n_empty):
    perm = rng.permutation(E)
    n_act = E - n_empty
    p = np.arange(1, n_act + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    ranks = np.stack([rng.choice(n_act, size=k, replace=False, p=p) for _ in range(T)])
    return perm[ranks].astype(np.int32)


def _largest_remainder(total, weights, floor):
    """Split ``total`` into integers proportional to ``weights``, each >= floor."""
    n = len(weights)
    base = np.full(n, floor, dtype=np.int64)
    rest = total - floor * n
    assert rest >= 0
    q = rest * np.asarray(weights, np.float64) / np.sum(weights)
    fl = np.floor(q).astype(np.int64)
    left = rest - int(fl.sum())
    order = np.argsort(-(q - fl), kind="stable")
    fl[order[:left]] += 1
    return base + fl


def route_exact(rng, T, E, k, hot_counts, n_empty, zipf_s):
    """Exact per-expert counts, then the fold layout: the expert-sorted multiset
    of T*k ids is cut into k columns of T entries, token t takes entries t, t+T,
    ...; entries of one token are distinct because no count exceeds T.  Tokens and
    slot order are then shuffled."""
    n = T * k
    perm = rng.permutation(E)
    counts = np.zeros(E, np.int64)
    for i, c in enumerate(hot_counts):
        counts[perm[i]] = c
    n_rest = E - len(hot_counts) - n_empty
    rest = n - int(sum(hot_counts))
    w = np.arange(1, n_rest + 1, dtype=np.float64) ** (-zipf_s)
    counts[perm[len(hot_counts):len(hot_counts) + n_rest]] = _largest_remainder(rest, w, 1)
    assert counts.sum() == n and counts.max() <= T
    flat = np.repeat(np.arange(E), counts)
    ids = flat.reshape(k, T).T.copy()
    ids = ids[rng.permutation(T)]
    for t in range(T):
        ids[t] = ids[t][rng.permutation(k)]
    return ids.astype(np.int32)


# ---------------------------------------------------------------- configs
CONFIGS = {
    "tiny": dict(index=0, T=64, E=8, k=2, d_h=256, d_e=128, mode=MODE_F32ACT, routing=("uniform",)),
    "qwen_bf16": dict(index=1, T=128, E=32, k=2, d_h=2048, d_e=768, mode=MODE_BF16, routing=("zipf", 1.1, 0)),
    "qwen_fp8": dict(index=2, T=1024, E=32, k=2, d_h=2048, d_e=768, mode=MODE_FP8, routing=("zipf", 1.2, 4)),
}
for _T in (128, 256, 512, 1024):
    CONFIGS[f"ds_fp8_{_T}"] = dict(index=3, T=_T, E=32, k=2, d_h=7168, d_e=2048, mode=MODE_FP8,
                                   routing=("exact", (int(round(0.4 * _T * 2)),), 3, 1.0))
CONFIGS["ds_fp8_8192"] = dict(index=4, T=8192, E=32, k=2, d_h=7168, d_e=2048, mode=MODE_FP8,
                              routing=("exact", (4915, 4915), 16, 1.0))
CONFIGS["qwen_mxfp8"] = dict(CONFIGS["qwen_fp8"], index=5, mode=MODE_MXFP8)
CONFIGS["ds_mxfp8_1024"] = dict(CONFIGS["ds_fp8_1024"], index=6, mode=MODE_MXFP8)
CONFIGS["ds_mxfp8_8192"] = dict(CONFIGS["ds_fp8_8192"], index=7, mode=MODE_MXFP8)
CONFIGS["qwen_int8"] = dict(CONFIGS["qwen_fp8"], index=8, mode=MODE_INT8)
CONFIGS["ds_int8_1024"] = dict(CONFIGS["ds_fp8_1024"], index=9, mode=MODE_INT8)


def make_routing(index, T, E, k, routing):
    rng = _rng(index, STREAM_ROUTE)
    kind = routing[0]
    if kind == "uniform":
        return route_uniform(rng, T, E, k)
    if kind == "zipf":
        return route_zipf(rng, T, E, k, routing[1], routing[2])
    if kind == "exact":
        return route_exact(rng, T, E, k, routing[1], routing[2], routing[3])
    raise ValueError(kind)


@functools.lru_cache(maxsize=2)
def _weights(index, E, d_h, d_e, mode):
    """Expert weights of one recipe; shared by every token count of that recipe."""
    r1, r2 = _rng(index, STREAM_W1), _rng(index, STREAM_W2)
    s1, s2 = np.float32(1.0 / np.sqrt(d_h)), np.float32(1.0 / np.sqrt(d_e))
    if mode == MODE_FP8:
        w1 = np.empty((E, 2 * d_e, d_h), np.uint8)
        w2 = np.empty((E, d_h, d_e), np.uint8)
        w1_scale = np.empty((E, 2 * d_e // QBLK, d_h // QBLK), np.float32)
        w2_scale = np.empty((E, d_h // QBLK, d_e // QBLK), np.float32)
        for e in range(E):
            w1[e], w1_scale[e] = quantize_blocks(r1.standard_normal((2 * d_e, d_h), dtype=np.float32) * s1)
        for e in range(E):
            w2[e], w2_scale[e] = quantize_blocks(r2.standard_normal((d_h, d_e), dtype=np.float32) * s2)
        return w1, w2, w1_scale, w2_scale
    if mode == MODE_MXFP8:
        w1 = np.empty((E, 2 * d_e, d_h), np.uint8)
        w2 = np.empty((E, d_h, d_e), np.uint8)
        w1_scale = np.empty((E, 2 * d_e, d_h // MXBLK), np.uint8)
        w2_scale = np.empty((E, d_h, d_e // MXBLK), np.uint8)
        for e in range(E):
            w1[e], w1_scale[e] = quantize_mx(r1.standard_normal((2 * d_e, d_h), dtype=np.float32) * s1)
        for e in range(E):
            w2[e], w2_scale[e] = quantize_mx(r2.standard_normal((d_h, d_e), dtype=np.float32) * s2)
        return w1, w2, w1_scale, w2_scale
    w1 = np.stack([to_bf16_bits(r1.standard_normal((2 * d_e, d_h), dtype=np.float32) * s1) for _ in range(E)])
    w2 = np.stack([to_bf16_bits(r2.standard_normal((d_h, d_e), dtype=np.float32) * s2) for _ in range(E)])
    return w1, w2, None, None


def make_workload(name, index, T, E, k, d_h, d_e, mode, routing, topk_ids=None, activation=0,
                  x_gain=1.0) -> MoEWorkload:
    if mode in (MODE_FP8, MODE_MXFP8):
        assert d_h % QBLK == 0 and d_e % QBLK == 0
    ids = make_routing(index, T, E, k, routing) if topk_ids is None else np.asarray(topk_ids, np.int32)
    lg = _rng(index, STREAM_LOGITS).standard_normal((T, k))
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    tw = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    xf = _rng(index, STREAM_X).standard_normal((T, d_h), dtype=np.float32)
    if x_gain != 1.0:  # wider pre-activations (reach the clamp of the clamped activation)
        xf = xf * np.float32(x_gain)
    w1, w2, w1_scale, w2_scale = _weights(index, E, d_h, d_e, mode)
    x_scale = None
    if mode == MODE_FP8:
        x, x_scale = quantize_rows(xf)
    elif mode == MODE_INT8:
        x, x_scale = quantize_int8_rows(xf)
    elif mode == MODE_MXFP8:
        x, x_scale = quantize_mx(xf)
    else:
        x = xf if mode == MODE_F32ACT else to_bf16_bits(xf)
    return MoEWorkload(name=name, mode=mode, T=T, E=E, k=k, d_h=d_h, d_e=d_e, x=x, topk_ids=ids, topk_w=tw,
                       w1=w1, w2=w2, x_scale=x_scale, w1_scale=w1_scale, w2_scale=w2_scale,
                       activation=activation, meta={"index": index, "routing": routing, "x_gain": x_gain})


@functools.lru_cache(maxsize=2)
def config(name: str) -> MoEWorkload:
    c = dict(CONFIGS[name])
    return make_workload(name=name, **c)


def custom(T, E, k, d_h, d_e, mode, seed=7, routing=("uniform",), topk_ids=None, activation=0,
           x_gain=1.0) -> MoEWorkload:
    """Any shape, for parity sweeps and edge cases (seed selects the streams)."""
    return make_workload(name=f"custom_T{T}_E{E}_k{k}_{d_h}x{d_e}_m{mode}_s{seed}_a{activation}_g{x_gain}",
                         index=seed, T=T, E=E, k=k, d_h=d_h, d_e=d_e, mode=mode, routing=routing,
                         topk_ids=topk_ids, activation=activation, x_gain=x_gain)


def flops(w: MoEWorkload) -> float:
    """Algorithmic FLOPs: 6 d_h d_e per valid assignment (padding, SwiGLU, combine excluded)."""
    return 6.0 * w.d_h * w.d_e * w.valid_assignments()


def algorithmic_bytes(w: MoEWorkload) -> float:
    """Bytes the layer must move once: the active experts' weights (+scales), x (+scales),
    out, and the routing ids and weights."""
    a = w.active_experts()
    wb = 1 if w.mode in (MODE_FP8, MODE_MXFP8) else 2
    per_expert = 3 * w.d_h * w.d_e * wb
    if w.mode == MODE_FP8:
        per_expert += 4 * (2 * w.d_e // QBLK) * (w.d_h // QBLK) + 4 * (w.d_h // QBLK) * (w.d_e // QBLK)
    if w.mode == MODE_MXFP8:
        per_expert += 3 * w.d_h * w.d_e // MXBLK
    xb = {MODE_F32ACT: 4, MODE_BF16: 2, MODE_FP8: 1, MODE_MXFP8: 1, MODE_INT8: 1}[w.mode]
    x_bytes = w.T * w.d_h * xb + (w.T * (w.d_h // QBLK) * 4 if w.mode == MODE_FP8 else 0)
    if w.mode == MODE_INT8:  # one fp32 scale per token
        x_bytes += w.T * 4
    if w.mode == MODE_MXFP8:
        x_bytes += w.T * (w.d_h // MXBLK)
    out_bytes = w.T * w.d_h * (4 if w.mode == MODE_F32ACT else 2)
    return float(a * per_expert + x_bytes + out_bytes + w.T * w.k * 8)
