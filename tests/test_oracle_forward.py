"""Pins of the oracle's layer output.

The pages print no worked example for the MoE layer, so the oracle's forward is
pinned by: the textbook dense computation written with torch fp64 library
matmuls over *all* experts (no routing, no permutation), the special case
top_k=1 / weight 1 reducing to one dense SwiGLU FFN, a hand-worked closed-form
example, fp32-vs-fp64 agreement, exact symmetries, and the intermediate's
rounding point checked against torch's casts.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


# ----------------------------------------------------- torch fp64 textbook MoE
def _deq_x(w):
    if w.mode == W.MODE_F32ACT:
        return torch.from_numpy(w.x).double()
    if w.mode == W.MODE_INT8:  # int8 code * the token's fp32 scale
        return torch.from_numpy(w.x.astype(np.int64)).double() * torch.from_numpy(w.x_scale).double()[:, None]
    if w.mode == W.MODE_BF16:
        return torch.from_numpy(w.x.view(np.int16)).view(torch.bfloat16).double()
    q = torch.from_numpy(w.x).view(torch.float8_e4m3fn).double()
    if w.mode == W.MODE_MXFP8:  # E8M0 byte b per token per 32 columns: 2^(b - 127)
        e = torch.from_numpy(w.x_scale.astype(np.int64) - 127).repeat_interleave(32, dim=1)
        return torch.ldexp(q, e)
    s = torch.from_numpy(w.x_scale).double().repeat_interleave(128, dim=1)
    return q * s


def _deq_w(w, a, s):
    if w.mode == W.MODE_MXFP8:  # [E, rows, cols/32] bytes, one per row per 32 along K
        q = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
        return torch.ldexp(q, torch.from_numpy(s.astype(np.int64) - 127).repeat_interleave(32, dim=2))
    if w.mode != W.MODE_FP8:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double()
    q = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    ss = torch.from_numpy(s).double().repeat_interleave(128, dim=1).repeat_interleave(128, dim=2)
    return q * ss


def _torch_h_round(a, mode):
    if mode in (W.MODE_F32ACT, W.MODE_BF16, W.MODE_INT8):
        return a.float().to(torch.bfloat16).double()
    if mode == W.MODE_MXFP8:
        # per row per 32: X = floor(log2(amax)) - 8 (from frexp's exponent), values / 2^X
        # clamped to the e4m3 range and cast by torch, times 2^X
        T, D = a.shape
        blk = a.reshape(T, D // 32, 32)
        amax = blk.abs().amax(dim=2, keepdim=True)
        _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
        x = torch.where(amax > 0, ex - 1 - 8, torch.zeros_like(ex)).clamp(-127, 127)
        q = torch.ldexp(blk, -x).clamp(-448, 448).float().to(torch.float8_e4m3fn).double()
        return torch.ldexp(q, x).reshape(T, D)
    T, D = a.shape
    blk = a.float().reshape(T, D // 128, 128)
    amax = blk.abs().amax(dim=2, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s).to(torch.float8_e4m3fn).float()
    return (q * s).reshape(T, D).double()


def dense_moe(w, h_round=False):
    """out[t] = sum_j w[t,j] FFN_{ids[t,j]}(x[t]), every expert run over every token."""
    x = _deq_x(w)
    W1 = _deq_w(w, w.w1, w.w1_scale)
    W2 = _deq_w(w, w.w2, w.w2_scale)
    ids = torch.from_numpy(w.topk_ids.astype(np.int64))
    tw = torch.from_numpy(w.topk_w).double()
    out = torch.zeros(w.T, w.d_h, dtype=torch.float64)
    for e in range(w.E):
        g = x @ W1[e, :w.d_e].T
        u = x @ W1[e, w.d_e:].T
        a = torch.nn.functional.silu(g) * u
        if h_round:
            a = _torch_h_round(a, w.mode)
        y = a @ W2[e].T
        coef = (tw * (ids == e).double()).sum(dim=1)
        out += coef[:, None] * y
    return out.numpy()


def _small(mode, T=24, E=5, k=3, d_h=256, d_e=256, seed=3, ids=None):
    routing = ("uniform",)
    return W.custom(T, E, k, d_h, d_e, mode, seed=seed, routing=routing, topk_ids=ids)


MODES = [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8]


@pytest.mark.parametrize("mode", MODES)
def test_dense_special_case_single_expert(oracle, mode):
    """top_k=1, weight 1, one expert: the layer is one dense SwiGLU FFN."""
    w = _small(mode, T=20, E=1, k=1)
    w.topk_w[:] = 1.0
    acc, _ = oracle.forward(w, mirror=False)
    x = _deq_x(w)
    W1 = _deq_w(w, w.w1, w.w1_scale)[0]
    W2 = _deq_w(w, w.w2, w.w2_scale)[0]
    ref = (torch.nn.functional.silu(x @ W1[:w.d_e].T) * (x @ W1[w.d_e:].T)) @ W2.T
    assert normwise(acc, ref.numpy()) < 1e-5


@pytest.mark.parametrize("mode", MODES)
def test_top1_unit_weight_is_per_token_expert_ffn(oracle, mode):
    w = _small(mode, T=30, E=6, k=1)
    w.topk_w[:] = 1.0
    acc, _ = oracle.forward(w, mirror=False)
    x = _deq_x(w)
    W1 = _deq_w(w, w.w1, w.w1_scale)
    W2 = _deq_w(w, w.w2, w.w2_scale)
    for t in range(w.T):
        e = int(w.topk_ids[t, 0])
        a = torch.nn.functional.silu(W1[e, :w.d_e] @ x[t]) * (W1[e, w.d_e:] @ x[t])
        assert normwise(acc[t], (W2[e] @ a).numpy()) < 1e-5


@pytest.mark.parametrize("mode", MODES)
def test_matches_dense_all_expert_moe(oracle, mode):
    """Routed oracle vs the textbook computation that runs every expert on every token."""
    ids = None
    w = _small(mode)
    ids = w.topk_ids.copy()
    ids[3, 1] = -1  # dropped assignment
    ids[7, 0] = w.E + 2  # dropped assignment
    w.topk_ids = ids
    acc, _ = oracle.forward(w, mirror=False)
    ref = dense_moe(w)
    assert normwise(acc, ref) < 1e-5


@pytest.mark.parametrize("mode", MODES)
def test_rounding_point_of_intermediate(oracle, mode):
    """Mirrored variant vs torch: intermediate rounded by torch's bf16 cast or
    the per-row-per-128 e4m3 requantisation.  The fp32/fp64 gap can flip a few
    rounding decisions, hence the small tolerance; the mirrored and pure
    variants must differ by more than that."""
    w = _small(mode, T=16)
    acc_m, _ = oracle.forward(w, mirror=True)
    acc_p, _ = oracle.forward(w, mirror=False)
    ref_m = dense_moe(w, h_round=True)
    assert normwise(acc_m, ref_m) < 2e-3
    gap = normwise(acc_p, acc_m)
    # MX requantisation saturates the largest values of a block (the shared
    # exponent leaves them in [256, 512) against an e4m3 maximum of 448)
    lo_hi = {W.MODE_FP8: (1e-3, 3e-2), W.MODE_MXFP8: (1e-3, 6e-2)}.get(mode, (1e-4, 5e-3))
    assert lo_hi[1] > gap > lo_hi[0]


@pytest.mark.parametrize("name", ["tiny"])
def test_fp32_agrees_with_fp64(oracle, name):
    w = W.config(name)
    a32, _ = oracle.forward(w, mirror=False)
    a64, _ = oracle.forward(w, mirror=False, acc64=True)
    assert normwise(a32, a64) < 1e-5


@pytest.mark.parametrize("mode", [W.MODE_BF16, W.MODE_FP8])
def test_fp32_agrees_with_fp64_larger_k(oracle, mode):
    w = W.custom(16, 8, 4, 512, 256, mode, seed=12)
    a32, _ = oracle.forward(w, mirror=False)
    a64, _ = oracle.forward(w, mirror=False, acc64=True)
    assert normwise(a32, a64) < 1e-5


def test_hand_worked_example(oracle):
    with open(os.path.join(GOLD, "hand_worked_moe.json")) as f:
        g = json.load(f)
    T, E, k, d_h, d_e = g["T"], g["E"], g["k"], g["d_h"], g["d_e"]
    w = W.MoEWorkload(name="hand", mode=W.MODE_F32ACT, T=T, E=E, k=k, d_h=d_h, d_e=d_e,
                      x=np.array(g["x"], np.float32), topk_ids=np.array(g["topk_ids"], np.int32),
                      topk_w=np.array(g["topk_w"], np.float32),
                      w1=W.to_bf16_bits(np.array(g["w1"], np.float32)),
                      w2=W.to_bf16_bits(np.array(g["w2"], np.float32)))
    acc, out = oracle.forward(w, mirror=False, acc64=True)
    # closed forms restated from the fixture: silu(v) = v / (1 + e^-v)
    silu = lambda v: v / (1.0 + math.exp(-v))
    exp = [[eval(s, {"silu": silu}) for s in row] for row in g["expected_closed_form"]]
    assert np.allclose(acc, np.array(exp), rtol=1e-12, atol=1e-12)
    assert np.allclose(acc, np.array(g["expected"]), rtol=1e-12, atol=1e-12)


def test_symmetries_are_exact(oracle):
    w = _small(W.MODE_F32ACT, T=12, E=4, k=2)
    _, base = oracle.forward(w)
    # relabel experts: permute weights along E and remap ids
    perm = np.array([2, 0, 3, 1])
    inv = np.argsort(perm)
    w2 = W.MoEWorkload(**{**w.__dict__})
    w2.w1, w2.w2 = w.w1[perm], w.w2[perm]
    w2.topk_ids = inv[w.topk_ids].astype(np.int32)
    _, o = oracle.forward(w2)
    assert np.array_equal(o, base)
    # permute tokens
    tp = np.random.default_rng(0).permutation(w.T)
    w3 = W.MoEWorkload(**{**w.__dict__})
    w3.x, w3.topk_ids, w3.topk_w = w.x[tp], w.topk_ids[tp], w.topk_w[tp]
    _, o = oracle.forward(w3)
    assert np.array_equal(o, base[tp])
    # swap the two slots of every token (k=2: a+b = b+a exactly)
    w4 = W.MoEWorkload(**{**w.__dict__})
    w4.topk_ids, w4.topk_w = w.topk_ids[:, ::-1].copy(), w.topk_w[:, ::-1].copy()
    _, o = oracle.forward(w4)
    assert np.array_equal(o, base)
    # doubling all routing weights doubles the fp32 output exactly
    w5 = W.MoEWorkload(**{**w.__dict__})
    w5.topk_w = w.topk_w * np.float32(2)
    _, o = oracle.forward(w5)
    assert np.array_equal(o, base * np.float32(2))


def test_row_subset_equals_full(oracle):
    w = _small(W.MODE_FP8, T=10)
    acc, out = oracle.forward(w)
    rows = [7, 0, 3]
    acc_s, out_s = oracle.forward(w, rows=rows)
    assert np.array_equal(acc_s, acc[rows]) and np.array_equal(out_s, out[rows])


def test_final_cast_is_bf16_rne_of_sum(oracle):
    w = _small(W.MODE_BF16, T=8)
    acc, out = oracle.forward(w)
    ref = torch.from_numpy(acc.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_all_dropped_token_is_zero(oracle):
    w = _small(W.MODE_BF16, T=6, E=3, k=2)
    ids = w.topk_ids.copy()
    ids[2, :] = -7
    w.topk_ids = ids
    acc, out = oracle.forward(w)
    assert np.all(acc[2] == 0) and np.all(out[2] == 0)


def test_mxfp8_with_power_of_two_blocks_equals_fp8(oracle):
    """MXFP8 whose scale bytes are constant over each 128x128 weight block and each
    128 activation columns is the FP8 block-scaled layer with scales 2^(b-127):
    both modes of the oracle must agree exactly (pins the MX scale indexing,
    per row and per 32 along the reduction dimension, to the pinned FP8 path)."""
    rng = np.random.default_rng(11)
    T, E, k, d_h, d_e = 12, 3, 2, 256, 256
    w = _small(W.MODE_FP8, T=T, E=E, k=k, d_h=d_h, d_e=d_e, seed=5)
    ex1 = rng.integers(-3, 4, size=w.w1_scale.shape)
    ex2 = rng.integers(-3, 4, size=w.w2_scale.shape)
    exx = rng.integers(-3, 4, size=w.x_scale.shape)
    w.w1_scale = np.ldexp(1.0, ex1).astype(np.float32)
    w.w2_scale = np.ldexp(1.0, ex2).astype(np.float32)
    w.x_scale = np.ldexp(1.0, exx).astype(np.float32)
    acc_fp8, _ = oracle.forward(w, mirror=False)
    m = W.custom(T, E, k, d_h, d_e, W.MODE_MXFP8, seed=5)
    m.x, m.w1, m.w2, m.topk_ids, m.topk_w = w.x, w.w1, w.w2, w.topk_ids, w.topk_w
    m.x_scale = (exx + 127).astype(np.uint8).repeat(4, axis=1)                      # [T, d_h/32]
    m.w1_scale = (ex1 + 127).astype(np.uint8).repeat(128, axis=1).repeat(4, axis=2)  # [E, 2 d_e, d_h/32]
    m.w2_scale = (ex2 + 127).astype(np.uint8).repeat(128, axis=1).repeat(4, axis=2)  # [E, d_h, d_e/32]
    acc_mx, _ = oracle.forward(m, mirror=False)
    assert np.array_equal(acc_fp8, acc_mx)


def test_int8_with_unit_scales_equals_bf16(oracle):
    """INT8 tokens whose scales are all 1 are the integers themselves, which
    bf16 holds exactly: the INT8 mode must give, bit for bit, the BF16 mode's
    output on x = bf16(code) with the same bf16 weights (pins the int8 decode,
    signs included, to the pinned BF16 path)."""
    w = _small(W.MODE_INT8, T=14, E=4, k=2, seed=8)
    w.x_scale = np.ones_like(w.x_scale)
    acc_i8, out_i8 = oracle.forward(w)
    b = W.MoEWorkload(**{**w.__dict__})
    b.mode = W.MODE_BF16
    b.x = W.to_bf16_bits(w.x.astype(np.float32))
    b.x_scale = None
    acc_bf, out_bf = oracle.forward(b)
    assert np.array_equal(acc_i8, acc_bf) and np.array_equal(out_i8, out_bf)
    assert (w.x < 0).any() and ((w.x == 127).any() or (w.x == -127).any())


def test_int8_scale_is_per_token(oracle):
    """Scaling one token's int8 scale by 2 (an exact change of its dequantised
    row) changes that token's output row and no other."""
    w = _small(W.MODE_INT8, T=10, E=4, k=2, seed=9)
    _, base = oracle.forward(w)
    w2 = W.MoEWorkload(**{**w.__dict__})
    w2.x_scale = w.x_scale.copy()
    w2.x_scale[4] *= np.float32(2)
    _, o = oracle.forward(w2)
    changed = np.nonzero((o != base).any(axis=1))[0].tolist()
    assert changed == [4]
