"""Pins of the oracle's clamped activation (the GPT-OSS variant of SwiGLU that
the PipeLink page names as an independent activation owner, section 5.3; the
definition taken is the published GPT-OSS one): gate clamped above at 7, up
clamped to [-7, 7], h = gate * sigmoid(1.702 * gate) * (up + 1).

Pinned by a hand-worked example whose expected value is a closed form of
math-library calls, by the dense single-expert case written with torch fp64
ops, and by the routed layer against the all-expert dense computation.
Inputs are widened (x scaled by 4) so that about a tenth of the gate and up
values lie beyond the clamp."""
import math

import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import workloads as W

from test_oracle_forward import _deq_w, _deq_x, normwise

ALPHA, LIMIT = 1.702, 7.0


def clamped_act(g, u):
    g = g.clamp(max=LIMIT)
    u = u.clamp(min=-LIMIT, max=LIMIT)
    return g * torch.sigmoid(ALPHA * g) * (u + 1.0)


def _wide(mode, T=24, E=5, k=3, seed=3):
    return W.custom(T, E, k, 256, 256, mode, seed=seed, activation=W.ACT_SWIGLU_CLAMPED, x_gain=4.0)


def test_hand_worked_clamped_example(oracle):
    """One token, one expert, d_h = 1, d_e = 3, values exact in bf16:
    gate pre-activations (10, 2, -3) and up (20, -0.5, -9); the clamp turns
    them into (7, 2, -3) and (7, -0.5, -7); W2 = (1, 1, 1) sums the three."""
    w = W.MoEWorkload(name="hand_clamped", mode=W.MODE_F32ACT, T=1, E=1, k=1, d_h=1, d_e=3,
                      x=np.array([[1.0]], np.float32), topk_ids=np.array([[0]], np.int32),
                      topk_w=np.array([[1.0]], np.float32),
                      w1=W.to_bf16_bits(np.array([[[10.0], [2.0], [-3.0], [20.0], [-0.5], [-9.0]]], np.float32)),
                      w2=W.to_bf16_bits(np.array([[[1.0, 1.0, 1.0]]], np.float32)),
                      activation=W.ACT_SWIGLU_CLAMPED)
    acc, _ = oracle.forward(w, mirror=False, acc64=True)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    a32 = float(np.float32(ALPHA))  # the oracle's slope is an fp32 constant
    want = 7.0 * sig(a32 * 7.0) * 8.0 + 2.0 * sig(a32 * 2.0) * 0.5 + (-3.0) * sig(a32 * -3.0) * (-6.0)
    assert abs(acc[0, 0] - want) <= 1e-12 * abs(want)
    # the plain SwiGLU of the same inputs is far away (the clamp and the +1 matter)
    w.activation = W.ACT_SWIGLU
    acc_s, _ = oracle.forward(w, mirror=False, acc64=True)
    assert abs(acc_s[0, 0] - want) > 1.0


@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8])
def test_clamped_dense_single_expert(oracle, mode):
    w = _wide(mode, T=20, E=1, k=1)
    w.topk_w[:] = 1.0
    acc, _ = oracle.forward(w, mirror=False)
    x = _deq_x(w)
    W1 = _deq_w(w, w.w1, w.w1_scale)[0]
    W2 = _deq_w(w, w.w2, w.w2_scale)[0]
    g, u = x @ W1[:w.d_e].T, x @ W1[w.d_e:].T
    assert (g > LIMIT).double().mean() > 0.02 and (u.abs() > LIMIT).double().mean() > 0.02
    ref = clamped_act(g, u) @ W2.T
    assert normwise(acc, ref.numpy()) < 1e-5


@pytest.mark.parametrize("mode", [W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8])
def test_clamped_matches_dense_all_expert_moe(oracle, mode):
    w = _wide(mode)
    x = _deq_x(w)
    W1 = _deq_w(w, w.w1, w.w1_scale)
    W2 = _deq_w(w, w.w2, w.w2_scale)
    ids = torch.from_numpy(w.topk_ids.astype(np.int64))
    tw = torch.from_numpy(w.topk_w).double()
    ref = torch.zeros(w.T, w.d_h, dtype=torch.float64)
    for e in range(w.E):
        y = clamped_act(x @ W1[e, :w.d_e].T, x @ W1[e, w.d_e:].T) @ W2[e].T
        ref += (tw * (ids == e).double()).sum(dim=1)[:, None] * y
    acc, _ = oracle.forward(w, mirror=False)
    assert normwise(acc, ref.numpy()) < 1e-5


def test_clamped_fp32_agrees_with_fp64(oracle):
    w = _wide(W.MODE_BF16, T=16, E=6, k=2, seed=8)
    a32, _ = oracle.forward(w, mirror=False)
    a64, _ = oracle.forward(w, mirror=False, acc64=True)
    assert normwise(a32, a64) < 1e-5
