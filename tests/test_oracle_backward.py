"""Pins of the oracle's backward pass (BF16 mode, g, u and h recomputed).

The pages print no backward formulas or values.  The oracle's gradients are
pinned by: torch autograd through the dense all-expert fp64 MoE (an independent,
mechanical differentiation of the forward that the forward pins already
fix); central finite differences of the oracle's own forward in fp64 for dx;
the routing-weight gradient against forward calls with one-hot weights;
exact linearity in the output gradient; and the bf16 rounding points of the
mirrored variant."""
import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import workloads as W


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def _case(T=14, E=4, k=2, d_h=128, d_e=128, seed=5, dropped=True, dup=False):
    w = W.custom(T, E, k, d_h, d_e, W.MODE_BF16, seed=seed)
    ids = w.topk_ids.copy()
    if dropped:
        ids[2, 1] = -1
        ids[5, 0] = E + 1
    if dup:
        ids[3, :] = ids[3, 0]
    w.topk_ids = ids
    rng = np.random.default_rng(seed + 100)
    dout = W.to_bf16_bits(rng.standard_normal((T, d_h), dtype=np.float32))
    return w, dout


def _bf16(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16).double()


def _autograd(w, dout):
    x = _bf16(w.x).requires_grad_()
    W1 = _bf16(w.w1).requires_grad_()
    W2 = _bf16(w.w2).requires_grad_()
    tw = torch.from_numpy(w.topk_w).double().requires_grad_()
    ids = torch.from_numpy(w.topk_ids.astype(np.int64))
    out = torch.zeros(w.T, w.d_h, dtype=torch.float64)
    for e in range(w.E):
        g = x @ W1[e, :w.d_e].T
        u = x @ W1[e, w.d_e:].T
        y = (torch.nn.functional.silu(g) * u) @ W2[e].T
        coef = (tw * (ids == e).double()).sum(dim=1)
        out = out + coef[:, None] * y
    (out * _bf16(dout)).sum().backward()
    return x.grad.numpy(), W1.grad.numpy(), W2.grad.numpy(), tw.grad.numpy()


@pytest.mark.parametrize("dup", [False, True])
def test_matches_torch_autograd_of_dense_moe(oracle, dup):
    w, dout = _case(dup=dup)
    ref = _autograd(w, dout)
    got64 = oracle.backward(w, dout, mirror=False, acc64=True)
    got32 = oracle.backward(w, dout, mirror=False, acc64=False)
    for name, g64, g32, r in zip(("dx", "dw1", "dw2", "dtopk_w"), got64, got32, ref):
        assert normwise(g64, r) < 1e-6, name  # fp64 vs fp64 (float32 storage of the result)
        assert normwise(g32, r) < 2e-5, name


def test_dx_matches_central_differences_of_forward(oracle):
    """<dout, out(x)> differentiated numerically with the oracle's own fp64
    forward (x taken as fp32, which the bf16 inputs are exactly)."""
    w, dout = _case(T=6, E=3, k=2, seed=9)
    dx, _, _, _ = oracle.backward(w, dout, mirror=False, acc64=True)
    f = W.MoEWorkload(**{**w.__dict__})
    f.mode = W.MODE_F32ACT
    x0 = _bf16(w.x).float().numpy()
    d = _bf16(dout).numpy()
    rng = np.random.default_rng(3)
    for _ in range(3):
        v = rng.standard_normal(x0.shape).astype(np.float32)
        eps = np.float32(1e-3)
        xp, xm = (x0 + eps * v).astype(np.float32), (x0 - eps * v).astype(np.float32)
        f.x = xp
        yp, _ = oracle.forward(f, mirror=False, acc64=True)
        f.x = xm
        ym, _ = oracle.forward(f, mirror=False, acc64=True)
        fd = float(((yp - ym) * d).sum()) / float(eps * 2)
        an = float((dx.astype(np.float64) * ((xp - xm) / (2 * eps))).sum())
        assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), (fd, an)


def test_routing_weight_gradient_is_forward_of_one_hot_weights(oracle):
    """d out / d topk_w[t, j] is the expert output of slot j alone: the forward
    with weight 1 on slot j and 0 elsewhere, dotted with dout."""
    w, dout = _case(T=8, E=4, k=2, seed=12)
    _, _, _, dtw = oracle.backward(w, dout, mirror=False, acc64=True)
    d = _bf16(dout).numpy()
    for j in range(w.k):
        f = W.MoEWorkload(**{**w.__dict__})
        f.topk_w = np.zeros_like(w.topk_w)
        f.topk_w[:, j] = 1.0
        y, _ = oracle.forward(f, mirror=False, acc64=True)
        assert np.allclose(dtw[:, j], (y * d).sum(axis=1), rtol=1e-6, atol=1e-9)
    assert dtw[2, 1] == 0.0 and dtw[5, 0] == 0.0  # dropped assignments


def test_gradients_are_linear_in_dout(oracle):
    w, dout = _case(T=8, seed=14)
    g1 = oracle.backward(w, dout, mirror=False, acc64=True)
    d2 = W.to_bf16_bits(2.0 * _bf16(dout).float().numpy())
    g2 = oracle.backward(w, d2, mirror=False, acc64=True)
    for a, b in zip(g1, g2):
        assert np.array_equal(2 * a, b)


def test_mirrored_rounding_points(oracle):
    """The mirrored variant (h, dg, du and w*dout rounded to bf16, as the GPU's
    bf16 GEMMs take them) stays within bf16 rounding of the unrounded one and
    differs from it."""
    w, dout = _case(T=12, seed=15)
    m = oracle.backward(w, dout, mirror=True)
    p = oracle.backward(w, dout, mirror=False)
    for name, a, b in zip(("dx", "dw1", "dw2", "dtopk_w"), m, p):
        gap = normwise(a, b)
        assert 1e-5 < gap < 1e-2, (name, gap)
