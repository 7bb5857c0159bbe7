"""Pins for the NA2D gradient oracle.

Each pin takes an ``oracle.OracleBwd`` and raises AssertionError when its
gradients are wrong.  The references are independent of the gradient code:
  - central finite differences of the (separately pinned) forward oracle,
    for every element of q, k, v and the bias table, on maps whose windows
    are clamped at every border;
  - torch autograd (fp64) of dense softmax attention with the relative bias
    gathered per (query, key) pair, at k = H = W where NA is self attention
    (CSDN translation, section 3.1);
  - two closed forms: the bias gradient of every head sums to zero (each
    query's softmax gradient sums to zero over its window), and the value
    gradients of a map sum to the sum of the upstream gradients (each
    query's weights sum to one).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(seed, shape, ks, bias=True):
    rng = _rng(seed)
    q, k, v, g = (rng.standard_normal(shape) for _ in range(4))
    heads = shape[1]
    rpb = rng.standard_normal((heads, 2 * ks - 1, 2 * ks - 1)) * 0.7 if bias else None
    return q, k, v, rpb, g


def pin_bwd_finite_differences(orc):
    """Every gradient element against central differences of sum(g * NA2D)."""
    fwd = oracle.default()
    eps = 1e-5
    for seed, shape, ks in ((1, (1, 2, 5, 6, 3), 3), (2, (1, 1, 6, 7, 2), 5)):
        q, k, v, rpb, g = _problem(seed, shape, ks)
        grads = dict(zip(("q", "k", "v", "rpb"), orc.backward(q, k, v, rpb, g, ks)))
        base = dict(q=q, k=k, v=v, rpb=rpb)
        for name in ("q", "k", "v", "rpb"):
            arr = base[name]
            fd = np.empty_like(arr)
            for idx in np.ndindex(arr.shape):
                vals = []
                for sgn in (1.0, -1.0):
                    t = arr.copy()
                    t[idx] += sgn * eps
                    a = dict(base, **{name: t})
                    vals.append((g * fwd.na2d_forward(a["q"], a["k"], a["v"], a["rpb"], ks)).sum())
                fd[idx] = (vals[0] - vals[1]) / (2 * eps)
            err = np.abs(fd - grads[name]).max()
            assert err < 1e-7 * max(1.0, np.abs(fd).max()), (name, shape, ks, err)


def pin_bwd_self_attention_autograd(orc):
    """k = H = W: torch autograd of dense softmax((Q K^T + B) / sqrt(d)) V."""
    B, heads, n, d = 2, 2, 5, 8
    q, k, v, rpb, g = _problem(3, (B, heads, n, n, d), n)
    got = orc.backward(q, k, v, rpb, g, n)
    t = [torch.tensor(a, requires_grad=True) for a in (q, k, v, rpb)]
    iy, ix = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    iy, ix = iy.ravel(), ix.ravel()
    ry = torch.from_numpy(iy[None, :] - iy[:, None] + n - 1)
    rx = torch.from_numpy(ix[None, :] - ix[:, None] + n - 1)
    qf, kf, vf = (x.reshape(B, heads, n * n, d) for x in t[:3])
    bias = t[3][:, ry, rx]                                  # [heads, HW, HW]
    logits = (qf @ kf.transpose(-1, -2) + bias[None]) / np.sqrt(d)
    out = torch.softmax(logits, -1) @ vf
    (out * torch.from_numpy(g).reshape(B, heads, n * n, d)).sum().backward()
    for mine, ref in zip(got, t):
        assert np.abs(mine - ref.grad.numpy()).max() < 1e-12


def pin_bwd_bias_gradient_sums_to_zero(orc):
    """sum_j dL/ds_ij = 0 for every query, so each head's bias gradient sums to 0
    (while its entries do not vanish)."""
    q, k, v, rpb, g = _problem(4, (3, 2, 9, 8, 4), 5)
    drpb = orc.backward(q, k, v, rpb, g, 5)[3]
    assert np.abs(drpb.sum(axis=(1, 2))).max() < 1e-11
    assert np.abs(drpb).max() > 1e-2


def pin_bwd_value_gradient_sum(orc):
    """Each query's weights sum to one, so a map's value gradients sum to the
    sum of its upstream gradients."""
    q, k, v, rpb, g = _problem(5, (2, 2, 7, 9, 6), 3)
    dv = orc.backward(q, k, v, rpb, g, 3)[2]
    assert np.abs(dv.sum(axis=(2, 3)) - g.sum(axis=(2, 3))).max() < 1e-11


def pin_bwd_no_bias(orc):
    """Without a bias table the gradients of q, k, v equal those with an
    all-zero table, and no bias gradient is produced."""
    q, k, v, _, g = _problem(6, (1, 2, 7, 7, 4), 5, bias=False)
    a = orc.backward(q, k, v, None, g, 5)
    b = orc.backward(q, k, v, np.zeros((2, 9, 9)), g, 5)
    assert a[3] is None
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


ALL_PINS_BWD = [pin_bwd_finite_differences, pin_bwd_self_attention_autograd,
                pin_bwd_bias_gradient_sums_to_zero, pin_bwd_value_gradient_sum, pin_bwd_no_bias]
