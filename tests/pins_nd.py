"""Pins for the N-axis oracle (NA1D, NA3D, SASA on a zero-padded 2D map).

Each pin takes an ``oracle.OracleND`` (and, where it compares against the 2D
NA oracle, the pinned ``oracle.Oracle``) and raises AssertionError when the
N-axis oracle is wrong.  The checks come from what the pages and mathematics
fix, not from re-typing the oracle's loop:
  - NA equals self attention at the largest neighbourhood (CSDN translation,
    section 3.1), checked against dense matrices and torch's
    scaled_dot_product_attention (section 2.1, Eq. 1), in 1D and 3D;
  - windows are the brute-force k-nearest sets per axis (section 1; qiita NA
    border figure), checked through the box mean with Q = 0;
  - interior translation equivariance (paperlayer summary, appendix C);
  - the sign and axis order of the bias index (one-hot bias tables);
  - SASA is NA run on the input zero-padded by k/2 (CSDN page, section 3.1
    after Eq. 4, and section 3.2), checked against the separately pinned 2D NA
    oracle on an explicitly padded map, and by its closed form with Q = 0
    (padded zeros count in the softmax denominator).
"""
from __future__ import annotations

import itertools

import numpy as np
import torch

import oracle
from pins import _nearest_set

NA, SASA = oracle.NA, oracle.SASA


def _rng(seed):
    return np.random.default_rng(seed)


def _as6(a, shape6):
    return np.reshape(a, shape6)


# --------------------------------------------------------------------- 1D

def _na1d(orc, q, k, v, rpb, ks):
    return oracle.na1d_forward(q, k, v, rpb, ks, orc=orc)


def pin1d_span(orc, _orc2=None):
    """NA windows are the brute-force k-nearest sets; SASA windows are centred."""
    for k in (1, 3, 5, 7, 9, 13):
        for L in range(k, 3 * k + 2):
            for i in range(L):
                s = orc.window_start(i, k, L, NA)
                assert list(range(s, s + k)) == _nearest_set(i, k, L), (i, k, L)
                assert orc.window_start(i, k, L, SASA) == i - k // 2


def pin1d_self_attention(orc, _orc2=None):
    """k = L: dense softmax((Q K^T + B) / sqrt(d)) V with B[i, j] = rpb[j - i + L - 1]."""
    rng = _rng(11)
    B, heads, L, d = 2, 2, 9, 16
    q, k, v = (rng.standard_normal((B, heads, L, d)) for _ in range(3))
    rpb = rng.standard_normal((heads, 2 * L - 1))
    got = _na1d(orc, q, k, v, rpb, L)
    i = np.arange(L)
    rel = i[None, :] - i[:, None] + L - 1
    for h in range(heads):
        logits = (q[:, h] @ np.swapaxes(k[:, h], -1, -2) + rpb[h][rel]) / np.sqrt(d)
        w = np.exp(logits - logits.max(-1, keepdims=True))
        w /= w.sum(-1, keepdims=True)
        assert np.abs(got[:, h] - w @ v[:, h]).max() < 1e-12


def pin1d_sdpa(orc, _orc2=None):
    """k = L and no bias: torch's fp64 scaled-dot-product attention."""
    rng = _rng(12)
    q, k, v = (rng.standard_normal((1, 3, 11, 8)) for _ in range(3))
    got = _na1d(orc, q, k, v, None, 11)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.abs(got - want).max() < 1e-12


def pin1d_box(orc, _orc2=None):
    """Q = 0, no bias: the mean of V over the brute-force nearest set."""
    rng = _rng(13)
    L, k = 12, 5
    v = rng.standard_normal((1, 1, L, 4))
    z = np.zeros_like(v)
    got = _na1d(orc, z, rng.standard_normal(v.shape), v, None, k)
    for i in range(L):
        want = v[0, 0, _nearest_set(i, k, L)].mean(0)
        assert np.abs(got[0, 0, i] - want).max() < 1e-13


def pin1d_bias_offset(orc, _orc2=None):
    """A one-hot +200 bias at offset +1 selects V one position to the right."""
    rng = _rng(14)
    L, k = 10, 3
    q, kk, v = (rng.standard_normal((1, 1, L, 8)) for _ in range(3))
    rpb = np.zeros((1, 2 * k - 1))
    rpb[0, k - 1 + 1] = 200.0
    got = _na1d(orc, q * 0.01, kk, v, rpb, k)
    for i in range(L - 1):
        assert np.abs(got[0, 0, i] - v[0, 0, i + 1]).max() < 1e-6, i


def pin1d_translation(orc, _orc2=None):
    """Shifting the input shifts the output at unclamped positions (bitwise)."""
    rng = _rng(15)
    k, n, s = 5, 20, 3
    full = [rng.standard_normal((1, 2, 30, 8)) for _ in range(3)]
    rpb = rng.standard_normal((2, 2 * k - 1))
    a = _na1d(orc, *(t[:, :, :n] for t in full), rpb, k)
    b = _na1d(orc, *(t[:, :, s:s + n] for t in full), rpb, k)
    r = k // 2
    for i in range(r + s, n - r):
        assert np.array_equal(a[:, :, i], b[:, :, i - s])


# --------------------------------------------------------------------- 3D

def pin3d_self_attention(orc, _orc2=None):
    """k = D = H = W: dense softmax with the bias of every relative 3D offset."""
    rng = _rng(21)
    B, heads, n, d = 1, 2, 3, 8
    q, k, v = (rng.standard_normal((B, heads, n, n, n, d)) for _ in range(3))
    rpb = rng.standard_normal((heads, 2 * n - 1, 2 * n - 1, 2 * n - 1))
    got = oracle.na3d_forward(q, k, v, rpb, n, orc=orc)
    pos = np.array(list(itertools.product(range(n), repeat=3)))
    rel = pos[None, :, :] - pos[:, None, :] + n - 1
    for h in range(heads):
        qf, kf, vf = (t[0, h].reshape(-1, d) for t in (q, k, v))
        bias = rpb[h][rel[..., 0], rel[..., 1], rel[..., 2]]
        logits = (qf @ kf.T + bias) / np.sqrt(d)
        w = np.exp(logits - logits.max(-1, keepdims=True))
        w /= w.sum(-1, keepdims=True)
        assert np.abs(got[0, h].reshape(-1, d) - w @ vf).max() < 1e-12


def pin3d_sdpa(orc, _orc2=None):
    """k = D = H = W and no bias: torch's fp64 scaled-dot-product attention."""
    rng = _rng(22)
    n, d = 3, 16
    q, k, v = (rng.standard_normal((2, 1, n, n, n, d)) for _ in range(3))
    got = oracle.na3d_forward(q, k, v, None, n, orc=orc)
    flat = lambda t: torch.from_numpy(t.reshape(2, 1, n ** 3, d))
    want = torch.nn.functional.scaled_dot_product_attention(flat(q), flat(k), flat(v)).numpy()
    assert np.abs(got.reshape(2, 1, n ** 3, d) - want).max() < 1e-12


def pin3d_box(orc, _orc2=None):
    """Q = 0, no bias: the mean of V over the product of brute-force nearest
    sets (a non-cubic grid catches an axis mix-up)."""
    rng = _rng(23)
    D, H, W, k = 4, 5, 7, 3
    v = rng.standard_normal((1, 1, D, H, W, 4))
    got = oracle.na3d_forward(np.zeros_like(v), rng.standard_normal(v.shape), v, None, k, orc=orc)
    for z, y, x in itertools.product(range(D), range(H), range(W)):
        zs, ys, xs = _nearest_set(z, k, D), _nearest_set(y, k, H), _nearest_set(x, k, W)
        want = v[0, 0][np.ix_(zs, ys, xs)].reshape(-1, 4).mean(0)
        assert np.abs(got[0, 0, z, y, x] - want).max() < 1e-13


def pin3d_bias_offset(orc, _orc2=None):
    """One-hot +200 bias at (dz, dy, dx) = (+1, 0, 0), then (0, 0, +1): pins the
    axis order and sign of the 3D bias index."""
    rng = _rng(24)
    n, k = 5, 3
    q, kk, v = (rng.standard_normal((1, 1, n, n, n, 8)) for _ in range(3))
    for off, shift in (((1, 0, 0), (1, 0, 0)), ((0, 0, 1), (0, 0, 1))):
        rpb = np.zeros((1, 2 * k - 1, 2 * k - 1, 2 * k - 1))
        rpb[0, k - 1 + off[0], k - 1 + off[1], k - 1 + off[2]] = 200.0
        got = oracle.na3d_forward(q * 0.01, kk, v, rpb, k, orc=orc)
        for z, y, x in itertools.product(range(n - 1), repeat=3):
            src = (z + shift[0], y + shift[1], x + shift[2])
            assert np.abs(got[0, 0, z, y, x] - v[0, 0][src]).max() < 1e-6, (off, z, y, x)


def pin3d_reduces_to_2d(orc, orc2d):
    """A single-plane grid with a 1 x k x k window is NA2D: equal to the
    separately pinned 2D oracle."""
    rng = _rng(25)
    B, heads, H, W, d, k = 2, 2, 9, 11, 16, 5
    q, kk, v = (rng.standard_normal((B, heads, H, W, d)) for _ in range(3))
    rpb = rng.standard_normal((heads, 2 * k - 1, 2 * k - 1))
    sh = (B, heads, 1, H, W, d)
    got = orc.forward(_as6(q, sh), _as6(kk, sh), _as6(v, sh), rpb.reshape(heads, 1, 2 * k - 1, 2 * k - 1),
                      (1, k, k), NA)
    want = orc2d.na2d_forward(q, kk, v, rpb, k)
    assert np.abs(got.reshape(want.shape) - want).max() < 1e-13


def pin3d_translation(orc, _orc2=None):
    """Shifting the input along every axis shifts the output at unclamped positions."""
    rng = _rng(26)
    k, n, s = 3, 7, (1, 2, 1)
    full = [rng.standard_normal((1, 1, 10, 10, 10, 4)) for _ in range(3)]
    rpb = rng.standard_normal((1, 2 * k - 1, 2 * k - 1, 2 * k - 1))
    crop = lambda t, o: t[:, :, o[0]:o[0] + n, o[1]:o[1] + n, o[2]:o[2] + n]
    a = oracle.na3d_forward(*(crop(t, (0, 0, 0)) for t in full), rpb, k, orc=orc)
    b = oracle.na3d_forward(*(crop(t, s) for t in full), rpb, k, orc=orc)
    r = k // 2
    for z, y, x in itertools.product(range(n), repeat=3):
        zz, yy, xx = z - s[0], y - s[1], x - s[2]
        if min(z, y, x) >= r and max(z, y, x) <= n - 1 - r and min(zz, yy, xx) >= r and \
                max(zz, yy, xx) <= n - 1 - r:
            assert np.array_equal(a[:, :, z, y, x], b[:, :, zz, yy, xx])


# --------------------------------------------------------------------- SASA

def pin_sasa_zero_padding(orc, orc2d):
    """SASA equals NA on the input zero-padded by k/2, read at the original
    pixels (the pages' own construction), with the 2D oracle doing the NA."""
    rng = _rng(31)
    B, heads, H, W, d = 1, 2, 7, 9, 8
    for k in (3, 5, 7):
        r = k // 2
        q, kk, v = (rng.standard_normal((B, heads, H, W, d)) for _ in range(3))
        rpb = rng.standard_normal((heads, 2 * k - 1, 2 * k - 1)) * 0.5
        got = oracle.sasa2d_forward(q, kk, v, rpb, k, orc=orc)
        pad = lambda t: np.pad(t, ((0, 0), (0, 0), (r, r), (r, r), (0, 0)))
        want = orc2d.na2d_forward(pad(q), pad(kk), pad(v), rpb, k)[:, :, r:r + H, r:r + W]
        assert np.abs(got - want).max() < 1e-13, k


def pin_sasa_box(orc, _orc2=None):
    """Q = 0, no bias: every window position weighs 1/k^2, padded zeros
    included, so out = (sum of the in-map V of the centred window) / k^2."""
    rng = _rng(32)
    H, W, k = 6, 8, 5
    r = k // 2
    v = rng.standard_normal((1, 1, H, W, 4))
    got = oracle.sasa2d_forward(np.zeros_like(v), rng.standard_normal(v.shape), v, None, k, orc=orc)
    for y, x in itertools.product(range(H), range(W)):
        ys = [j for j in range(y - r, y + r + 1) if 0 <= j < H]
        xs = [j for j in range(x - r, x + r + 1) if 0 <= j < W]
        want = v[0, 0][np.ix_(ys, xs)].reshape(-1, 4).sum(0) / (k * k)
        assert np.abs(got[0, 0, y, x] - want).max() < 1e-13


def pin_sasa_interior(orc, orc2d):
    """Where the centred window lies inside the map, SASA and NA coincide."""
    rng = _rng(33)
    H, W, k = 10, 12, 5
    r = k // 2
    q, kk, v = (rng.standard_normal((1, 2, H, W, 8)) for _ in range(3))
    rpb = rng.standard_normal((2, 2 * k - 1, 2 * k - 1))
    a = oracle.sasa2d_forward(q, kk, v, rpb, k, orc=orc)
    b = orc2d.na2d_forward(q, kk, v, rpb, k)
    assert np.abs(a[:, :, r:H - r, r:W - r] - b[:, :, r:H - r, r:W - r]).max() < 1e-13
    assert np.abs(a[:, :, 0, 0] - b[:, :, 0, 0]).max() > 1e-3  # and differ at a corner


ALL_PINS_ND = [pin1d_span, pin1d_self_attention, pin1d_sdpa, pin1d_box, pin1d_bias_offset,
               pin1d_translation, pin3d_self_attention, pin3d_sdpa, pin3d_box, pin3d_bias_offset,
               pin3d_reduces_to_2d, pin3d_translation, pin_sasa_zero_padding, pin_sasa_box,
               pin_sasa_interior]
