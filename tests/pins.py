"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when that oracle
is wrong.  None of them re-types the oracle's own loop: they use the special
cases the pages state (NA equals self attention at the largest neighbourhood,
translational equivariance away from the borders, the same span at the
borders), closed forms (box mean, identity), a library routine (torch's
scaled-dot-product attention) and brute force on tiny inputs (k-nearest sets
by sorting distances).

Sources: "Neighborhood Attention Transformer" (CSDN translation, sections 1,
2.1 Eq. 1, 3.1 Eq. 2-4, 3.2), the paperlayer summary of arXiv 2204.07143v5
(appendix C, "Notes on translational equivariance"), and the qiita article
"NAT: スライディングウィンドウアテンションの革新" (NA border figure).
"""
from __future__ import annotations

import numpy as np
import torch


def _rng(seed):
    return np.random.default_rng(seed)


def _nearest_set(i: int, k: int, L: int):
    """The k indices of [0, L) nearest to i, by sorting |j - i| (brute force)."""
    order = sorted(range(L), key=lambda j: (abs(j - i), j))
    chosen = sorted(order[:k])
    # the k-th and (k+1)-th distances differ for odd k, so the set is unique
    if k < L:
        assert abs(order[k - 1] - i) != abs(order[k] - i), (i, k, L)
    return chosen


def pin_span(orc):
    """Every query keeps exactly k in-bounds neighbours per axis, equal to the
    brute-force k-nearest set, and windows slide by 0 or 1 (section 1, 3.1;
    qiita border figure)."""
    for k in (1, 3, 5, 7, 9, 13, 21):
        for L in range(k, 4 * k + 1):
            prev = None
            for i in range(L):
                s = orc.window_start(i, k, L)
                assert 0 <= s and s + k <= L, (k, L, i, s)
                assert i >= s and i < s + k, "query outside its own window"
                assert list(range(s, s + k)) == _nearest_set(i, k, L), (k, L, i, s)
                if prev is not None:
                    assert s - prev in (0, 1), (k, L, i)
                prev = s


def _dense_bias(rpb_h, H, W, k):
    """Dense [HW, HW] bias for k = H = W from relative offsets (meshgrid form)."""
    ys, xs = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ys, xs = ys.ravel(), xs.ravel()
    dy = ys[None, :] - ys[:, None]          # key row - query row
    dx = xs[None, :] - xs[:, None]
    return rpb_h[dy + (k - 1), dx + (k - 1)]


def _full_sa(q, k_, v, rpb, ksize):
    """softmax((Q K^T + B) / sqrt(d)) V over the whole map, as dense matrices."""
    B, heads, H, W, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        for h in range(heads):
            Q = q[b, h].reshape(H * W, d)
            K = k_[b, h].reshape(H * W, d)
            V = v[b, h].reshape(H * W, d)
            S = Q @ K.T
            if rpb is not None:
                S = S + _dense_bias(rpb[h], H, W, ksize)
            S = S / np.sqrt(d)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P = P / P.sum(axis=1, keepdims=True)
            out[b, h] = (P @ V).reshape(H, W, d)
    return out


def pin_self_attention(orc):
    """k = H = W: NA equals full self attention with the same bias (section 3.1:
    NA approaches SA as k grows and equals it at the largest neighbourhood)."""
    r = _rng(11)
    for (B, heads, n, d) in [(1, 1, 7, 32), (2, 3, 5, 8), (1, 2, 3, 4), (1, 1, 1, 5)]:
        q = r.standard_normal((B, heads, n, n, d))
        k = r.standard_normal((B, heads, n, n, d))
        v = r.standard_normal((B, heads, n, n, d))
        rpb = r.standard_normal((heads, 2 * n - 1, 2 * n - 1))   # strong bias: N(0, 1)
        got = orc.na2d_forward(q, k, v, rpb, n)
        want = _full_sa(q, k, v, rpb, n)
        err = np.abs(got - want).max()
        assert err <= 1e-12, ("SA equality", n, err)


def pin_sdpa(orc):
    """k = H = W and no bias: torch's fp64 scaled-dot-product attention, i.e.
    softmax(Q K^T / sqrt(d)) V (section 2.1, Eq. 1)."""
    r = _rng(12)
    for (B, heads, n, d) in [(2, 2, 7, 32), (1, 1, 5, 16)]:
        q = r.standard_normal((B, heads, n, n, d)) * 2.0
        k = r.standard_normal((B, heads, n, n, d))
        v = r.standard_normal((B, heads, n, n, d))
        got = orc.na2d_forward(q, k, v, None, n)
        zero = orc.na2d_forward(q, k, v, np.zeros((heads, 2 * n - 1, 2 * n - 1)), n)
        tq = torch.from_numpy(q).reshape(B, heads, n * n, d)
        tk = torch.from_numpy(k).reshape(B, heads, n * n, d)
        tv = torch.from_numpy(v).reshape(B, heads, n * n, d)
        want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
        want = want.reshape(B, heads, n, n, d).numpy()
        assert np.abs(got - want).max() <= 1e-12, ("SDPA", n, np.abs(got - want).max())
        assert np.abs(zero - want).max() <= 1e-12, ("SDPA zero bias", n)


def pin_translation(orc):
    """Interior queries are translation-equivariant: shifting the input shifts
    the output (paperlayer summary, appendix C; qiita "translational
    equivariance").  Compared bitwise: the same neighbours in the same order."""
    r = _rng(13)
    d, ksize, big, crop = 8, 5, 40, 24
    heads = 2
    q = r.standard_normal((1, heads, big, big, d))
    k = r.standard_normal((1, heads, big, big, d))
    v = r.standard_normal((1, heads, big, big, d))
    rpb = r.standard_normal((heads, 2 * ksize - 1, 2 * ksize - 1))
    rad = ksize // 2
    base = orc.na2d_forward(q[:, :, :crop, :crop], k[:, :, :crop, :crop],
                            v[:, :, :crop, :crop], rpb, ksize)
    for (oy, ox) in [(1, 0), (0, 3), (7, 5), (16, 16)]:
        sl = (slice(None), slice(None), slice(oy, oy + crop), slice(ox, ox + crop))
        sh = orc.na2d_forward(q[sl], k[sl], v[sl], rpb, ksize)
        # query (y, x) of the shifted crop is pixel (y + oy, x + ox) of the big
        # map, i.e. query (y + oy, x + ox) of the unshifted crop when that one
        # is inside it; both must be unclamped (rad <= . < crop - rad).
        checked = 0
        for y in range(rad, crop - rad):
            yb = y + oy
            if not (rad <= yb < crop - rad):
                continue
            xs = [x for x in range(rad, crop - rad) if rad <= x + ox < crop - rad]
            if not xs:
                continue
            xb = [x + ox for x in xs]
            assert np.array_equal(sh[:, :, y, xs], base[:, :, yb, xb]), (oy, ox, y)
            checked += len(xs)
        assert checked > 0 or (oy, ox) == (16, 16)


def pin_flip_transpose(orc):
    """Mirroring the map along x with the bias table mirrored mirrors the output;
    transposing H and W with the table transposed transposes it (the clamp is
    symmetric for odd k).  Non-square maps catch an H/W mix-up."""
    r = _rng(14)
    for (B, heads, H, W, d, ksize) in [(1, 2, 9, 13, 8, 5), (2, 1, 7, 11, 4, 7), (1, 1, 3, 8, 6, 3)]:
        q = r.standard_normal((B, heads, H, W, d))
        k = r.standard_normal((B, heads, H, W, d))
        v = r.standard_normal((B, heads, H, W, d))
        rpb = r.standard_normal((heads, 2 * ksize - 1, 2 * ksize - 1))
        base = orc.na2d_forward(q, k, v, rpb, ksize)
        fx = orc.na2d_forward(q[:, :, :, ::-1], k[:, :, :, ::-1], v[:, :, :, ::-1],
                              rpb[:, :, ::-1], ksize)
        assert np.abs(fx - base[:, :, :, ::-1]).max() <= 1e-12, ("flip x", H, W)
        fy = orc.na2d_forward(q[:, :, ::-1], k[:, :, ::-1], v[:, :, ::-1], rpb[:, ::-1], ksize)
        assert np.abs(fy - base[:, :, ::-1]).max() <= 1e-12, ("flip y", H, W)
        tr = orc.na2d_forward(q.transpose(0, 1, 3, 2, 4), k.transpose(0, 1, 3, 2, 4),
                              v.transpose(0, 1, 3, 2, 4), rpb.transpose(0, 2, 1), ksize)
        assert np.abs(tr - base.transpose(0, 1, 3, 2, 4)).max() <= 1e-12, ("transpose", H, W)


def pin_box_mean(orc):
    """Q = 0 and no bias: the weights are uniform, so the output is the mean of V
    over the k-nearest window, computed here by 2D prefix sums over the
    brute-force nearest sets."""
    r = _rng(15)
    for (B, heads, H, W, d, ksize) in [(1, 1, 9, 12, 3, 5), (2, 2, 7, 7, 4, 7), (1, 1, 11, 6, 2, 3),
                                       (1, 1, 5, 9, 2, 1)]:
        v = r.standard_normal((B, heads, H, W, d))
        q = np.zeros_like(v)
        k = r.standard_normal((B, heads, H, W, d))
        got = orc.na2d_forward(q, k, v, None, ksize)
        P = np.zeros((B, heads, H + 1, W + 1, d))
        P[:, :, 1:, 1:] = v.cumsum(axis=2).cumsum(axis=3)
        want = np.empty_like(v)
        for y in range(H):
            ry = _nearest_set(y, ksize, H)
            y0, y1 = ry[0], ry[-1] + 1
            for x in range(W):
                rx = _nearest_set(x, ksize, W)
                x0, x1 = rx[0], rx[-1] + 1
                s = P[:, :, y1, x1] - P[:, :, y0, x1] - P[:, :, y1, x0] + P[:, :, y0, x0]
                want[:, :, y, x] = s / (ksize * ksize)
        assert np.abs(got - want).max() <= 1e-12, ("box mean", H, W, ksize)


def pin_identity(orc):
    """k = 1 gives out = V exactly; a constant V gives that constant."""
    r = _rng(16)
    q = r.standard_normal((2, 2, 6, 5, 8))
    k = r.standard_normal((2, 2, 6, 5, 8))
    v = r.standard_normal((2, 2, 6, 5, 8))
    out = orc.na2d_forward(q, k, v, r.standard_normal((2, 1, 1)), 1)
    assert np.array_equal(out, v), "k=1 identity"
    c = np.broadcast_to(r.standard_normal((1, 1, 1, 1, 8)), v.shape).copy()
    out = orc.na2d_forward(q, k, c, r.standard_normal((2, 9, 9)), 5)
    assert np.abs(out - c).max() <= 1e-14, "constant V"


def pin_bias_offset(orc):
    """A one-hot bias of +200 at relative offset (dy, dx) = (+1, 0) (key one row
    below the query) makes each query copy the V of that key wherever that key
    is in its window; where it is not (last row), the weights are uniform.
    Pins the sign and the (row, column) order of the bias index."""
    r = _rng(17)
    ksize, d = 3, 4
    H, W = 6, 7
    q = r.standard_normal((1, 1, H, W, d)) * 1e-3
    k = r.standard_normal((1, 1, H, W, d)) * 1e-3
    v = r.standard_normal((1, 1, H, W, d))
    rpb = np.zeros((1, 2 * ksize - 1, 2 * ksize - 1))
    rpb[0, 1 + ksize - 1, 0 + ksize - 1] = 200.0
    out = orc.na2d_forward(q, k, v, rpb, ksize)
    for y in range(H - 1):
        for x in range(W):
            assert np.abs(out[0, 0, y, x] - v[0, 0, y + 1, x]).max() < 1e-9, (y, x)
    # last row: offset +1 is outside the map, so no neighbour carries the bias
    y = H - 1
    for x in range(W):
        ys = _nearest_set(y, ksize, H)
        xs = _nearest_set(x, ksize, W)
        mean = v[0, 0][np.ix_(ys, xs)].reshape(-1, d).mean(axis=0)
        assert np.abs(out[0, 0, y, x] - mean).max() < 1e-5, (y, x)


def pin_softmax_shift(orc):
    """Adding a constant to every bias entry leaves the output unchanged
    (softmax is shift-invariant), while scaling Q by s scales the logits by s:
    with Q = 0 every bias-free output equals the box mean already pinned, and
    the output is finite for large logits."""
    r = _rng(18)
    q = r.standard_normal((1, 2, 8, 9, 16)) * 30.0       # peaked softmax, large logits
    k = r.standard_normal((1, 2, 8, 9, 16))
    v = r.standard_normal((1, 2, 8, 9, 16))
    rpb = r.standard_normal((2, 9, 9))
    a = orc.na2d_forward(q, k, v, rpb, 5)
    b = orc.na2d_forward(q, k, v, rpb + 123.0, 5)
    assert np.isfinite(a).all()
    assert np.abs(a - b).max() <= 1e-10, np.abs(a - b).max()


def pin_lse(orc):
    """The log softmax denominator ln sum_j exp(s_j), s_j = (q.k_j + B_j)/sqrt(d):
    with Q = 0 and no bias every logit is 0, so it is ln(k^2) exactly; at
    k = H = W it is scipy's logsumexp of the dense logits of full self
    attention; a constant c added to the bias adds c/sqrt(d); and the output
    returned beside it is the pinned forward's, bit for bit."""
    from scipy.special import logsumexp
    r = _rng(19)
    v = r.standard_normal((2, 2, 9, 11, 8))
    for ks in (1, 3, 5, 9):
        _, lse = orc.na2d_forward_lse(np.zeros_like(v), v, v, None, ks)
        assert np.abs(lse - np.log(ks * ks)).max() <= 1e-12, ("box", ks)
    for (B, heads, n, d) in [(1, 2, 5, 8), (2, 1, 7, 32)]:
        q = r.standard_normal((B, heads, n, n, d)) * 2.0
        k = r.standard_normal((B, heads, n, n, d))
        vv = r.standard_normal((B, heads, n, n, d))
        rpb = r.standard_normal((heads, 2 * n - 1, 2 * n - 1))
        out, lse = orc.na2d_forward_lse(q, k, vv, rpb, n)
        for b in range(B):
            for h in range(heads):
                S = q[b, h].reshape(n * n, d) @ k[b, h].reshape(n * n, d).T
                S = (S + _dense_bias(rpb[h], n, n, n)) / np.sqrt(d)
                want = logsumexp(S, axis=1).reshape(n, n)
                assert np.abs(lse[b, h] - want).max() <= 1e-12, ("dense", n)
        _, shifted = orc.na2d_forward_lse(q, k, vv, rpb + 3.0, n)
        assert np.abs(shifted - lse - 3.0 / np.sqrt(d)).max() <= 1e-12, ("shift", n)
        assert np.array_equal(out, orc.na2d_forward(q, k, vv, rpb, n))


def pin_sampled_index(orc):
    """The sampled form returns, for each linear query index
    ((b * heads + h) * H + y) * W + x, exactly the row of the whole-map forward
    (already pinned above) at that index: on ragged maps with several batches
    and heads, where a swapped batch/head or row/column split lands on another
    query. Indices come in shuffled order, with the first and last query."""
    r = _rng(20)
    for (B, heads, H, W, d, ks) in [(3, 2, 9, 11, 8, 5), (2, 3, 7, 12, 4, 7), (4, 5, 6, 5, 8, 3)]:
        q = r.standard_normal((B, heads, H, W, d))
        k = r.standard_normal((B, heads, H, W, d))
        v = r.standard_normal((B, heads, H, W, d))
        rpb = r.standard_normal((heads, 2 * ks - 1, 2 * ks - 1))
        full = orc.na2d_forward(q, k, v, rpb, ks).reshape(-1, d)
        n = full.shape[0]
        idx = np.concatenate([[n - 1, 0], r.permutation(n)[: n // 2]]).astype(np.int64)
        got = orc.na2d_forward_sampled(q, k, v, rpb, ks, idx)
        assert got.shape == (idx.size, d)
        assert np.array_equal(got, full[idx]), (B, heads, H, W, ks)


ALL_PINS = [pin_span, pin_self_attention, pin_sdpa, pin_translation, pin_flip_transpose,
            pin_box_mean, pin_identity, pin_bias_offset, pin_softmax_shift, pin_lse,
            pin_sampled_index]
