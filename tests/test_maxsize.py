"""The largest problems the kernels address, checked on sampled outputs.

- One map as large as 32-bit byte offsets inside a map allow (H*W*d*4 just
  under 2^31: 4096 x 4095 at d = 32), on the halo kernel (k = 7) and the
  wide-window kernel (k = 15).
- A batch of more than 2^31 elements (80 x 16 maps of 256 x 256 x 32), so
  that element offsets past 2^31 - 1 need 64 bits, on both kernels.

A sampled query is checked against the fp64 oracle run on a crop of the
inputs: its window is the same in a crop of 2k rows and columns anchored to
the borders it is near, because the clamped window of a query within k of a
border is pinned to that border and an interior query's window is unclamped
in both.  The backward at the large batch is checked the same way for dq (a
query's dq depends only on its own window), and by closed forms over every
element: per map the value gradients sum to the upstream gradients and the
key gradients to zero (the softmax weights of a query sum to one, and its
dS to zero), and per head the bias gradient sums to zero.

Inputs are seeded normals drawn on the GPU (the sizes rule out drawing them
on the host); the oracle gets the exact 16-bit values widened to fp64.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d

pytestmark = pytest.mark.gpu

TOL16 = 2e-3


def crop_span(i, L, k):
    """Rows (or columns) [lo, hi) of a crop in which index i keeps its window."""
    size = 2 * k
    if L <= size:
        return 0, L
    if i < k:
        return 0, size
    if i >= L - k:
        return L - size, L
    return i - k, i - k + size


def sample_queries(B, heads, H, W, n, seed):
    """The four corners and edge midpoints of the last map, plus n random
    queries from all maps (map index, y, x)."""
    rng = np.random.default_rng(seed)
    last = B * heads - 1
    fixed = [(last, y, x) for y in (0, H // 2, H - 1) for x in (0, W // 2, W - 1)]
    rand = [(int(rng.integers(B * heads)), int(rng.integers(H)), int(rng.integers(W))) for _ in range(n)]
    return fixed + rand


def draw(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * scale).to(dtype)


def crop(t, m, ys, xs, heads):
    """[1, 1, h, w, d] fp64 crop of map m of a [B, heads, H, W, d] tensor."""
    b, h = divmod(m, heads)
    return t[b, h, ys[0]:ys[1], xs[0]:xs[1]].double().cpu().numpy()[None, None]


def check_forward(q, k, v, rpb, ks, out, queries):
    B, heads, H, W, d = q.shape
    worst = 0.0
    for m, y, x in queries:
        ys, xs = crop_span(y, H, ks), crop_span(x, W, ks)
        h = m % heads
        want = oracle.na2d_forward(crop(q, m, ys, xs, heads), crop(k, m, ys, xs, heads),
                                   crop(v, m, ys, xs, heads), rpb[h:h + 1].double().cpu().numpy(), ks)
        b = m // heads
        got = out[b, h, y, x].double().cpu().numpy()
        worst = max(worst, float(np.abs(got - want[0, 0, y - ys[0], x - xs[0]]).max()))
    return worst


@pytest.mark.parametrize("ks,dtype", [(7, torch.float16), (15, torch.float16)], ids=["halo-k7", "wide-window-k15"])
def test_forward_largest_map(ks, dtype):
    B, heads, H, W, d = 1, 1, 4096, 4095, 32
    assert 2 ** 31 - 2 ** 20 <= H * W * d * 4 < 2 ** 31
    print("largest map", H, W, "k", ks, flush=True)
    q, k, v = (draw((B, heads, H, W, d), dtype, s) for s in (1, 2, 3))
    rpb = draw((heads, 2 * ks - 1, 2 * ks - 1), torch.float32, 4)
    out = na2d.forward(q, k, v, rpb, ks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = check_forward(q, k, v, rpb, ks, out, sample_queries(B, heads, H, W, 64, 5))
    print("  max|err| %.3g" % err, flush=True)
    assert err <= TOL16
    del out, q, k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ks,dtype", [(7, torch.float16), (13, torch.float16), (13, torch.bfloat16),
                                      (21, torch.bfloat16)],
                         ids=["halo-k7", "halo-k13", "wide-window-k13-bf16", "wide-window-k21-bf16"])
def test_forward_past_2_31_elements(ks, dtype):
    B, heads, H, W, d = 80, 16, 256, 256, 32
    assert B * heads * H * W * d > 2 ** 31
    print("past 2^31 elements, k =", ks, dtype, flush=True)
    q, k, v = (draw((B, heads, H, W, d), dtype, s) for s in (11, 12, 13))
    rpb = draw((heads, 2 * ks - 1, 2 * ks - 1), torch.float32, 14)
    out = na2d.forward(q, k, v, rpb, ks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = check_forward(q, k, v, rpb, ks, out, sample_queries(B, heads, H, W, 48, 15))
    print("  max|err| %.3g" % err, flush=True)
    assert err <= TOL16
    del out, q, k, v
    torch.cuda.empty_cache()


def check_backward(B, heads, H, W, d, ks, seed, n_sampled):
    q, k, v = (draw((B, heads, H, W, d), torch.float16, s) for s in (seed, seed + 1, seed + 2))
    rpb = draw((heads, 2 * ks - 1, 2 * ks - 1), torch.float32, seed + 3)
    g = draw((B, heads, H, W, d), torch.float32, seed + 4)
    out = na2d.forward(q, k, v, rpb, ks, algo=na2d.NA2D_ALGO_VALU)  # fp32 arithmetic
    lse = na2d.forward_lse(q, k, v, rpb, ks)[1]
    dq, dk, dv, drpb = na2d.backward(q, k, v, rpb, out, g, ks, lse=lse)
    torch.cuda.synchronize()
    for t in (dq, dk, dv, drpb):
        assert torch.isfinite(t).all()
    # closed forms over every element, per map / per head (fp64 sums of the fp32 results)
    f64 = torch.float64
    gsum, dvsum = g.sum(dim=(2, 3), dtype=f64), dv.sum(dim=(2, 3), dtype=f64)
    scale = g.abs().sum(dim=(2, 3), dtype=f64)
    assert ((dvsum - gsum).abs() <= 1e-5 * scale + 1e-3).all(), (dvsum - gsum).abs().max()
    dksum, dkscale = dk.sum(dim=(2, 3), dtype=f64), dk.abs().sum(dim=(2, 3), dtype=f64)
    assert (dksum.abs() <= 1e-5 * dkscale + 1e-3).all(), dksum.abs().max()
    dbsum = drpb.sum(dim=(1, 2), dtype=f64)
    assert (dbsum.abs() <= 1e-5 * drpb.abs().sum(dim=(1, 2), dtype=f64) + 1e-3).all(), dbsum
    # dq of sampled queries against the oracle's gradients on their crops
    worst = 0.0
    for m, y, x in sample_queries(B, heads, H, W, n_sampled, seed + 5):
        ys, xs = crop_span(y, H, ks), crop_span(x, W, ks)
        hh = m % heads
        want = oracle.na2d_backward(crop(q, m, ys, xs, heads), crop(k, m, ys, xs, heads),
                                    crop(v, m, ys, xs, heads), rpb[hh:hh + 1].double().cpu().numpy(),
                                    crop(g, m, ys, xs, heads), ks)[0]
        b = m // heads
        got = dq[b, hh, y, x].double().cpu().numpy()
        ref = want[0, 0, y - ys[0], x - xs[0]]
        worst = max(worst, float(np.abs(got - ref).max() / max(1.0, np.abs(ref).max())))
    print("  dq max relative err %.3g" % worst, flush=True)
    assert worst <= 1e-4
    del q, k, v, g, out, lse, dq, dk, dv, drpb
    torch.cuda.empty_cache()


def test_backward_past_2_31_elements():
    B, heads, H, W, d, ks = 80, 16, 256, 256, 32, 7
    assert B * heads * H * W * d > 2 ** 31
    print("backward past 2^31 elements", flush=True)
    check_backward(B, heads, H, W, d, ks, 21, 32)


@pytest.mark.parametrize("H,W,algo", [(4096, 4095, na2d.NA2D_ALGO_MFMA),
                                      (4096, 4096, na2d.NA2D_ALGO_VALU)])
def test_backward_largest_map(H, W, algo):
    """The largest map whose fp32 rows the matrix-core backward addresses with
    32-bit byte offsets (H * W * 128 < 2^31), and the first map past it, which
    the selection sends to the VALU kernels (64-bit offsets)."""
    d, ks = 32, 7
    assert na2d.na2d_backward_select_algo(H, W, d, ks, na2d.NA2D_F16) == algo
    print("backward largest map", H, W, "algo", algo, flush=True)
    check_backward(1, 1, H, W, d, ks, 31, 24)
