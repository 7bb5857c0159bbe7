"""A seeded sweep over map shapes, window sizes, dtypes and window modes.

Every kernel the automatic choice can take is reached: for k = 7 the
register-prefetch kernel and the column-ring kernel (one-tile and long runs),
the LDS-DMA kernel for other k up to 13 and for SASA, and the streaming kernel
for wide NA windows. The maps come in many sizes and aspect ratios: tiles
ragged on both axes, maps narrower than a tile, and H or W equal to k. Each
case is checked element by element against the fp64 oracle: forward outputs
(and on every fourth NA case the saved log-sum-exp) and, on a subset,
the gradients. Tolerances are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-3          # 16-bit inputs, fp32 accumulation
LSE_TOL = 2e-5      # the saved log-sum-exp (fp32 statistics)
GRAD_RTOL = 1e-4    # gradients, relative to max(1, max |want|)
KS = [3, 5, 7, 9, 11, 13, 15, 17, 19, 21, 23, 25]


def forward_cases(n=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ks = int(rng.choice(KS))
        mode = "sasa" if i % 3 == 2 else "na"
        lo = 1 if mode == "sasa" else ks  # NA needs the window to fit the map
        H = int(rng.integers(lo, max(lo + 1, 50)))
        W = int(rng.integers(lo, max(lo + 1, 50)))
        B, heads = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        dtype = "f16" if i % 2 == 0 else "bf16"
        out.append(((B, heads, H, W, 32), ks, dtype, mode, 100 + i))
    return out


def backward_cases(n=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ks = int(rng.choice(KS[:8]))  # k <= 17 keeps the fp64 gradients quick
        H = int(rng.integers(ks, ks + 24))
        W = int(rng.integers(ks, ks + 24))
        dtype = "f16" if i % 2 == 0 else "bf16"
        out.append(((1, int(rng.integers(1, 3)), H, W, 32), ks, dtype, 300 + i))
    return out


def dev(t):
    return t.to(torch.device("cuda"))


@pytest.mark.parametrize("case", forward_cases(), ids=lambda c: "%s-k%d-%s-%s" % (c[0][:4], c[1], c[2], c[3]))
def test_forward_sweep(case):
    shape, ks, dtype, mode, seed = case
    print("sweep", shape, ks, dtype, mode, seed, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, rpb_std=1.0)
    q, k, v, rpb = dev(x.q), dev(x.k), dev(x.v), dev(x.rpb)
    if mode == "sasa":
        got = na2d.forward_sasa2d(q, k, v, rpb, ks)
        want = oracle.sasa2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    elif seed % 4 == 0:
        got, lse = na2d.forward_lse(q, k, v, rpb, ks)
        want, want_lse = oracle.na2d_forward_lse(x.q64, x.k64, x.v64, x.rpb64, ks)
        lerr = np.abs(lse.cpu().double().numpy() - want_lse).max()
        assert lerr <= LSE_TOL, "lse max|err| %.3g" % lerr
    else:
        got = na2d.forward(q, k, v, rpb, ks)
        want = oracle.na2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL, "max|err| %.3g > %.3g" % (err, TOL)


@pytest.mark.parametrize("case", backward_cases(), ids=lambda c: "%s-k%d-%s" % (c[0][:4], c[1], c[2]))
def test_backward_sweep(case):
    shape, ks, dtype, seed = case
    print("sweep backward", shape, ks, dtype, seed, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, rpb_std=1.0)
    q, k, v, rpb = dev(x.q), dev(x.k), dev(x.v), dev(x.rpb)
    g64 = np.random.default_rng(seed + 1).standard_normal(x.q64.shape)
    g = dev(torch.from_numpy(g64).float())
    # out from the fp32 (VALU) forward, so that its own rounding is not measured here
    out = na2d.forward(q, k, v, rpb, ks, algo=na2d.NA2D_ALGO_VALU)
    lse = na2d.forward_lse(q, k, v, rpb, ks)[1]
    got = na2d.backward(q, k, v, rpb, out, g, ks, lse=lse)
    torch.cuda.synchronize()
    want = oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64, g.cpu().double().numpy(), ks)
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, want):
        a = a.cpu().double().numpy()
        assert np.isfinite(a).all(), name
        err = np.abs(a - b).max()
        bound = GRAD_RTOL * max(1.0, np.abs(b).max())
        assert err <= bound, "%s max|err| %.3g > %.3g" % (name, err, bound)
