"""A second, wider seeded sweep, element by element against the fp64 oracle.

Beyond tests/test_sweep.py: maps up to 140 on a side and up to three images
and heads, both bias scales (0.02 and 1) and peaked softmaxes (Q x 4) for the
2D forward (NA, SASA, and the saved log-sum-exp); gradients with and without
the forward's log-sum-exp; NA1D windows up to 63 and NA3D windows up to 7,
including fp32 inputs and head sizes 16 and 64, which take the VALU kernel.
Tolerances are those of the other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
LSE_TOL = 2e-5
GRAD_RTOL = 1e-4
KS = [3, 5, 7, 9, 11, 13, 15, 17, 19, 21, 23, 25]


def forward_cases(n=240, seed=424242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ks = int(rng.choice(KS))
        mode = "sasa" if rng.random() < 0.3 else "na"
        lo = 1 if mode == "sasa" else ks
        span = int(rng.choice([40, 70, 140]))
        H = int(rng.integers(lo, max(lo + 1, span)))
        W = int(rng.integers(lo, max(lo + 1, span)))
        shape = (int(rng.integers(1, 4)), int(rng.integers(1, 4)), H, W, 32)
        dtype = "f16" if rng.random() < 0.5 else "bf16"
        rpb_std = float(rng.choice([0.02, 1.0]))
        q_scale = float(rng.choice([1.0, 1.0, 4.0]))
        lse = mode == "na" and rng.random() < 0.3
        out.append((shape, ks, dtype, mode, rpb_std, q_scale, lse, 5000 + i))
    return out


def backward_cases(n=40, seed=4243):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ks = int(rng.choice(KS[:9]))
        H = int(rng.integers(ks, ks + 30))
        W = int(rng.integers(ks, ks + 30))
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 3)), H, W, 32)
        dtype = "f16" if rng.random() < 0.5 else "bf16"
        out.append((shape, ks, dtype, rng.random() < 0.7, 7000 + i))
    return out


def nd_cases(n=80, seed=4244):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        op = "na1d" if rng.random() < 0.5 else "na3d"
        dtype = str(rng.choice(["f16", "bf16", "f32"]))
        d = int(rng.choice([32, 32, 32, 16, 64])) if dtype == "f32" or rng.random() < 0.2 else 32
        if op == "na1d":
            ks = int(rng.choice([3, 5, 7, 9, 13, 21, 31, 49, 63]))
            shape = (int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(ks, ks + 300)), d)
        else:
            ks = int(rng.choice([3, 5, 7]))
            D, H, W = (int(rng.integers(ks, ks + 12)) for _ in range(3))
            shape = (int(rng.integers(1, 3)), int(rng.integers(1, 3)), D, H, W, d)
        out.append((op, shape, ks, dtype, 9000 + i))
    return out


def dev(t):
    return t.to(torch.device("cuda"))


@pytest.mark.parametrize("case", forward_cases(), ids=lambda c: "%s-k%d-%s-%s" % (c[0][:4], c[1], c[2], c[3]))
def test_forward_wide(case):
    shape, ks, dtype, mode, rpb_std, q_scale, use_lse, seed = case
    print("wide sweep", case, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, rpb_std=rpb_std, q_scale=q_scale)
    q, k, v, rpb = dev(x.q), dev(x.k), dev(x.v), dev(x.rpb)
    if mode == "sasa":
        got = na2d.forward_sasa2d(q, k, v, rpb, ks)
        want = oracle.sasa2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    elif use_lse:
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
    assert err <= TOL[dtype], "max|err| %.3g > %.3g" % (err, TOL[dtype])


@pytest.mark.parametrize("case", backward_cases(), ids=lambda c: "%s-k%d-%s" % (c[0][:4], c[1], c[2]))
def test_backward_wide(case):
    shape, ks, dtype, use_lse, seed = case
    print("wide sweep backward", case, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, rpb_std=1.0)
    q, k, v, rpb = dev(x.q), dev(x.k), dev(x.v), dev(x.rpb)
    g64 = np.random.default_rng(seed + 1).standard_normal(x.q64.shape)
    g = dev(torch.from_numpy(g64).float())
    # out from the fp32 (VALU) forward, so that its own rounding is not measured here
    out = na2d.forward(q, k, v, rpb, ks, algo=na2d.NA2D_ALGO_VALU)
    lse = na2d.forward_lse(q, k, v, rpb, ks)[1] if use_lse else None
    got = na2d.backward(q, k, v, rpb, out, g, ks, lse=lse)
    torch.cuda.synchronize()
    want = oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64, g.cpu().double().numpy(), ks)
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, want):
        a = a.cpu().double().numpy()
        assert np.isfinite(a).all(), name
        err = np.abs(a - b).max()
        bound = GRAD_RTOL * max(1.0, np.abs(b).max())
        assert err <= bound, "%s max|err| %.3g > %.3g" % (name, err, bound)


@pytest.mark.parametrize("case", nd_cases(), ids=lambda c: "%s-%s-k%d-%s" % (c[0], c[1][2:-1], c[2], c[3]))
def test_nd_wide(case):
    op, shape, ks, dtype, seed = case
    print("wide sweep nd", case, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, rpb_std=1.0, op=op)
    if op == "na1d":
        got = na2d.forward_1d(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), ks)
        want = oracle.na1d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    else:
        got = na2d.forward_3d(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), ks)
        want = oracle.na3d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL[dtype], "max|err| %.3g > %.3g" % (err, TOL[dtype])
