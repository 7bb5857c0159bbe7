"""GPU path vs the N-axis fp64 oracle for NA1D, NA3D and SASA windows, and the
general entry point with rectangular windows, element by element on small and
ragged grids.  Tolerances as for NA2D: max-abs 1e-5 for float32 inputs, 2e-3
for fp16/bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def dev(t):
    return None if t is None else t.to("cuda")


def finish(got, want, dtype, what):
    got = got.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    assert err <= TOL[dtype], "%s: max|err| %.3g > %.3g" % (what, err, TOL[dtype])


NA1D = [((2, 2, 37, 32), 7), ((1, 3, 100, 32), 49), ((1, 1, 9, 32), 9), ((2, 1, 64, 16), 5),
        ((1, 2, 70, 64), 13), ((1, 1, 33, 128), 3), ((1, 1, 5, 32), 1)]


@pytest.mark.parametrize("shape,ks", NA1D, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_na1d(shape, ks, dtype):
    print("na1d", shape, ks, dtype, flush=True)
    x = make_inputs(shape, ks, dtype, seed=1, rpb_std=1.0, op="na1d")
    got = na2d.forward_1d(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), ks)
    torch.cuda.synchronize()
    finish(got, oracle.na1d_forward(x.q64, x.k64, x.v64, x.rpb64, ks), dtype, "na1d %s k=%d" % (shape, ks))


NA3D = [((1, 2, 6, 7, 9, 32), 3), ((2, 1, 5, 5, 5, 32), 5), ((1, 2, 7, 9, 11, 32), 5),
        ((1, 1, 4, 12, 10, 16), 3), ((1, 1, 9, 9, 9, 64), 7),
        # volumes with waves none of whose windows is clamped (the matrix-core
        # kernel's interior path), next to border waves, for each block shape
        ((1, 2, 6, 16, 16, 32), 3), ((1, 1, 9, 20, 20, 32), 5), ((1, 1, 9, 16, 24, 32), 7)]


@pytest.mark.parametrize("shape,ks", NA3D, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_na3d(shape, ks, dtype):
    print("na3d", shape, ks, dtype, flush=True)
    x = make_inputs(shape, ks, dtype, seed=2, rpb_std=1.0, op="na3d")
    got = na2d.forward_3d(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), ks)
    torch.cuda.synchronize()
    finish(got, oracle.na3d_forward(x.q64, x.k64, x.v64, x.rpb64, ks), dtype, "na3d %s k=%d" % (shape, ks))


SASA = [((2, 2, 13, 17, 32), 3), ((1, 2, 13, 17, 32), 7), ((1, 1, 5, 6, 32), 7),
        ((2, 1, 20, 9, 16), 5), ((1, 1, 8, 8, 64), 11), ((1, 1, 6, 6, 32), 1)]


@pytest.mark.parametrize("shape,ks", SASA, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_sasa2d(shape, ks, dtype):
    print("sasa2d", shape, ks, dtype, flush=True)
    x = make_inputs(shape, ks, dtype, seed=3, rpb_std=1.0)
    got = na2d.forward_sasa2d(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), ks)
    torch.cuda.synchronize()
    finish(got, oracle.sasa2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks), dtype,
           "sasa2d %s k=%d" % (shape, ks))


@pytest.mark.parametrize("window,mode", [((3, 5, 1), 0), ((1, 3, 7), 0), ((3, 3, 5), 1),
                                         ((5, 1, 3), 1)], ids=str)
def test_general_rectangular(window, mode):
    """na_forward_nd with rectangular windows, in both window modes (no bias and with)."""
    shape = (2, 2, 6, 7, 8, 32)
    kd, kh, kw = window
    rng = np.random.default_rng(4)
    x = make_inputs(shape, 1, "f16", seed=4)
    rpb = (rng.standard_normal((2, 2 * kd - 1, 2 * kh - 1, 2 * kw - 1))).astype(np.float32)
    orc = oracle.default_nd()
    for bias in (None, rpb):
        got = na2d.forward_nd(dev(x.q), dev(x.k), dev(x.v),
                              None if bias is None else torch.from_numpy(bias).cuda(), window, mode)
        torch.cuda.synchronize()
        want = orc.forward(x.q64, x.k64, x.v64, None if bias is None else bias.astype(np.float64),
                           window, mode)
        finish(got, want, "f16", "nd %s mode %d" % (window, mode))


def test_general_matches_na2d():
    """The 2D NA case of the general entry point is na2d_forward (bitwise, same kernel)."""
    x = make_inputs((2, 2, 30, 26, 32), 7, "f16", seed=5)
    a = na2d.forward(dev(x.q), dev(x.k), dev(x.v), dev(x.rpb), 7, algo=na2d.NA2D_ALGO_VALU)
    sh = (2, 2, 1, 30, 26, 32)
    b = na2d.forward_nd(dev(x.q).reshape(sh), dev(x.k).reshape(sh), dev(x.v).reshape(sh),
                        dev(x.rpb).reshape(2, 1, 13, 13), (1, 7, 7), algo=na2d.NA2D_ALGO_VALU)
    torch.cuda.synchronize()
    assert torch.equal(a.reshape(sh), b)


SASA_MFMA = [((2, 2, 13, 17, 32), 3), ((1, 2, 21, 19, 32), 7), ((1, 1, 5, 6, 32), 7),
             ((2, 1, 20, 9, 32), 5), ((1, 2, 30, 33, 32), 9), ((1, 1, 8, 8, 32), 11),
             ((1, 2, 29, 37, 32), 11), ((1, 1, 27, 25, 32), 13), ((1, 1, 23, 23, 32), 21),
             ((1, 1, 10, 12, 32), 25), ((2, 2, 57, 55, 32), 7)]


@pytest.mark.parametrize("shape,ks", SASA_MFMA, ids=str)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("algo", [na2d.NA2D_ALGO_VALU, na2d.NA2D_ALGO_MFMA])
def test_sasa2d_both_kernels(shape, ks, dtype, algo):
    """SASA through each kernel family: ragged maps, windows up to 25, windows
    wider than the map (all padding past the edge)."""
    print("sasa2d", shape, ks, dtype, algo, flush=True)
    x = make_inputs(shape, ks, dtype, seed=6, rpb_std=1.0)
    B, heads, H, W, d = shape
    sh = (B, heads, 1, H, W, d)
    got = na2d.forward_nd(dev(x.q).reshape(sh), dev(x.k).reshape(sh), dev(x.v).reshape(sh),
                          dev(x.rpb).reshape(heads, 1, 2 * ks - 1, 2 * ks - 1), (1, ks, ks),
                          na2d.NA_WINDOW_SASA, algo)
    torch.cuda.synchronize()
    finish(got.reshape(shape), oracle.sasa2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks), dtype,
           "sasa2d %s k=%d algo=%d" % (shape, ks, algo))


NA1D_MFMA = [((2, 2, 37, 32), 7), ((1, 3, 100, 32), 49), ((1, 1, 9, 32), 9), ((2, 1, 64, 32), 5),
             ((1, 2, 130, 32), 17), ((1, 2, 131, 32), 19), ((1, 1, 63, 32), 63),
             ((2, 2, 257, 32), 63), ((1, 1, 3, 32), 3), ((3, 2, 1000, 32), 33),
             ((1, 1, 129, 32), 51)]


@pytest.mark.parametrize("shape,ks", NA1D_MFMA, ids=str)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("algo", [na2d.NA2D_ALGO_VALU, na2d.NA2D_ALGO_MFMA])
def test_na1d_both_kernels(shape, ks, dtype, algo):
    """NA1D through each kernel family: sequences shorter than, equal to and
    ragged against the 64-query tile, windows from 3 to 63, L = k."""
    print("na1d", shape, ks, dtype, algo, flush=True)
    x = make_inputs(shape, ks, dtype, seed=7, rpb_std=1.0, op="na1d")
    B, heads, L, d = shape
    sh = (B, heads, 1, 1, L, d)
    got = na2d.forward_nd(dev(x.q).reshape(sh), dev(x.k).reshape(sh), dev(x.v).reshape(sh),
                          dev(x.rpb).reshape(heads, 1, 1, 2 * ks - 1), (1, 1, ks),
                          na2d.NA_WINDOW_NA, algo)
    torch.cuda.synchronize()
    finish(got.reshape(shape), oracle.na1d_forward(x.q64, x.k64, x.v64, x.rpb64, ks), dtype,
           "na1d %s k=%d algo=%d" % (shape, ks, algo))


# The matrix-core kernel for other NA windows: 3D windows (cubic or not, a
# window of 1 on some axis) and rectangular 2D windows; ragged 8 x 8 patches,
# windows as wide as the axis, and both odd and even counts of key blocks.
ND_MFMA = [((2, 2, 6, 7, 9, 32), (3, 3, 3)), ((1, 2, 7, 19, 21, 32), (5, 5, 5)),
           ((1, 1, 5, 17, 17, 32), (5, 7, 3)), ((1, 1, 9, 9, 10, 32), (9, 9, 9)),
           ((2, 1, 3, 13, 11, 32), (1, 3, 5)), ((1, 2, 1, 23, 18, 32), (1, 3, 9)),
           ((1, 1, 1, 12, 40, 32), (1, 9, 1)), ((1, 1, 4, 16, 16, 32), (3, 1, 1)),
           ((1, 1, 2, 8, 8, 32), (1, 1, 1))]


@pytest.mark.parametrize("shape,window", ND_MFMA, ids=str)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("algo", [na2d.NA2D_ALGO_VALU, na2d.NA2D_ALGO_MFMA])
def test_nd_windows_both_kernels(shape, window, dtype, algo):
    print("nd", shape, window, dtype, algo, flush=True)
    kd, kh, kw = window
    x = make_inputs(shape, 1, dtype, seed=6, op="na3d")
    rng = np.random.default_rng(7)
    rpb = rng.standard_normal((shape[1], 2 * kd - 1, 2 * kh - 1, 2 * kw - 1))
    got = na2d.forward_nd(dev(x.q), dev(x.k), dev(x.v), torch.from_numpy(rpb.astype(np.float32)).cuda(),
                          window, na2d.NA_WINDOW_NA, algo)
    torch.cuda.synchronize()
    want = oracle.default_nd().forward(x.q64, x.k64, x.v64, rpb.astype(np.float32).astype(np.float64),
                                       window, na2d.NA_WINDOW_NA)
    finish(got, want, dtype, "nd %s %s algo=%d" % (shape, window, algo))
