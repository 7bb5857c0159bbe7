"""GPU path vs the fp64 oracle, element by element, on small and ragged maps.

Tolerances (max-abs over every output element): 1e-5 for float32 inputs,
2e-3 for fp16/bf16 inputs with fp32 accumulation.  Every case runs through
the C ABI (ctypes binding), once per kernel family that supports it.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
VALU, MFMA = na2d.NA2D_ALGO_VALU, na2d.NA2D_ALGO_MFMA


def gpu_forward(x, ks, algo, with_bias=True):
    dev = torch.device("cuda")
    rpb = x.rpb.to(dev) if with_bias else None
    out = na2d.forward(x.q.to(dev), x.k.to(dev), x.v.to(dev), rpb, ks, algo=algo)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def check(shape, ks, dtype, algo, seed=0, with_bias=True, **kw):
    print("case", shape, ks, dtype, algo, kw, flush=True)
    x = make_inputs(shape, ks, dtype, seed=seed, **kw)
    got = gpu_forward(x, ks, algo, with_bias)
    want = oracle.na2d_forward(x.q64, x.k64, x.v64, x.rpb64 if with_bias else None, ks)
    err = np.abs(got - want).max()
    assert np.isfinite(got).all()
    assert err <= TOL[dtype], "max|err| %.3g > %.3g for %s k=%d %s algo=%d" % (
        err, TOL[dtype], shape, ks, dtype, algo)
    return err


# (shape [B, heads, H, W, d], ksize)
RAGGED = [
    ((1, 1, 14, 14, 32), 7),    # the tiny workload
    ((1, 1, 7, 7, 32), 7),      # k = H = W: full self attention
    ((1, 3, 13, 29, 32), 3),
    ((1, 2, 13, 29, 32), 5),
    ((2, 2, 57, 55, 32), 7),    # several tiles plus ragged tails
    ((1, 1, 7, 30, 32), 7),     # H = k < W
    ((1, 1, 31, 7, 32), 7),     # W = k < H
    ((1, 2, 13, 29, 32), 9),
    ((1, 2, 13, 29, 32), 11),
    ((2, 1, 29, 37, 32), 13),
    ((1, 1, 23, 33, 32), 15),
    ((1, 1, 21, 21, 32), 21),   # k = H = W at k = 21
    ((1, 2, 45, 38, 32), 21),
    ((1, 1, 25, 40, 32), 25),
    ((1, 1, 3, 3, 32), 3),
]


@pytest.mark.parametrize("shape,ks", RAGGED, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mfma_ragged(shape, ks, dtype):
    check(shape, ks, dtype, MFMA)


@pytest.mark.parametrize("shape,ks", RAGGED, ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_valu_ragged(shape, ks, dtype):
    check(shape, ks, dtype, VALU)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_valu_head_dims(dtype, d):
    check((1, 2, 11, 13, d), 5, dtype, VALU)


@pytest.mark.parametrize("algo", [VALU, MFMA])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_stress_bias_and_peaked(algo, dtype):
    """RPB ~ N(0, 1) (the default 0.02 moves outputs by less than the tolerance)
    and Q scaled by 4 (peaked softmax)."""
    check((2, 2, 30, 26, 32), 7, dtype, algo, rpb_std=1.0)
    check((2, 2, 30, 26, 32), 7, dtype, algo, q_scale=4.0)
    check((1, 2, 40, 40, 32), 13, dtype, algo, rpb_std=1.0, q_scale=2.0)


@pytest.mark.parametrize("algo", [VALU, MFMA])
def test_no_bias(algo):
    check((2, 2, 20, 24, 32), 7, "f16", algo, with_bias=False)


def test_valu_f32_stress():
    check((1, 2, 19, 17, 32), 7, "f32", VALU, rpb_std=1.0, q_scale=3.0)
    check((1, 1, 16, 16, 32), 1, "f32", VALU)


def test_k1_identity():
    """k = 1: every query attends to itself only, so out = V exactly."""
    x = make_inputs((2, 2, 9, 10, 32), 1, "f16", seed=3)
    got = gpu_forward(x, 1, VALU)
    assert np.array_equal(got, x.v64)


@pytest.mark.parametrize("algo", [VALU, MFMA])
def test_deterministic(algo):
    x = make_inputs((4, 2, 56, 56, 32), 7, "f16", seed=5)
    a = gpu_forward(x, 7, algo)
    b = gpu_forward(x, 7, algo)
    assert np.array_equal(a, b)


def test_auto_selects_mfma_for_16bit():
    assert na2d.na2d_select_algo(56, 56, 32, 7, na2d.NA2D_F16) == MFMA
    assert na2d.na2d_select_algo(56, 56, 32, 7, na2d.NA2D_F32) == VALU
    assert na2d.na2d_select_algo(56, 56, 64, 7, na2d.NA2D_BF16) == VALU


def _replace_v(x, v64, dtype):
    """The inputs with V replaced by v64 rounded to the storage dtype."""
    import dataclasses
    from vision_sliding_window_amd.inputs import DTYPES
    vt = torch.from_numpy(v64).to(DTYPES[dtype])
    return dataclasses.replace(x, v=vt, v64=vt.double().numpy())


@pytest.mark.parametrize("shape,ks", [((1, 2, 45, 38, 32), 21), ((1, 1, 23, 33, 32), 15),
                                      ((2, 1, 40, 44, 32), 25)], ids=lambda v: str(v))
def test_bf16_values_past_fp16_range(shape, ks):
    """bf16 values of V beyond the fp16 range (the wide-window kernel takes V
    as fp16 where it fits).  (a) V times 2^20: the output scales by exactly
    2^20, so out / 2^20 is checked against the oracle on the unscaled V at
    the usual tolerance.  (b) a sparse 0.5% of V's entries times 2^17, so
    that some rows fit fp16 and some do not: checked against the oracle with
    the bound that fp16 weights give, 2e-3 + 2^-10 * sum_j p_j |v_j| per
    element (the sum is the oracle's output for |V|)."""
    x = make_inputs(shape, ks, "bf16", seed=7, rpb_std=1.0)
    dev = torch.device("cuda")
    want = oracle.na2d_forward(x.q64, x.k64, x.v64, x.rpb64, ks)
    xs = _replace_v(x, x.v64 * 2.0 ** 20, "bf16")
    got = gpu_forward(xs, ks, MFMA) / 2.0 ** 20
    assert np.isfinite(got).all()
    err = np.abs(got - want).max()
    print("  scaled V: max|err| %.3g" % err, flush=True)
    assert err <= TOL["bf16"]
    rng = np.random.default_rng(8)
    v = x.v64.copy()
    v[rng.random(v.shape) < 0.005] *= 2.0 ** 17
    xb = _replace_v(x, v, "bf16")
    assert np.abs(xb.v64).max() > 65520.0
    got = gpu_forward(xb, ks, MFMA)
    assert np.isfinite(got).all()
    want = oracle.na2d_forward(xb.q64, xb.k64, xb.v64, xb.rpb64, ks)
    bound = 2e-3 + 2.0 ** -10 * oracle.na2d_forward(xb.q64, xb.k64, np.abs(xb.v64), xb.rpb64, ks)
    ratio = (np.abs(got - want) / bound).max()
    print("  sparse large V: max|err| / bound %.3g" % ratio, flush=True)
    assert ratio <= 1.0
    # the LSE variant runs the same rows
    o2, _ = na2d.forward_lse(xb.q.to(dev), xb.k.to(dev), xb.v.to(dev), xb.rpb.to(dev), ks)
    torch.cuda.synchronize()
    assert np.array_equal(o2.cpu().double().numpy(), got)
