"""GPU gradients of the NA2D forward vs the fp64 gradient oracle.

The kernels compute in fp32 from inputs that are exact in both places, so one
bound serves every dtype: max|got - want| <= 1e-4 * max(1, max|want|) per
gradient (the largest sums have about 10^5 fp32 terms: the bias gradient of a
full-size map; relative error of such sums stays near 1e-6)."""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def run(x, ks, with_bias=True, seed=0):
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed + 100)
    g64 = rng.standard_normal(x.q64.shape)
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    rpb = x.rpb.to(dev) if with_bias else None
    out = na2d.forward(q, k, v, rpb, ks, algo=na2d.NA2D_ALGO_VALU)
    grads = na2d.backward(q, k, v, rpb, out, torch.from_numpy(g64).float().to(dev), ks)
    torch.cuda.synchronize()
    # the oracle takes the same (fp32-rounded) upstream gradient
    g = torch.from_numpy(g64).float().double().numpy()
    want = oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64 if with_bias else None, g, ks)
    return [None if t is None else t.cpu().double().numpy() for t in grads], want


def check(shape, ks, dtype, with_bias=True, **kw):
    print("backward", shape, ks, dtype, with_bias, kw, flush=True)
    x = make_inputs(shape, ks, dtype, seed=8, **kw)
    got, want = run(x, ks, with_bias)
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, want):
        if b is None:
            assert a is None
            continue
        assert np.isfinite(a).all(), name
        err = np.abs(a - b).max()
        bound = RTOL * max(1.0, np.abs(b).max())
        assert err <= bound, "%s %s k=%d %s: max|err| %.3g > %.3g" % (name, shape, ks, dtype, err, bound)


SHAPES = [((1, 2, 13, 17, 32), 3), ((1, 2, 13, 17, 32), 5), ((2, 2, 20, 24, 32), 7),
          ((1, 1, 9, 9, 32), 9), ((1, 1, 7, 30, 32), 7), ((1, 1, 25, 23, 32), 11),
          ((1, 1, 40, 41, 32), 33), ((1, 1, 6, 6, 32), 1)]


@pytest.mark.parametrize("shape,ks", SHAPES, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_backward(shape, ks, dtype):
    check(shape, ks, dtype, rpb_std=1.0)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_backward_head_dims(d):
    check((1, 2, 11, 13, d), 5, "f16", rpb_std=1.0)


def test_backward_no_bias_and_peaked():
    check((2, 2, 15, 14, 32), 7, "bf16", with_bias=False)
    check((1, 2, 15, 14, 32), 7, "f32", q_scale=4.0, rpb_std=1.0)


def test_backward_full_size_stage1():
    """NAT-Tiny stage 1 at full size, every gradient element."""
    w = WORKLOADS["nat_tiny_stage1_f16"]
    x = workload_inputs(w, seed=0)
    got, want = run(x, w.k)
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, want):
        err = np.abs(a - b).max()
        print("  %s max|err| %.3g (max|want| %.3g)" % (name, err, np.abs(b).max()), flush=True)
        assert err <= RTOL * max(1.0, np.abs(b).max()), name
