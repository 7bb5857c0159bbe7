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


def run(x, ks, with_bias=True, seed=0, use_lse=False):
    """Gradients on the GPU and from the oracle.  out comes from the VALU
    forward (fp32 arithmetic), so that out's own rounding is not measured here;
    with use_lse the softmax statistics come from na2d_forward_lse (automatic
    kernel choice) instead of being recomputed by the backward."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(seed + 100)
    g64 = rng.standard_normal(x.q64.shape)
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    rpb = x.rpb.to(dev) if with_bias else None
    out = na2d.forward(q, k, v, rpb, ks, algo=na2d.NA2D_ALGO_VALU)
    lse = na2d.forward_lse(q, k, v, rpb, ks)[1] if use_lse else None
    grads = na2d.backward(q, k, v, rpb, out, torch.from_numpy(g64).float().to(dev), ks, lse=lse)
    torch.cuda.synchronize()
    # the oracle takes the same (fp32-rounded) upstream gradient
    g = torch.from_numpy(g64).float().double().numpy()
    want = oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64 if with_bias else None, g, ks)
    return [None if t is None else t.cpu().double().numpy() for t in grads], want


def check(shape, ks, dtype, with_bias=True, use_lse=False, **kw):
    print("backward", shape, ks, dtype, with_bias, use_lse, kw, flush=True)
    x = make_inputs(shape, ks, dtype, seed=8, **kw)
    got, want = run(x, ks, with_bias, use_lse=use_lse)
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
          ((1, 1, 40, 41, 32), 33), ((1, 1, 6, 6, 32), 1),
          # the widest windows of the matrix-core passes (k <= 25), ragged tiles on both axes
          ((1, 1, 27, 29, 32), 13), ((1, 1, 19, 33, 32), 17), ((1, 1, 30, 26, 32), 25)]


@pytest.mark.parametrize("shape,ks", SHAPES, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("use_lse", [False, True], ids=["recomputed", "from_forward"])
def test_backward(shape, ks, dtype, use_lse):
    check(shape, ks, dtype, rpb_std=1.0, use_lse=use_lse)


LSE_SHAPES = [((2, 2, 20, 24, 32), 7), ((1, 2, 13, 17, 32), 5), ((1, 1, 19, 21, 32), 9),
              ((1, 1, 27, 25, 32), 13), ((1, 1, 23, 23, 32), 21), ((1, 1, 6, 6, 32), 1),
              ((1, 2, 11, 13, 64), 5)]


@pytest.mark.parametrize("shape,ks", LSE_SHAPES, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_forward_lse(shape, ks, dtype):
    """na2d_forward_lse: lse against the oracle's log softmax denominator
    (fp32 logits of exact inputs: within 2e-5 absolute), and the same output
    as na2d_forward, bit for bit (the statistics are an extra store)."""
    print("forward_lse", shape, ks, dtype, flush=True)
    x = make_inputs(shape, ks, dtype, seed=9, rpb_std=1.0)
    dev = torch.device("cuda")
    q, k, v, rpb = x.q.to(dev), x.k.to(dev), x.v.to(dev), x.rpb.to(dev)
    out, lse = na2d.forward_lse(q, k, v, rpb, ks)
    plain = na2d.forward(q, k, v, rpb, ks)
    torch.cuda.synchronize()
    _, want = oracle.na2d_forward_lse(x.q64, x.k64, x.v64, x.rpb64, ks)
    err = np.abs(lse.cpu().double().numpy() - want).max()
    assert err <= 2e-5, "lse %s k=%d %s: max|err| %.3g" % (shape, ks, dtype, err)
    assert torch.equal(out, plain)


@pytest.mark.parametrize("d", [16, 64, 128])
def test_backward_head_dims(d):
    check((1, 2, 11, 13, d), 5, "f16", rpb_std=1.0)


def test_backward_no_bias_and_peaked():
    check((2, 2, 15, 14, 32), 7, "bf16", with_bias=False)
    check((1, 2, 15, 14, 32), 7, "f32", q_scale=4.0, rpb_std=1.0)


@pytest.mark.parametrize("use_lse", [False, True], ids=["recomputed", "from_forward"])
def test_backward_full_size_stage1(use_lse):
    """NAT-Tiny stage 1 at full size, every gradient element."""
    w = WORKLOADS["nat_tiny_stage1_f16"]
    x = workload_inputs(w, seed=0)
    got, want = run(x, w.k, use_lse=use_lse)
    for name, a, b in zip(("dq", "dk", "dv", "drpb"), got, want):
        err = np.abs(a - b).max()
        print("  %s max|err| %.3g (max|want| %.3g)" % (name, err, np.abs(b).max()), flush=True)
        assert err <= RTOL * max(1.0, np.abs(b).max()), name
