"""na2d_backward_noalloc: the backward for callers that cannot allocate, with
its workspace in a fixed per-device array, against na2d_backward with a
caller-allocated workspace on the same inputs.

Two calls in a row on one GPU, the second on a smaller problem (another
dtype, window and map), so that the second call runs on the array as the
first call left it. dq, dk and dv come from the same kernels and must match
bit for bit; the bias gradient is summed with float atomics, so it is held to
the backward's bound: max|err| <= 1e-4 * max(1, max|ref|). Both are also
checked against the fp64 gradient oracle to that bound.
"""
import numpy as np
import pytest
import torch

import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

CASES = [  # (shape, ksize, dtype): the second is smaller than the first
    ((4, 2, 56, 56, 32), 7, "f16"),
    ((1, 3, 19, 23, 32), 5, "bf16"),
]


def run_both(shape, ks, dt, seed):
    dev = torch.device("cuda")
    x = make_inputs(shape, ks, dt, seed=seed, rpb_std=1.0)
    q, k, v, rpb = x.q.to(dev), x.k.to(dev), x.v.to(dev), x.rpb.to(dev)
    out, lse = na2d.forward_lse(q, k, v, rpb, ks)
    g64 = np.random.default_rng(seed + 100).standard_normal(x.q64.shape)
    g = torch.from_numpy(g64.astype(np.float32)).to(dev)
    want = na2d.backward(q, k, v, rpb, out, g, ks, lse=lse)
    f32 = dict(dtype=torch.float32, device=dev)
    got = [torch.full(q.shape, float("nan"), **f32) for _ in range(3)]
    got.append(torch.full(rpb.shape, float("nan"), **f32))
    B, heads, H, W, d = shape
    st = na2d.na2d_backward_noalloc(q, k, v, rpb, out, lse, g, *got, B, heads, H, W, d, ks,
                                    na2d.TORCH_DTYPE_CODE[q.dtype],
                                    torch.cuda.current_stream(dev))
    assert st == na2d.NA2D_OK, na2d.na2d_strerror(st)
    torch.cuda.synchronize()
    ref = oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64, g.cpu().double().numpy(), ks)
    return got, want, ref


def test_noalloc_matches_workspace_backward_twice():
    for i, (shape, ks, dt) in enumerate(CASES):
        print("no-alloc backward call", i, shape, ks, dt, flush=True)
        got, want, ref = run_both(shape, ks, dt, seed=40 + i)
        for name, a, b in zip(("dq", "dk", "dv"), got[:3], want[:3]):
            assert torch.equal(a, b), "%s differs from na2d_backward (call %d)" % (name, i)
        bound = 1e-4 * max(1.0, float(want[3].abs().max()))
        assert float((got[3] - want[3]).abs().max()) <= bound, "drpb (call %d)" % i
        for name, a, r in zip(("dq", "dk", "dv", "drpb"), got, ref):
            err = float(np.abs(a.cpu().double().numpy() - r).max())
            assert err <= 1e-4 * max(1.0, float(np.abs(r).max())), (name, i, err)
