"""Streams and graph capture: every kernel family run on a side stream gives
the default stream's results bit for bit; calls on two streams at once do not
interfere (the library keeps no state between calls); and forward and
backward captured in a HIP graph give, on every replay, the eager results
(replays interleaved with eager work and synchronisations)."""
import pytest
import torch

from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def dev(x):
    return {f: getattr(x, f).cuda() for f in ("q", "k", "v", "rpb")}


# (name, shape, ksize, dtype, call): one case per kernel family
def _cases():
    return [
        ("2d persistent k7", (2, 2, 40, 36, 32), 7, "f16", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("2d ring k7", (1, 1, 136, 16, 32), 7, "f16", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("2d halo k11", (1, 2, 30, 29, 32), 11, "f16", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("2d wide-window 8x8 tiles k21", (1, 1, 45, 38, 32), 21, "bf16", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("2d wide-window 4x16 tiles k15", (1, 2, 37, 45, 32), 15, "f16", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("2d valu f32", (1, 2, 19, 17, 32), 5, "f32", lambda t, ks, s: na2d.forward(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
        ("sasa", (1, 2, 21, 19, 32), 7, "f16", lambda t, ks, s: na2d.forward_sasa2d(t["q"], t["k"], t["v"], t["rpb"], ks, stream=s)),
    ]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c[0])
def test_side_stream_matches_default(case):
    name, shape, ks, dtype, call = case
    print("side stream", name, flush=True)
    t = dev(make_inputs(shape, ks, dtype, seed=31, rpb_std=1.0))
    want = call(t, ks, None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = call(t, ks, side)
    side.synchronize()
    assert torch.equal(got, want)


def test_nd_and_1d_on_side_stream():
    side = torch.cuda.Stream()
    x1 = dev(make_inputs((2, 2, 100, 32), 13, "f16", seed=32, op="na1d"))
    x3 = dev(make_inputs((1, 2, 6, 11, 13, 32), 3, "bf16", seed=33, op="na3d"))
    w1 = na2d.forward_1d(x1["q"], x1["k"], x1["v"], x1["rpb"], 13)
    w3 = na2d.forward_3d(x3["q"], x3["k"], x3["v"], x3["rpb"], 3)
    torch.cuda.synchronize()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g1 = na2d.forward_1d(x1["q"], x1["k"], x1["v"], x1["rpb"], 13, stream=side)
        g3 = na2d.forward_3d(x3["q"], x3["k"], x3["v"], x3["rpb"], 3, stream=side)
    side.synchronize()
    assert torch.equal(g1, w1) and torch.equal(g3, w3)


def test_two_streams_at_once():
    """Forward and backward of two problems launched on two streams together."""
    xa = dev(make_inputs((4, 2, 56, 56, 32), 7, "f16", seed=34, rpb_std=1.0))
    xb = dev(make_inputs((2, 2, 40, 44, 32), 7, "bf16", seed=35, rpb_std=1.0))

    def run(t, s):
        out, lse = na2d.forward_lse(t["q"], t["k"], t["v"], t["rpb"], 7, stream=s)
        g = torch.ones_like(out)
        return (out, lse) + na2d.backward(t["q"], t["k"], t["v"], t["rpb"], out, g, 7, stream=s, lse=lse)

    want_a, want_b = run(xa, None), run(xb, None)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sa):
        got_a = run(xa, sa)
    with torch.cuda.stream(sb):
        got_b = run(xb, sb)
    torch.cuda.synchronize()
    for got, want in ((got_a, want_a), (got_b, want_b)):
        for i, (a, b) in enumerate(zip(got, want)):
            if i == 5:  # the bias gradient is summed with float atomics: last bits may differ
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-6)
            else:
                assert torch.equal(a, b), i


@pytest.mark.parametrize("ks,shape,dtype", [(7, (2, 2, 40, 36, 32), "f16"), (7, (1, 1, 136, 16, 32), "bf16"),
                                            (21, (1, 1, 45, 38, 32), "bf16"), (13, (1, 2, 30, 29, 32), "bf16")],
                         ids=str)
def test_graph_replays(ks, shape, dtype):
    """Forward (with lse) and backward captured in one graph, replayed four
    times with fresh inputs copied in and eager work in between."""
    print("graph", shape, ks, dtype, flush=True)
    x = dev(make_inputs(shape, ks, dtype, seed=36, rpb_std=1.0))
    static = {n: t.clone() for n, t in x.items()}
    static["g"] = torch.randn(shape, device="cuda")

    def step(t):
        out, lse = na2d.forward_lse(t["q"], t["k"], t["v"], t["rpb"], ks)
        dq, dk, dv, drpb = na2d.backward(t["q"], t["k"], t["v"], t["rpb"], out, t["g"], ks, lse=lse)
        return out, lse, dq, dk, dv, drpb

    # warm up on a side stream (as graph capture requires), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step(static)
    for rep in range(4):
        fresh = {n: (t * (1.0 + 0.25 * rep)).to(t.dtype) for n, t in x.items()}
        fresh["g"] = torch.randn(shape, device="cuda")
        for n in fresh:
            static[n].copy_(fresh[n])
        graph.replay()
        torch.cuda.synchronize()
        eager = step(fresh)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            if i == 5:
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-6), (rep, i)
            else:
                assert torch.equal(a, b), (rep, i)
        # eager work between replays
        torch.matmul(torch.randn(256, 256, device="cuda"), torch.randn(256, 256, device="cuda"))
