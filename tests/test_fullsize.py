"""Every workload at its full size, launched as the benchmark launches it
(automatic kernel selection, one launch over the whole batch), against the
fp64 oracle on every output element: all queries of all (b, head) maps, the
definition applied "for every pixel" (Neighborhood Attention Transformer,
CSDN translation, section 3.1, Eq. 2-4).

Tolerances as in the small-map parity tests: max-abs 1e-5 for float32
inputs, 2e-3 for fp16/bf16 inputs with fp32 accumulation.  The whole-output
max-abs error of each workload is printed.
"""
import numpy as np
import pytest
import torch

import conftest
import oracle
from vision_sliding_window_amd import na2d
from vision_sliding_window_amd.inputs import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def oracle_full(w, x):
    """The fp64 oracle over the whole workload, shaped [queries, d]."""
    if w.op == "na2d":
        want = oracle.na2d_forward(x.q64, x.k64, x.v64, x.rpb64, w.k)
    else:
        ref = {"na1d": oracle.na1d_forward, "na3d": oracle.na3d_forward,
               "sasa2d": oracle.sasa2d_forward}[w.op]
        want = ref(x.q64, x.k64, x.v64, x.rpb64, w.k)
    return want.reshape(-1, w.d)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_full_size_every_output(name):
    w = WORKLOADS[name]
    print("workload", name, flush=True)
    x = workload_inputs(w, seed=0)
    dev = torch.device("cuda")
    fwd = {"na2d": na2d.forward, "na1d": na2d.forward_1d, "na3d": na2d.forward_3d,
           "sasa2d": na2d.forward_sasa2d}[w.op]
    out = fwd(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.rpb.to(dev), w.k)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(-1, w.d)
    del out
    assert np.isfinite(got).all()
    want = oracle_full(w, x)
    assert got.shape == want.shape == (w.queries, w.d)
    err = np.abs(got - want)
    worst = int(np.argmax(err.max(axis=1)))
    line = ("%-24s max|err| %.3g over all %d queries x %d dims (tolerance %.0e)"
            % (name, err.max(), w.queries, w.d, TOL[w.dtype]))
    print(line, flush=True)
    conftest.PARITY_REPORT.append(line)
    assert err.max() <= TOL[w.dtype], "%s: max|err| %.3g > %.3g at query %d" % (
        name, err.max(), TOL[w.dtype], worst)
