"""Benchmark of the fused Neighborhood Attention forward on one MI355X.

One step = one fused forward launch over the whole batch of a workload, by
default NAT-Tiny stage 1 (B=32, 2 heads, 56x56, d=32, k=7, fp16 inputs, fp32
output), inputs already resident in HBM.  `--workload` also takes the other
NA2D shapes and the NA1D, NA3D and SASA workloads (see inputs.WORKLOADS).  The
timed region rotates over enough input/output sets (>= 1 GiB) that the 256 MB
Infinity Cache cannot hold them, so the figure is an HBM figure.  Prints one
JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--algo auto|valu|mfma]

``--gpus N`` with N > 1 is refused: this build measures one GPU (the op
shards over (batch, head) maps with no communication at all).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NA2D fwd queries/s and achieved HBM GB/s (% roofline), NAT-Tiny stage1 k=7"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
ALGOS = {"auto": 0, "valu": 1, "mfma": 2}
# kernel family -> its source (a committed traffic summary is used only when it
# was taken on the source as it is now)
KERNEL_SOURCES = {"na_valu": "na_valu.hip", "na2d_mfma": "na2d_mfma.hip",
                  "na2d_large_mfma": "na2d_large_mfma.hip",
                  "na1d_mfma": "na1d_mfma.hip", "na3d_mfma": "na3d_mfma.hip",
                  "na2d_bwd": "na2d_bwd_mfma.hip"}
# NA windows wider than this go to the wide-window kernel (the library's
# routing, csrc/na2d_api.cpp: halo_max_na_k)
HALO_MAX_NA_K = {"f16": 13, "bf16": 9}


def kernel_id(op: str, algo: int, k: int = 7, dtype: str = "f16") -> str:
    if algo == 1:
        return "na_valu"
    if op == "na2d" and k > HALO_MAX_NA_K.get(dtype, 13):
        return "na2d_large_mfma"
    return {"na1d": "na1d_mfma", "na3d": "na3d_mfma"}.get(op, "na2d_mfma")


def algorithmic_bytes(w) -> int:
    """Bytes the op itself must move: read q, k, v once, write fp32 out once,
    read the bias table once (halo re-reads are not counted)."""
    es = 4 if w.dtype == "f32" else 2
    per_query = 3 * w.d * es + 4 * w.d
    return w.queries * per_query + 4 * math.prod(w.rpb_shape)


def algorithmic_flops(w) -> int:
    """QK and AV: 2 * keys * d multiply-adds per query, a multiply-add = 2 flops."""
    return w.queries * 4 * w.keys_per_query * w.d


def source_digest(name: str) -> str:
    """First 16 hex digits of the SHA-256 of a kernel source followed by every
    header it may include (csrc/*.h, then include/*.h, each sorted by name) and
    the build script with its compiler flags, so that an edit to a shared
    header or a flag also marks a profile as stale."""
    csrc = os.path.join(ROOT, "vision_sliding_window_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    paths = [os.path.join(ROOT, "vision_sliding_window_amd", "_build.py"), os.path.join(csrc, name)]
    paths += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc)) if f.endswith(".h")]
    paths += [os.path.join(inc, f) for f in sorted(os.listdir(inc)) if f.endswith(".h")]
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def settle_clocks(launch, torch, min_ms: float):
    """Run `launch` untimed until at least `min_ms` of wall time has passed,
    before the warm-up steps. Under load the GPU raises its clocks over a few
    milliseconds; a benchmark that starts cold otherwise times that ramp.
    Measured at stage 1: 21.1-21.6 us per step after 20 warm-up launches alone,
    19.1 us after 2000. Returns the number of launches run."""
    n, t0 = 0, time.perf_counter()
    while min_ms > 0:
        for _ in range(32):
            launch(n)
            n += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            break
    return n


def read_traffic(workload: str, kid: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    kernel family `kid` on `workload`, if it was taken on the kernel source as
    it is now (else None)."""
    kernel_src = KERNEL_SOURCES[kid]
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.txt" % (kid, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    try:
        if vals.get("kernel_source_sha256_16") != source_digest(kernel_src):
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, x, seconds: float = 10.0):
    """The fp64 oracle as it stands, on the host cores, on a bounded sample of
    the same workload: repeated passes over a random sample of its queries (at
    most the whole workload) until about `seconds` of CPU time have passed."""
    import numpy as np
    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    if w.op == "na2d":
        def run(idx):
            oracle.na2d_forward_sampled(x.q64, x.k64, x.v64, x.rpb64, w.k, idx, nthreads=cores)
    else:
        ref = {"na1d": oracle.na1d_forward, "na3d": oracle.na3d_forward,
               "sasa2d": oracle.sasa2d_forward}[w.op]

        def run(idx):
            ref(x.q64, x.k64, x.v64, x.rpb64, w.k, idx=idx, nthreads=cores)
    rng = np.random.default_rng(1)
    probe = rng.choice(w.queries, size=min(w.queries, 4096), replace=False)
    t0 = time.perf_counter()
    run(probe)
    rate = probe.size / max(time.perf_counter() - t0, 1e-6)
    n = int(min(w.queries, max(probe.size, rate * seconds)))
    sample = rng.choice(w.queries, size=n, replace=False)
    t0 = time.perf_counter()
    done = 0
    while True:
        run(sample)
        done += n
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # a per-core figure: one thread on a smaller sample, about a tenth of the time
    n1 = int(min(n, max(64, rate / cores * seconds / 10)))
    t1 = time.perf_counter()
    if w.op == "na2d":
        oracle.na2d_forward_sampled(x.q64, x.k64, x.v64, x.rpb64, w.k, sample[:n1], nthreads=1)
    else:
        ref(x.q64, x.k64, x.v64, x.rpb64, w.k, idx=sample[:n1], nthreads=1)
    one = n1 / max(time.perf_counter() - t1, 1e-6)
    return {"value": done / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": "%d random queries of %s (seed 1), %d pass(es), fp64, %.1f s"
                      % (n, w.name, done // n, el),
            "cpu_model": cpu_model(), "one_thread_value": round(one, 1)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def d2d_copy_gbs(torch, dev, nbytes: int = 2 ** 30, reps: int = 10) -> float:
    """Read + write rate of a plain device-to-device copy of nbytes on this GPU."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def backward_bytes(w, with_lse: bool = False) -> int:
    """Bytes the gradients must move: read q, k, v, out and dout (and the
    forward's per-query log-sum-exp when it is reused), write dq, dk, dv once,
    read the bias table and write its gradient."""
    es = 4 if w.dtype == "f32" else 2
    per_query = 3 * w.d * es + 2 * 4 * w.d + 3 * 4 * w.d + (4 if with_lse else 0)
    return w.queries * per_query + 2 * 4 * math.prod(w.rpb_shape)


def bench_backward(args, w, wname, lib, dev, dtype_code):
    import torch
    from vision_sliding_window_amd import na2d
    from vision_sliding_window_amd.inputs import workload_inputs
    x = workload_inputs(w, seed=0)
    set_bytes = backward_bytes(w, with_lse=not args.recompute_stats)
    nsets = max(1, math.ceil(args.min_footprint_gib * 2 ** 30 / set_bytes))
    rpb = x.rpb.to(dev)
    q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    # the training forward: out and each query's log-sum-exp, which the
    # backward reuses unless --recompute-stats asks it to recompute them
    out0, lse0 = na2d.forward_lse(q0, k0, v0, rpb, w.k)
    if args.recompute_stats:
        lse0 = None
    g0 = torch.randn(w.shape, generator=torch.Generator().manual_seed(1)).to(dev)
    ws_bytes = na2d.na2d_backward_workspace_bytes(w.B, w.heads, w.H, w.W, w.k)
    f32 = dict(dtype=torch.float32, device=dev)
    sets = []
    for i in range(nsets):
        c = (lambda t: t.clone()) if i else (lambda t: t)
        sets.append((c(q0), c(k0), c(v0), c(out0), None if lse0 is None else c(lse0), c(g0),
                     torch.empty(w.shape, **f32),
                     torch.empty(w.shape, **f32), torch.empty(w.shape, **f32),
                     torch.empty(rpb.shape, **f32), torch.empty(ws_bytes // 4, **f32)))
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def launch(i):
        q, k, v, out, lse, g, dq, dk, dv, drpb, ws = sets[i % nsets]
        st = lib.na2d_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                               out.data_ptr(), None if lse is None else lse.data_ptr(),
                               g.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), drpb.data_ptr(), ws.data_ptr(), w.B, w.heads, w.H,
                               w.W, w.d, w.k, dtype_code, sptr)
        if st != 0:
            raise RuntimeError("na2d_backward failed: %s" % na2d.na2d_strerror(st))

    settled = settle_clocks(launch, torch, args.settle_ms)
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = set_bytes / (ms * 1e-3) / 1e9
    rec = {
        "metric": "NA2D bwd queries/s and achieved HBM GB/s (%% roofline), %s" % wname,
        "value": round(w.queries / (ms * 1e-3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic: Q,K,V ~ N(0,1), RPB ~ N(0,0.02), dout ~ N(0,1)",
        "config": {"workload": wname, "pass": "backward", "B": w.B, "heads": w.heads, "H": w.H,
                   "W": w.W, "d": w.d, "k": w.k, "rotating_sets": nsets,
                   "clock_settle_ms": args.settle_ms, "clock_settle_launches": settled,
                   # 16-bit inputs with d = 32 and k <= 25 run on the matrix cores
                   "kernel": "mfma" if w.dtype != "f32" and w.d == 32 and w.k <= 25 else "valu",
                   "roofline_scope": "whole backward (all its kernels)",
                   "softmax_stats": "recomputed" if lse0 is None else "from the forward (lse)",
                   "algorithmic_bytes_per_step": set_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": (lambda t: None if t is None else int(t))(
                         read_traffic(wname, "na2d_bwd"))},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_backward(w, x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def cpu_baseline_backward(w, x, seconds):
    """The fp64 gradient oracle as it stands on the host cores: whole-workload
    passes until about `seconds` have passed (at least one)."""
    import numpy as np
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        cores = min(cores, int(env))
    g = np.random.default_rng(1).standard_normal(x.q64.shape)
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.na2d_backward(x.q64, x.k64, x.v64, x.rpb64, g, w.k, nthreads=cores)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n * w.queries / el, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": "%d whole pass(es) over %s, fp64, %.1f s" % (n, w.name, el)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="untimed launches for at least this long before the warm-up steps, so that "
                         "the GPU clocks have settled (0: none)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--algo", default="auto", choices=sorted(ALGOS))
    ap.add_argument("--min-footprint-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-floor", action="store_true",
                    help="skip the streaming reference leg (16-bit workloads)")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the cache-resident (single-set) timing")
    ap.add_argument("--q-scale", type=float, default=1.0,
                    help="stress: Q times this (peaked softmax); 1 is the graded input")
    ap.add_argument("--hot", action="store_true",
                    help="(the default) also time one cache-resident input set, reported separately")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--recompute-stats", action="store_true",
                    help="--backward without the forward's log-sum-exp (the backward recomputes it)")
    ap.add_argument("--backward", action="store_true",
                    help="time the NA2D gradients (na2d_backward) instead of the forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device-to-device copy of MIB "
                         "MiB a few times (calibrates HBM byte counters under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the NA2D forward shards over (batch, head) "
              "maps with no communication, so N > 1 is not run here", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": max(args.steps, 1)}), flush=True)
        return
    from vision_sliding_window_amd import na2d
    from vision_sliding_window_amd.inputs import BENCH_WORKLOAD, WORKLOADS, workload_inputs

    wname = args.workload or BENCH_WORKLOAD
    w = WORKLOADS[wname]
    lib = na2d.load()  # raises if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dtype_code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    algo = ALGOS[args.algo]
    # the grid and window of the general entry point: [B, heads, D, H, W], (kd, kh, kw)
    grid = (w.depth, w.H, w.W)
    window = {"na1d": (1, 1, w.k), "na3d": (w.k, w.k, w.k)}.get(w.op, (1, w.k, w.k))
    mode = na2d.NA_WINDOW_SASA if w.op == "sasa2d" else na2d.NA_WINDOW_NA
    if algo == 0:  # the family the library's own automatic choice resolves to
        algo = na2d.na_select_algo_nd(*grid, w.d, window, mode, dtype_code)
        if algo < 0:
            raise RuntimeError("unsupported workload: %s" % na2d.na2d_strerror(algo))
    algo_name = {1: "valu", 2: "mfma"}[algo]

    if args.backward:
        if w.op != "na2d":
            print("--backward covers the NA2D workloads", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args, w, wname, lib, dev, dtype_code)

    x = workload_inputs(w, seed=0, q_scale=args.q_scale)
    set_bytes = algorithmic_bytes(w)
    nsets = max(1, math.ceil(args.min_footprint_gib * 2 ** 30 / set_bytes))
    q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    rpb = x.rpb.to(dev)
    sets = []
    for i in range(nsets):
        sets.append((q0.clone() if i else q0, k0.clone() if i else k0, v0.clone() if i else v0,
                     torch.empty(w.shape, dtype=torch.float32, device=dev)))
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    def launch(i):
        q, k, v, out = sets[i % nsets]
        if w.op == "na2d":
            st = lib.na2d_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                     out.data_ptr(), w.B, w.heads, w.H, w.W, w.d, w.k, dtype_code,
                                     algo, sptr)
        else:
            st = lib.na_forward_nd(q.data_ptr(), k.data_ptr(), v.data_ptr(), rpb.data_ptr(),
                                   out.data_ptr(), w.B, w.heads, *grid, w.d, *window, mode,
                                   dtype_code, algo, sptr)
        if st != 0:
            raise RuntimeError("forward failed: %s" % na2d.na2d_strerror(st))

    settled = settle_clocks(launch, torch, args.settle_ms)
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        launch(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    hot_ms = None
    if not args.no_hot:  # cache-resident figure (one set, L2/MALL hits), labelled as such
        hs = torch.cuda.Event(enable_timing=True)
        he = torch.cuda.Event(enable_timing=True)
        hs.record(stream)
        for _ in range(args.steps):
            launch(0)
        he.record(stream)
        torch.cuda.synchronize()
        hot_ms = hs.elapsed_time(he) / args.steps

    # labelled reference leg: a plain streaming kernel that reads the same
    # three 16-bit inputs and writes the same fp32 output, once each, over the
    # same rotating sets -- the rate a launch of these bytes gets with no
    # attention work (not part of the step)
    floor_ms = None
    if w.dtype != "f32" and not args.no_stream_floor:
        elems = w.queries * w.d

        def stream_ref(i):
            q, k, v, out = sets[i % nsets]
            st = lib.na_stream_reference(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         elems, sptr)
            if st != 0:
                raise RuntimeError("stream reference failed: %s" % na2d.na2d_strerror(st))

        for i in range(args.warmup):
            stream_ref(i)
        fs, fe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fs.record(stream)
        for i in range(args.steps):
            stream_ref(i)
        fe.record(stream)
        torch.cuda.synchronize()
        floor_ms = fs.elapsed_time(fe) / args.steps

    copy_gbs = d2d_copy_gbs(torch, dev)
    value = w.queries / (ms * 1e-3)
    gbs = set_bytes / (ms * 1e-3) / 1e9
    tflops = algorithmic_flops(w) / (ms * 1e-3) / 1e12
    traffic = read_traffic(wname, kernel_id(w.op, algo, w.k, w.dtype))
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else int(traffic)}
    rec = {
        "metric": METRIC if wname == BENCH_WORKLOAD else
        "%s fwd queries/s and achieved HBM GB/s (%% roofline), %s" % (w.op.upper(), wname),
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: Q,K,V ~ N(0,1), RPB ~ N(0,0.02), seed 0" +
                ("" if args.q_scale == 1.0 else "; stress: Q x %g (not graded)" % args.q_scale),
        "config": {"workload": wname, "op": w.op, "B": w.B, "heads": w.heads, "D": w.depth,
                   "H": w.H, "W": w.W, "d": w.d, "k": w.k, "kernel": algo_name,
                   "rotating_sets": nsets,
                   "clock_settle_ms": args.settle_ms, "clock_settle_launches": settled,
                   "footprint_bytes": nsets * set_bytes, "algorithmic_bytes_per_step": set_bytes,
                   "hot_ms_per_step": None if hot_ms is None else round(hot_ms, 6),
                   "stream_floor_us": None if floor_ms is None else round(floor_ms * 1e3, 3),
                   "stream_floor_note": "na_stream_reference over the same rotating sets: "
                                        "the same bytes read and written once, no attention",
                   "frac_of_stream_floor": None if floor_ms is None else round(floor_ms / ms, 4),
                   "useful_tflops": round(tflops, 2),
                   "d2d_copy_gbs": round(copy_gbs, 1),
                   "frac_of_d2d_copy": round(gbs / copy_gbs, 4),
                   "q_scale": args.q_scale},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
