"""fp64 CPU oracle for 2D Neighborhood Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The product library never loads it
and shares no code with it.

The arithmetic lives in ``na2d_oracle.c`` (plain loops, double precision,
OpenMP over rows); this module only builds and calls it.  Definition: the NA
equations 2-4 of "Neighborhood Attention Transformer" (CSDN translation,
section 3.1), with the per-axis clamped window of section 1 / section 3.1 and
the qiita article's border figure.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "na2d_oracle.c")
LIBRARY = os.path.join(_HERE, "libna2d_oracle.so")
ND_SOURCE = os.path.join(_HERE, "na_nd_oracle.c")
ND_LIBRARY = os.path.join(_HERE, "libna_nd_oracle.so")
BWD_SOURCE = os.path.join(_HERE, "na2d_bwd_oracle.c")
BWD_LIBRARY = os.path.join(_HERE, "libna2d_bwd_oracle.so")

NA, SASA = 0, 1  # window modes of the N-axis oracle


def compile_oracle(src: str, out: str) -> str:
    """Compile an oracle source with gcc (OpenMP, -O2, no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_oracle(SOURCE, LIBRARY)
    if force or not os.path.exists(ND_LIBRARY):
        compile_oracle(ND_SOURCE, ND_LIBRARY)
    if force or not os.path.exists(BWD_LIBRARY):
        compile_oracle(BWD_SOURCE, BWD_LIBRARY)
    return LIBRARY


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.na2d_oracle_window_start.argtypes = [I, I, I]
        lib.na2d_oracle_window_start.restype = I
        lib.na2d_oracle_f64.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I]
        lib.na2d_oracle_f64.restype = I
        lib.na2d_oracle_f64_lse.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I]
        lib.na2d_oracle_f64_lse.restype = I
        lib.na2d_oracle_f64_sampled.argtypes = [P, P, P, P, P, I64, P, I, I, I, I, I, I, I]
        lib.na2d_oracle_f64_sampled.restype = I
        self.lib = lib
        self.path = path

    def window_start(self, i: int, k: int, L: int) -> int:
        """Start of the clamped window of size k around index i on an axis of length L."""
        return self.lib.na2d_oracle_window_start(i, k, L)

    def na2d_forward(self, q, k, v, rpb, ksize: int, nthreads: int = 0) -> np.ndarray:
        """NA2D forward.  q, k, v: [B, heads, H, W, d]; rpb: [heads, 2k-1, 2k-1] or None."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        assert q.ndim == 5 and q.shape == k.shape == v.shape
        B, heads, H, W, d = q.shape
        if rpb is not None:
            rpb = _f64(rpb)
            assert rpb.shape == (heads, 2 * ksize - 1, 2 * ksize - 1)
        out = np.empty_like(q)
        rc = self.lib.na2d_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out),
                                      B, heads, H, W, d, ksize, nthreads)
        if rc != 0:
            raise ValueError("oracle rejected sizes B=%d heads=%d H=%d W=%d d=%d k=%d"
                             % (B, heads, H, W, d, ksize))
        return out

    def na2d_forward_lse(self, q, k, v, rpb, ksize: int, nthreads: int = 0):
        """(out, lse): the forward and each query's log softmax denominator
        ln sum_j exp((q.k_j + B_j)/sqrt(d)), lse shaped [B, heads, H, W]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        assert q.ndim == 5 and q.shape == k.shape == v.shape
        B, heads, H, W, d = q.shape
        if rpb is not None:
            rpb = _f64(rpb)
            assert rpb.shape == (heads, 2 * ksize - 1, 2 * ksize - 1)
        out = np.empty_like(q)
        lse = np.empty(q.shape[:4], dtype=np.float64)
        rc = self.lib.na2d_oracle_f64_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(out),
                                          _ptr(lse), B, heads, H, W, d, ksize, nthreads)
        if rc != 0:
            raise ValueError("oracle rejected sizes")
        return out, lse

    def na2d_forward_sampled(self, q, k, v, rpb, ksize: int, idx, nthreads: int = 0):
        """Outputs [n, d] for the queries with linear index ((b*heads+h)*H+y)*W+x."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, heads, H, W, d = q.shape
        if rpb is not None:
            rpb = _f64(rpb)
            assert rpb.shape == (heads, 2 * ksize - 1, 2 * ksize - 1)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        out = np.empty((idx.size, d), dtype=np.float64)
        rc = self.lib.na2d_oracle_f64_sampled(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(idx),
                                              idx.size, _ptr(out), B, heads, H, W, d, ksize,
                                              nthreads)
        if rc != 0:
            raise ValueError("oracle rejected the request")
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build()
        _default = Oracle(LIBRARY)
    return _default


def window_start(i: int, k: int, L: int) -> int:
    return default().window_start(i, k, L)


def na2d_forward(q, k, v, rpb, ksize: int, nthreads: int = 0) -> np.ndarray:
    return default().na2d_forward(q, k, v, rpb, ksize, nthreads)


def na2d_forward_sampled(q, k, v, rpb, ksize: int, idx, nthreads: int = 0) -> np.ndarray:
    return default().na2d_forward_sampled(q, k, v, rpb, ksize, idx, nthreads)


def na2d_forward_lse(q, k, v, rpb, ksize: int, nthreads: int = 0):
    return default().na2d_forward_lse(q, k, v, rpb, ksize, nthreads)


class OracleND:
    """ctypes front of the N-axis oracle (na_nd_oracle.c): NA over 1, 2 or 3
    axes (mode NA) and SASA windows on a zero-padded input (mode SASA)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.na_nd_window_start.argtypes = [I, I, I, I]
        lib.na_nd_window_start.restype = I
        lib.na_nd_oracle_f64.argtypes = [P, P, P, P, P, I64, P] + [I] * 11
        lib.na_nd_oracle_f64.restype = I
        self.lib = lib
        self.path = path

    def window_start(self, i: int, k: int, L: int, mode: int = NA) -> int:
        return self.lib.na_nd_window_start(i, k, L, mode)

    def forward(self, q, k, v, rpb, ksizes, mode: int = NA, idx=None, nthreads: int = 0):
        """q, k, v: [B, heads, L0, L1, L2, d]; rpb: [heads, 2k0-1, 2k1-1, 2k2-1] or None.
        Returns [B, heads, L0, L1, L2, d], or [n, d] for the linear query indices idx."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        assert q.ndim == 6 and q.shape == k.shape == v.shape
        B, heads, L0, L1, L2, d = q.shape
        k0, k1, k2 = ksizes
        if rpb is not None:
            rpb = _f64(rpb)
            assert rpb.shape == (heads, 2 * k0 - 1, 2 * k1 - 1, 2 * k2 - 1)
        if idx is None:
            out = np.empty_like(q)
            n = q.size // d
        else:
            idx = np.ascontiguousarray(idx, dtype=np.int64)
            out = np.empty((idx.size, d), dtype=np.float64)
            n = idx.size
        rc = self.lib.na_nd_oracle_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(idx), n,
                                       _ptr(out), B, heads, L0, L1, L2, d, k0, k1, k2, mode,
                                       nthreads)
        if rc != 0:
            raise ValueError("oracle rejected sizes %s k=%s mode=%d" % (q.shape, ksizes, mode))
        return out


_default_nd = None


def default_nd() -> OracleND:
    global _default_nd
    if _default_nd is None:
        if not os.path.exists(ND_LIBRARY):
            build()
        _default_nd = OracleND(ND_LIBRARY)
    return _default_nd


def na1d_forward(q, k, v, rpb, ksize: int, idx=None, nthreads: int = 0, orc=None):
    """NA1D: q, k, v [B, heads, L, d], rpb [heads, 2k-1] or None."""
    orc = orc or default_nd()
    B, heads, L, d = q.shape
    sh = (B, heads, 1, 1, L, d)
    r = None if rpb is None else np.asarray(rpb).reshape(heads, 1, 1, 2 * ksize - 1)
    out = orc.forward(np.reshape(q, sh), np.reshape(k, sh), np.reshape(v, sh), r, (1, 1, ksize),
                      NA, idx, nthreads)
    return out if idx is not None else out.reshape(q.shape)


def na3d_forward(q, k, v, rpb, ksize: int, idx=None, nthreads: int = 0, orc=None):
    """NA3D: q, k, v [B, heads, D, H, W, d], rpb [heads, 2k-1, 2k-1, 2k-1] or None."""
    orc = orc or default_nd()
    return orc.forward(q, k, v, rpb, (ksize, ksize, ksize), NA, idx, nthreads)


def sasa2d_forward(q, k, v, rpb, ksize: int, idx=None, nthreads: int = 0, orc=None):
    """SASA on a 2D map (centred k x k windows, zero padding): q, k, v
    [B, heads, H, W, d], rpb [heads, 2k-1, 2k-1] or None."""
    orc = orc or default_nd()
    B, heads, H, W, d = q.shape
    sh = (B, heads, 1, H, W, d)
    r = None if rpb is None else np.asarray(rpb).reshape(heads, 1, 2 * ksize - 1, 2 * ksize - 1)
    out = orc.forward(np.reshape(q, sh), np.reshape(k, sh), np.reshape(v, sh), r, (1, ksize, ksize),
                      SASA, idx, nthreads)
    return out if idx is not None else out.reshape(q.shape)


class OracleBwd:
    """ctypes front of the NA2D gradient oracle (na2d_bwd_oracle.c)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.na2d_oracle_backward_f64.argtypes = [P] * 9 + [I] * 7
        lib.na2d_oracle_backward_f64.restype = I
        self.lib = lib
        self.path = path

    def backward(self, q, k, v, rpb, dout, ksize: int, nthreads: int = 0):
        """Gradients (dq, dk, dv, drpb) of sum(dout * NA2D(q, k, v, rpb)); drpb is
        None when rpb is None."""
        q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
        assert q.ndim == 5 and q.shape == k.shape == v.shape == g.shape
        B, heads, H, W, d = q.shape
        drpb = None
        if rpb is not None:
            rpb = _f64(rpb)
            assert rpb.shape == (heads, 2 * ksize - 1, 2 * ksize - 1)
            drpb = np.empty_like(rpb)
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        rc = self.lib.na2d_oracle_backward_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(rpb), _ptr(g),
                                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drpb), B, heads,
                                               H, W, d, ksize, nthreads)
        if rc != 0:
            raise ValueError("backward oracle rejected sizes %s k=%d" % (q.shape, ksize))
        return dq, dk, dv, drpb


_default_bwd = None


def default_bwd() -> OracleBwd:
    global _default_bwd
    if _default_bwd is None:
        if not os.path.exists(BWD_LIBRARY):
            build()
        _default_bwd = OracleBwd(BWD_LIBRARY)
    return _default_bwd


def na2d_backward(q, k, v, rpb, dout, ksize: int, nthreads: int = 0):
    return default_bwd().backward(q, k, v, rpb, dout, ksize, nthreads)
