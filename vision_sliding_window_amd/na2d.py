"""Python binding of libna2d.so (C ABI in include/na2d.h): argument marshalling only.

The functions named like the C entry points take raw device pointers (ints)
or torch tensors (their ``data_ptr()`` is passed) and return the C status.
``forward`` is a convenience that allocates the fp32 output with torch and
raises on a non-zero status.  Every step of the attention runs in the HIP
library; if it is missing this module raises on first use -- there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libna2d.so")

NA2D_F32, NA2D_F16, NA2D_BF16 = 0, 1, 2
NA2D_ALGO_AUTO, NA2D_ALGO_VALU, NA2D_ALGO_MFMA = 0, 1, 2
NA_WINDOW_NA, NA_WINDOW_SASA = 0, 1
NA2D_OK = 0
NA2D_ERR_NULL = -1
NA2D_ERR_SHAPE = -2
NA2D_ERR_KSIZE = -3
NA2D_ERR_DTYPE = -4
NA2D_ERR_UNSUPPORTED = -5
NA2D_ERR_ALIGN = -6
NA2D_ERR_ALIAS = -7
NA2D_ERR_HIP = -8
NA2D_ERR_ALGO = -9
NA2D_ERR_SCRATCH = -10
NA2D_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ["na2d_forward", "na2d_forward_ex", "na2d_forward_lse", "na2d_check_args",
           "na2d_select_algo",
           "na_select_algo_nd",
           "na2d_strerror", "na2d_last_error", "na2d_version", "na_forward_nd",
           "na_check_args_nd", "na1d_forward", "na3d_forward", "sasa2d_forward",
           "na2d_backward", "na2d_backward_workspace_bytes", "na2d_backward_check_args",
           "na2d_backward_select_algo", "na2d_occupancy_queries", "na_stream_reference",
           "na2d_backward_noalloc"]

TORCH_DTYPE_CODE = {torch.float32: NA2D_F32, torch.float16: NA2D_F16, torch.bfloat16: NA2D_BF16}

_lib = None


class NA2DError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        msg = "na2d status %d: %s" % (status, na2d_strerror(status))
        if detail:
            msg += " (%s)" % detail
        super().__init__(msg)
        self.status = status


def load() -> ctypes.CDLL:
    """Load libna2d.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError("libna2d.so not built: run `python -c 'import __graft_entry__ as g; "
                              "g.build()'` or `python vision_sliding_window_amd/_build.py`")
        lib = ctypes.CDLL(LIBRARY)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.na2d_forward.argtypes = [P, P, P, P, P] + [I] * 7 + [P]
        lib.na2d_forward.restype = I
        lib.na2d_forward_ex.argtypes = [P, P, P, P, P] + [I] * 8 + [P]
        lib.na2d_forward_ex.restype = I
        lib.na2d_forward_lse.argtypes = [P] * 6 + [I] * 7 + [P]
        lib.na2d_forward_lse.restype = I
        lib.na2d_check_args.argtypes = [P, P, P, P, P] + [I] * 8
        lib.na2d_check_args.restype = I
        lib.na2d_select_algo.argtypes = [I] * 5
        lib.na2d_select_algo.restype = I
        lib.na_select_algo_nd.argtypes = [I] * 9
        lib.na_select_algo_nd.restype = I
        lib.na2d_strerror.argtypes = [I]
        lib.na2d_strerror.restype = ctypes.c_char_p
        lib.na2d_last_error.argtypes = []
        lib.na2d_last_error.restype = ctypes.c_char_p
        lib.na2d_version.argtypes = []
        lib.na2d_version.restype = I
        lib.na_forward_nd.argtypes = [P, P, P, P, P] + [I] * 12 + [P]
        lib.na_forward_nd.restype = I
        lib.na_check_args_nd.argtypes = [P, P, P, P, P] + [I] * 12
        lib.na_check_args_nd.restype = I
        lib.na1d_forward.argtypes = [P, P, P, P, P] + [I] * 6 + [P]
        lib.na1d_forward.restype = I
        lib.na3d_forward.argtypes = [P, P, P, P, P] + [I] * 8 + [P]
        lib.na3d_forward.restype = I
        lib.sasa2d_forward.argtypes = [P, P, P, P, P] + [I] * 7 + [P]
        lib.sasa2d_forward.restype = I
        lib.na2d_backward.argtypes = [P] * 12 + [I] * 7 + [P]
        lib.na2d_backward.restype = I
        lib.na2d_backward_workspace_bytes.argtypes = [I] * 5
        lib.na2d_backward_workspace_bytes.restype = ctypes.c_longlong
        lib.na2d_backward_check_args.argtypes = [P] * 12 + [I] * 7
        lib.na2d_backward_check_args.restype = I
        lib.na2d_backward_select_algo.argtypes = [I] * 5
        lib.na2d_backward_select_algo.restype = I
        lib.na2d_occupancy_queries.argtypes = []
        lib.na2d_occupancy_queries.restype = ctypes.c_longlong
        lib.na_stream_reference.argtypes = [P, P, P, P, ctypes.c_longlong, P]
        lib.na_stream_reference.restype = I
        lib.na2d_backward_noalloc.argtypes = [P] * 11 + [I] * 7 + [P]
        lib.na2d_backward_noalloc.restype = I
        _lib = lib
    return _lib


def _addr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(s):
    if s is None:
        return None
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def na2d_forward(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, stream=None) -> int:
    return load().na2d_forward(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out),
                               B, heads, H, W, d, ksize, dtype, _stream(stream))


def na2d_forward_ex(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, algo,
                    stream=None) -> int:
    return load().na2d_forward_ex(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out),
                                  B, heads, H, W, d, ksize, dtype, algo, _stream(stream))


def na2d_forward_lse(q, k, v, rpb, out, lse, B, heads, H, W, d, ksize, dtype,
                     stream=None) -> int:
    return load().na2d_forward_lse(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out),
                                   _addr(lse), B, heads, H, W, d, ksize, dtype, _stream(stream))


def na2d_check_args(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, algo) -> int:
    return load().na2d_check_args(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out),
                                  B, heads, H, W, d, ksize, dtype, algo)


def na2d_select_algo(H, W, d, ksize, dtype) -> int:
    return load().na2d_select_algo(H, W, d, ksize, dtype)


def na_select_algo_nd(D, H, W, d, window, mode, dtype) -> int:
    """The kernel family AUTO picks for na_forward_nd; window = (kd, kh, kw)."""
    kd, kh, kw = window
    return load().na_select_algo_nd(D, H, W, d, kd, kh, kw, mode, dtype)


def na_forward_nd(q, k, v, rpb, out, B, heads, D, H, W, d, kd, kh, kw, mode, dtype, algo,
                  stream=None) -> int:
    return load().na_forward_nd(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out), B, heads,
                                D, H, W, d, kd, kh, kw, mode, dtype, algo, _stream(stream))


def na_check_args_nd(q, k, v, rpb, out, B, heads, D, H, W, d, kd, kh, kw, mode, dtype,
                     algo) -> int:
    return load().na_check_args_nd(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out), B,
                                   heads, D, H, W, d, kd, kh, kw, mode, dtype, algo)


def na1d_forward(q, k, v, rpb, out, B, heads, L, d, ksize, dtype, stream=None) -> int:
    return load().na1d_forward(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out), B, heads,
                               L, d, ksize, dtype, _stream(stream))


def na3d_forward(q, k, v, rpb, out, B, heads, D, H, W, d, ksize, dtype, stream=None) -> int:
    return load().na3d_forward(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out), B, heads,
                               D, H, W, d, ksize, dtype, _stream(stream))


def sasa2d_forward(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, stream=None) -> int:
    return load().sasa2d_forward(_addr(q), _addr(k), _addr(v), _addr(rpb), _addr(out), B, heads,
                                 H, W, d, ksize, dtype, _stream(stream))


def na2d_backward(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, workspace, B, heads, H, W, d,
                  ksize, dtype, stream=None) -> int:
    return load().na2d_backward(*(_addr(t) for t in (q, k, v, rpb, out, lse, dout, dq, dk, dv,
                                                     drpb, workspace)),
                                B, heads, H, W, d, ksize, dtype, _stream(stream))


def na2d_backward_noalloc(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, B, heads, H, W, d,
                          ksize, dtype, stream=None) -> int:
    return load().na2d_backward_noalloc(*(_addr(t) for t in (q, k, v, rpb, out, lse, dout, dq, dk,
                                                             dv, drpb)),
                                        B, heads, H, W, d, ksize, dtype, _stream(stream))


def na2d_backward_workspace_bytes(B, heads, H, W, ksize) -> int:
    return load().na2d_backward_workspace_bytes(B, heads, H, W, ksize)


def na2d_backward_check_args(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, workspace, B, heads,
                             H, W, d, ksize, dtype) -> int:
    return load().na2d_backward_check_args(*(_addr(t) for t in (q, k, v, rpb, out, lse, dout, dq,
                                                                dk, dv, drpb, workspace)),
                                           B, heads, H, W, d, ksize, dtype)


def na2d_backward_select_algo(H, W, d, ksize, dtype) -> int:
    return load().na2d_backward_select_algo(H, W, d, ksize, dtype)


def na2d_occupancy_queries() -> int:
    return load().na2d_occupancy_queries()


def na_stream_reference(a, b, c, out, elems, stream=None) -> int:
    return load().na_stream_reference(_addr(a), _addr(b), _addr(c), _addr(out), elems,
                                      _stream(stream))


def na2d_strerror(status: int) -> str:
    return load().na2d_strerror(status).decode()


def na2d_last_error() -> str:
    return load().na2d_last_error().decode()


def na2d_version() -> int:
    return load().na2d_version()


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rpb, ksize: int,
            algo: int = NA2D_ALGO_AUTO, out: torch.Tensor | None = None, stream=None):
    """Fused NA2D forward on [B, heads, H, W, d] device tensors; returns fp32 out.

    The tensors must be contiguous and on the GPU; ``stream`` defaults to
    torch's current stream on q's device."""
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 5):
            raise ValueError("q, k, v must be contiguous 5-d GPU tensors [B, heads, H, W, d]")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if rpb is not None and not (rpb.is_cuda and rpb.is_contiguous() and rpb.dtype == torch.float32):
        raise ValueError("rpb must be a contiguous float32 GPU tensor [heads, 2k-1, 2k-1]")
    B, heads, H, W, d = q.shape
    if rpb is not None and tuple(rpb.shape) != (heads, 2 * ksize - 1, 2 * ksize - 1):
        raise ValueError("rpb must have shape [heads, 2k-1, 2k-1]")
    if q.dtype not in TORCH_DTYPE_CODE:
        raise ValueError("unsupported dtype %s" % q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = na2d_forward_ex(q, k, v, rpb, out, B, heads, H, W, d, ksize, TORCH_DTYPE_CODE[q.dtype],
                         algo, stream)
    if st != NA2D_OK:
        raise NA2DError(st, na2d_last_error() if st == NA2D_ERR_HIP else "")
    return out


def forward_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rpb, ksize: int, stream=None):
    """The training forward: (out, lse) with lse [B, heads, H, W] float32 the
    log-sum-exp of each query's logits, for ``backward(..., lse=lse)``."""
    _check_inputs(q, k, v, rpb, 5, (q.shape[1], 2 * ksize - 1, 2 * ksize - 1))
    B, heads, H, W, d = q.shape
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:4], dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = na2d_forward_lse(q, k, v, rpb, out, lse, B, heads, H, W, d, ksize,
                          TORCH_DTYPE_CODE[q.dtype], stream)
    if st != NA2D_OK:
        raise NA2DError(st, na2d_last_error() if st == NA2D_ERR_HIP else "")
    return out, lse


def _check_inputs(q, k, v, rpb, ndim, rpb_shape):
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == ndim):
            raise ValueError("q, k, v must be contiguous %d-d GPU tensors" % ndim)
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    if q.dtype not in TORCH_DTYPE_CODE:
        raise ValueError("unsupported dtype %s" % q.dtype)
    if rpb is not None:
        if not (rpb.is_cuda and rpb.is_contiguous() and rpb.dtype == torch.float32):
            raise ValueError("rpb must be a contiguous float32 GPU tensor")
        if tuple(rpb.shape) != tuple(rpb_shape):
            raise ValueError("rpb must have shape %s" % (tuple(rpb_shape),))


def _run(fn, q, out, stream, *args):
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fn(*args[:4], out, *args[4:], stream)
    if st != NA2D_OK:
        raise NA2DError(st, na2d_last_error() if st == NA2D_ERR_HIP else "")
    return out


def forward_1d(q, k, v, rpb, ksize: int, out=None, stream=None):
    """NA1D on [B, heads, L, d] device tensors (rpb [heads, 2k-1]); returns fp32 out."""
    _check_inputs(q, k, v, rpb, 4, (q.shape[1], 2 * ksize - 1))
    B, heads, L, d = q.shape
    return _run(na1d_forward, q, out, stream, q, k, v, rpb, B, heads, L, d, ksize,
                TORCH_DTYPE_CODE[q.dtype])


def forward_3d(q, k, v, rpb, ksize: int, out=None, stream=None):
    """NA3D on [B, heads, D, H, W, d] device tensors (rpb [heads, 2k-1, 2k-1, 2k-1])."""
    n = 2 * ksize - 1
    _check_inputs(q, k, v, rpb, 6, (q.shape[1], n, n, n))
    B, heads, D, H, W, d = q.shape
    return _run(na3d_forward, q, out, stream, q, k, v, rpb, B, heads, D, H, W, d, ksize,
                TORCH_DTYPE_CODE[q.dtype])


def forward_sasa2d(q, k, v, rpb, ksize: int, out=None, stream=None):
    """SASA (centred windows, zero padding) on [B, heads, H, W, d] device tensors."""
    _check_inputs(q, k, v, rpb, 5, (q.shape[1], 2 * ksize - 1, 2 * ksize - 1))
    B, heads, H, W, d = q.shape
    return _run(sasa2d_forward, q, out, stream, q, k, v, rpb, B, heads, H, W, d, ksize,
                TORCH_DTYPE_CODE[q.dtype])


def forward_nd(q, k, v, rpb, window, mode=NA_WINDOW_NA, algo=NA2D_ALGO_AUTO, out=None,
               stream=None):
    """The general form on [B, heads, D, H, W, d] tensors with a (kd, kh, kw) window."""
    kd, kh, kw = window
    _check_inputs(q, k, v, rpb, 6, (q.shape[1], 2 * kd - 1, 2 * kh - 1, 2 * kw - 1))
    B, heads, D, H, W, d = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = na_forward_nd(q, k, v, rpb, out, B, heads, D, H, W, d, kd, kh, kw, mode,
                       TORCH_DTYPE_CODE[q.dtype], algo, stream)
    if st != NA2D_OK:
        raise NA2DError(st, na2d_last_error() if st == NA2D_ERR_HIP else "")
    return out


def backward(q, k, v, rpb, out, dout, ksize: int, stream=None, lse=None):
    """Gradients (dq, dk, dv, drpb) of the NA2D forward on device tensors: q, k,
    v, rpb as for ``forward``, out its float32 output, dout float32 of out's
    shape, lse (optional) the log-sum-exp from ``forward_lse``.  drpb is None
    when rpb is None.  Allocates the outputs and the workspace with torch."""
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 5):
            raise ValueError("q, k, v must be contiguous 5-d GPU tensors [B, heads, H, W, d]")
    for t in (out, dout):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and t.shape == q.shape):
            raise ValueError("out and dout must be contiguous float32 GPU tensors shaped like q")
    B, heads, H, W, d = q.shape
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty(q.shape, **f32), torch.empty(q.shape, **f32), torch.empty(q.shape, **f32)
    drpb = None if rpb is None else torch.empty(rpb.shape, **f32)
    ws = torch.empty(max(1, na2d_backward_workspace_bytes(B, heads, H, W, ksize) // 4), **f32)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if lse is not None and not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32
                                and lse.shape == q.shape[:4]):
        raise ValueError("lse must be a contiguous float32 GPU tensor [B, heads, H, W]")
    st = na2d_backward(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, ws, B, heads, H, W, d,
                       ksize, TORCH_DTYPE_CODE[q.dtype], stream)
    if st != NA2D_OK:
        raise NA2DError(st, na2d_last_error() if st == NA2D_ERR_HIP else "")
    return dq, dk, dv, drpb
