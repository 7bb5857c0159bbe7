"""The C-ABI library loads, exports every function include/na2d.h declares, and
rejects invalid arguments on the host before any launch (CPU only: no compute
call is made)."""
import ctypes
import os
import re

import pytest

from vision_sliding_window_amd import na2d

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "na2d.h")

# fake but 16-byte aligned, non-overlapping device addresses: only compared
Q, K, V, RPB, OUT = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000
GOOD = dict(B=2, heads=2, H=14, W=15, d=32, ksize=7)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:na|na1d|na2d|na3d|sasa2d)_[a-z_0-9]+)\s*\(", text)))


def declared_arity():
    """Parameter count of every prototype in the header."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b((?:na|na1d|na2d|na3d|sasa2d)_[a-z_0-9]+)\s*\(([^)]*)\)",
                                    text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_argument_counts_match_header():
    lib = na2d.load()
    for name, n in declared_arity().items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_exports_every_declared_function():
    lib = na2d.load()
    names = declared_functions()
    assert set(names) == set(na2d.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def check(q=Q, k=K, v=V, rpb=RPB, out=OUT, dtype=na2d.NA2D_F16, algo=0, **kw):
    a = dict(GOOD)
    a.update(kw)
    return na2d.na2d_check_args(q, k, v, rpb, out, a["B"], a["heads"], a["H"], a["W"], a["d"],
                                a["ksize"], dtype, algo)


def test_valid_arguments():
    assert check() == na2d.NA2D_OK
    assert check(rpb=None) == na2d.NA2D_OK                  # no positional bias
    assert check(dtype=na2d.NA2D_F32) == na2d.NA2D_OK
    assert check(ksize=1, algo=na2d.NA2D_ALGO_VALU) == na2d.NA2D_OK
    assert check(H=7, W=7, ksize=7) == na2d.NA2D_OK          # k = H = W
    assert check(q=Q, k=Q, v=Q) == na2d.NA2D_OK              # inputs may alias each other


@pytest.mark.parametrize("field", ["q", "k", "v", "out"])
def test_null_pointers(field):
    assert check(**{field: None}) == na2d.NA2D_ERR_NULL


@pytest.mark.parametrize("field", ["B", "heads", "H", "W", "d"])
@pytest.mark.parametrize("val", [0, -3])
def test_bad_sizes(field, val):
    assert check(**{field: val}) == na2d.NA2D_ERR_SHAPE


@pytest.mark.parametrize("ks", [0, -1, 2, 6, 17])
def test_bad_ksize(ks):
    assert check(ksize=ks) == na2d.NA2D_ERR_KSIZE  # even, < 1, or > H / W (14, 15)


def test_ksize_larger_than_one_axis():
    assert check(H=6, W=40, ksize=7) == na2d.NA2D_ERR_KSIZE
    assert check(H=40, W=6, ksize=7) == na2d.NA2D_ERR_KSIZE


def test_dtype_and_algo():
    assert check(dtype=3) == na2d.NA2D_ERR_DTYPE
    assert check(dtype=-1) == na2d.NA2D_ERR_DTYPE
    assert check(algo=7) == na2d.NA2D_ERR_ALGO


def test_unsupported():
    assert check(d=48) == na2d.NA2D_ERR_UNSUPPORTED                  # no kernel for d = 48
    assert check(d=64, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_ERR_UNSUPPORTED
    assert check(dtype=na2d.NA2D_F32, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_ERR_UNSUPPORTED
    assert check(ksize=1, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK  # the general kernel
    big = dict(H=64, W=64, ksize=27)
    assert check(algo=na2d.NA2D_ALGO_MFMA, **big) == na2d.NA2D_ERR_UNSUPPORTED
    assert check(**big) == na2d.NA2D_OK                              # AUTO falls back to VALU
    assert check(H=70, W=70, ksize=65) == na2d.NA2D_ERR_UNSUPPORTED  # beyond every kernel


@pytest.mark.parametrize("field", ["q", "k", "v", "rpb", "out"])
def test_alignment(field):
    base = {"q": Q, "k": K, "v": V, "rpb": RPB, "out": OUT}[field]
    assert check(**{field: base + 8}) == na2d.NA2D_ERR_ALIGN


def test_alias():
    n = GOOD["B"] * GOOD["heads"] * GOOD["H"] * GOOD["W"] * GOOD["d"]
    assert check(out=Q) == na2d.NA2D_ERR_ALIAS
    assert check(out=Q + 16 * ((n * 2) // 16 - 1)) == na2d.NA2D_ERR_ALIAS  # tail overlap
    assert check(out=Q + n * 2) == na2d.NA2D_OK                           # just after q
    assert check(out=K - 16) == na2d.NA2D_ERR_ALIAS                        # spills into k
    assert check(out=RPB - 16) == na2d.NA2D_ERR_ALIAS


def test_forward_rejects_before_launch():
    """Invalid calls return their status without touching the GPU."""
    st = na2d.na2d_forward(Q, K, V, RPB, OUT, 2, 2, 14, 15, 32, 8, na2d.NA2D_F16, None)
    assert st == na2d.NA2D_ERR_KSIZE
    lse = 0xC0000000
    st = na2d.na2d_forward_lse(Q, K, V, RPB, OUT, None, 2, 2, 14, 15, 32, 7, na2d.NA2D_F16, None)
    assert st == na2d.NA2D_ERR_NULL
    st = na2d.na2d_forward_lse(Q, K, V, RPB, OUT, lse + 4, 2, 2, 14, 15, 32, 7, na2d.NA2D_F16, None)
    assert st == na2d.NA2D_ERR_ALIGN
    st = na2d.na2d_forward_lse(Q, K, V, RPB, OUT, OUT + 64, 2, 2, 14, 15, 32, 7, na2d.NA2D_F16,
                               None)
    assert st == na2d.NA2D_ERR_ALIAS
    st = na2d.na2d_forward_lse(Q, K, V, RPB, OUT, lse, 2, 2, 14, 15, 32, 8, na2d.NA2D_F16, None)
    assert st == na2d.NA2D_ERR_KSIZE
    st = na2d.na2d_forward_ex(Q, K, V, RPB, Q, 2, 2, 14, 15, 32, 7, na2d.NA2D_F16, 0, None)
    assert st == na2d.NA2D_ERR_ALIAS


def test_select_algo():
    assert na2d.na2d_select_algo(56, 56, 32, 7, na2d.NA2D_F16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na2d_select_algo(128, 128, 32, 21, na2d.NA2D_BF16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na2d_select_algo(14, 14, 32, 7, na2d.NA2D_F32) == na2d.NA2D_ALGO_VALU
    # a window of 1 is served by the general matrix-core kernel
    assert na2d.na2d_select_algo(14, 14, 32, 1, na2d.NA2D_F16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na2d_select_algo(14, 14, 64, 7, na2d.NA2D_F16) == na2d.NA2D_ALGO_VALU
    NA, SASA = na2d.NA_WINDOW_NA, na2d.NA_WINDOW_SASA
    f16 = na2d.NA2D_F16
    assert na2d.na_select_algo_nd(16, 56, 56, 32, (5, 5, 5), NA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(16, 56, 56, 32, (11, 5, 5), NA, f16) == na2d.NA2D_ALGO_VALU
    assert na2d.na_select_algo_nd(1, 20, 30, 32, (1, 3, 7), NA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(1, 20, 30, 32, (1, 3, 7), SASA, f16) == na2d.NA2D_ALGO_VALU
    assert na2d.na_select_algo_nd(1, 20, 30, 32, (1, 7, 7), SASA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(1, 1, 3136, 32, (1, 1, 49), NA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(4, 9, 9, 32, (3, 3, 3), NA, na2d.NA2D_F32) == na2d.NA2D_ALGO_VALU
    assert na2d.na_select_algo_nd(4, 9, 9, 32, (3, 3, 3), 7, f16) == na2d.NA2D_ERR_UNSUPPORTED
    assert na2d.na_select_algo_nd(4, 9, 9, 32, (11, 3, 3), NA, f16) == na2d.NA2D_ERR_KSIZE
    # wide 2D windows: NA on the streaming kernel, SASA on the halo kernel, both MFMA
    assert na2d.na_select_algo_nd(1, 64, 64, 32, (1, 21, 21), NA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(1, 64, 64, 32, (1, 21, 21), SASA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(1, 64, 64, 32, (1, 25, 9), NA, f16) == na2d.NA2D_ALGO_MFMA
    assert na2d.na_select_algo_nd(1, 64, 64, 32, (1, 27, 27), NA, f16) == na2d.NA2D_ALGO_VALU
    assert na2d.na_select_algo_nd(12, 64, 64, 32, (3, 11, 3), NA, f16) == na2d.NA2D_ALGO_VALU
    assert na2d.na2d_select_algo(14, 14, 32, 8, na2d.NA2D_F16) == na2d.NA2D_ERR_KSIZE


def test_strerror_and_version():
    for code in range(-9, 1):
        assert na2d.na2d_strerror(code) != "unknown status"
    assert na2d.na2d_strerror(-100) == "unknown status"
    assert na2d.na2d_last_error() == ""
    assert na2d.na2d_version() >= 10000


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(na2d, "_lib", None)
    monkeypatch.setattr(na2d, "LIBRARY", str(tmp_path / "libna2d.so"))
    with pytest.raises(ImportError):
        na2d.load()


def check_nd(B=2, heads=2, D=5, H=6, W=7, d=32, kd=3, kh=3, kw=5, mode=0, dtype=na2d.NA2D_F16,
             algo=0, q=Q, k=K, v=V, rpb=RPB, out=OUT):
    return na2d.na_check_args_nd(q, k, v, rpb, out, B, heads, D, H, W, d, kd, kh, kw, mode, dtype,
                                 algo)


def test_nd_valid():
    assert check_nd() == na2d.NA2D_OK                                     # 3D, rectangular
    assert check_nd(D=1, H=1, W=40, kd=1, kh=1, kw=9) == na2d.NA2D_OK     # 1D
    assert check_nd(D=1, kd=1, kh=7, kw=9, mode=1) == na2d.NA2D_OK        # SASA wider than the map
    assert check_nd(dtype=na2d.NA2D_F32, d=128) == na2d.NA2D_OK


def test_nd_errors():
    assert check_nd(mode=2) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_nd(kd=7) == na2d.NA2D_ERR_KSIZE          # NA window longer than its axis
    assert check_nd(kw=4) == na2d.NA2D_ERR_KSIZE          # even
    assert check_nd(kh=4, mode=1) == na2d.NA2D_ERR_KSIZE  # even SASA window
    assert check_nd(kh=0, mode=1) == na2d.NA2D_ERR_KSIZE
    assert check_nd(D=0) == na2d.NA2D_ERR_SHAPE
    assert check_nd(kw=65, mode=1) == na2d.NA2D_ERR_UNSUPPORTED
    # the general matrix-core kernel: NA windows up to 9 on every axis
    assert check_nd(algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK                   # 3D
    assert check_nd(D=1, kd=1, kh=5, kw=3, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK
    assert check_nd(D=12, kd=11, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_nd(D=1, kd=1, kh=5, kw=3, mode=1,
                    algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_ERR_UNSUPPORTED   # rectangular SASA
    assert check_nd(d=64, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_ERR_UNSUPPORTED
    one_d = dict(D=1, H=1, W=300, kd=1, kh=1)
    assert check_nd(kw=63, algo=na2d.NA2D_ALGO_MFMA, **one_d) == na2d.NA2D_OK       # NA1D kernel
    assert check_nd(kw=65, algo=na2d.NA2D_ALGO_MFMA, **one_d) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_nd(kw=9, mode=1, algo=na2d.NA2D_ALGO_MFMA, **one_d) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_nd(kw=9, d=64, algo=na2d.NA2D_ALGO_MFMA, **one_d) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_nd(D=1, kd=1, kh=5, kw=5, mode=1, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK
    assert check_nd(D=1, kd=1, kh=9, kw=9, H=6, W=7, mode=1,
                    algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK      # SASA window wider than the map
    assert check_nd(D=1, kd=1, kh=5, kw=5, algo=na2d.NA2D_ALGO_MFMA) == na2d.NA2D_OK
    n = 2 * 2 * 5 * 6 * 7 * 32
    assert check_nd(out=Q + 16 * ((n * 2) // 16 - 1)) == na2d.NA2D_ERR_ALIAS
    assert check_nd(rpb=RPB + 4) == na2d.NA2D_ERR_ALIGN


def test_nd_wrappers_reject_before_launch():
    f16 = na2d.NA2D_F16
    assert na2d.na1d_forward(Q, K, V, RPB, OUT, 2, 2, 30, 32, 31, f16, None) == na2d.NA2D_ERR_KSIZE
    assert na2d.na3d_forward(Q, K, V, RPB, OUT, 2, 2, 4, 9, 9, 32, 5, f16, None) == na2d.NA2D_ERR_KSIZE
    assert na2d.sasa2d_forward(Q, K, V, RPB, OUT, 2, 2, 9, 9, 32, 6, f16, None) == na2d.NA2D_ERR_KSIZE
    assert na2d.sasa2d_forward(Q, K, V, RPB, Q, 2, 2, 9, 9, 32, 5, f16, None) == na2d.NA2D_ERR_ALIAS


DQ, DK, DV, DRPB, WS, DOUT = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000, 0xB0000000
LSE = 0xC0000000


def check_bwd(B=2, heads=2, H=14, W=15, d=32, ksize=7, dtype=na2d.NA2D_F16, **ptr):
    p = dict(q=Q, k=K, v=V, rpb=RPB, out=OUT, lse=None, dout=DOUT, dq=DQ, dk=DK, dv=DV,
             drpb=DRPB, ws=WS)
    p.update(ptr)
    return na2d.na2d_backward_check_args(p["q"], p["k"], p["v"], p["rpb"], p["out"], p["lse"],
                                         p["dout"], p["dq"], p["dk"], p["dv"], p["drpb"], p["ws"],
                                         B, heads, H, W, d, ksize, dtype)


def test_backward_args():
    assert check_bwd() == na2d.NA2D_OK
    assert check_bwd(rpb=None, drpb=None) == na2d.NA2D_OK
    assert check_bwd(drpb=None) == na2d.NA2D_ERR_NULL        # bias without its gradient
    assert check_bwd(rpb=None) == na2d.NA2D_ERR_NULL         # gradient without a bias
    assert check_bwd(ws=None) == na2d.NA2D_ERR_NULL
    assert check_bwd(dout=None) == na2d.NA2D_ERR_NULL
    assert check_bwd(ksize=8) == na2d.NA2D_ERR_KSIZE
    assert check_bwd(d=48) == na2d.NA2D_ERR_UNSUPPORTED
    assert check_bwd(dq=DQ + 4) == na2d.NA2D_ERR_ALIGN
    assert check_bwd(dq=Q) == na2d.NA2D_ERR_ALIAS             # output on an input
    assert check_bwd(dk=DQ + 64) == na2d.NA2D_ERR_ALIAS       # two outputs overlap
    assert check_bwd(ws=DOUT + 16) == na2d.NA2D_ERR_ALIAS
    assert check_bwd(ws=DOUT - 4096) == na2d.NA2D_ERR_ALIAS   # the bias-gradient tables reach dout
    # the forward's log-sum-exp: optional, aligned, written by nothing here
    assert check_bwd(lse=LSE) == na2d.NA2D_OK
    assert check_bwd(lse=LSE + 4) == na2d.NA2D_ERR_ALIGN
    assert check_bwd(lse=LSE, dq=LSE - 16) == na2d.NA2D_ERR_ALIAS
    assert check_bwd(lse=LSE, ws=LSE + 2 * 2 * 14 * 15 * 4 - 16) == na2d.NA2D_ERR_ALIAS
    # statistics (8 bytes a query, padded to 256) then a (2k-1)^2 table per 8 x 8 tile
    stats = (2 * 2 * 14 * 15 * 8 + 255) // 256 * 256
    assert na2d.na2d_backward_workspace_bytes(2, 2, 14, 15, 5) == stats + 2 * 2 * 2 * 2 * 81 * 4
    assert na2d.na2d_backward_workspace_bytes(0, 2, 14, 15, 5) == 0
    assert na2d.na2d_backward_workspace_bytes(2, 2, 14, 15, 0) == 0
    st = na2d.na2d_backward(Q, K, V, RPB, OUT, None, DOUT, DQ, DK, DV, DRPB, WS, 2, 2, 14, 15, 32,
                            17, na2d.NA2D_F16, None)
    assert st == na2d.NA2D_ERR_KSIZE                          # rejected before any launch


def test_holder_ranges_closed_form():
    """The backward's key pass visits, per axis, the positions whose clamped
    window holds key j: lo = 0 if j < k else j - k//2, hi = L - 1 if
    j >= L - k else j + k//2 (the closed form in na2d_bwd.hip), which must be
    exactly the brute-force set."""
    def start(i, k, L):
        return min(max(i - k // 2, 0), L - k)
    for k in (1, 3, 5, 7, 9, 13, 25, 63):
        for L in range(k, 3 * k + 5):
            for j in range(L):
                members = [i for i in range(L) if start(i, k, L) <= j < start(i, k, L) + k]
                lo = 0 if j < k else j - k // 2
                hi = L - 1 if j >= L - k else j + k // 2
                assert members == list(range(lo, hi + 1)), (k, L, j)


def test_backward_select_algo():
    """The matrix-core backward takes 16-bit inputs, d = 32, k <= 25 and maps
    whose fp32 rows fit 32-bit byte offsets (H * W * 128 < 2^31); past that
    bound, and for anything else, the VALU kernels (64-bit offsets) run."""
    MFMA, VALU = na2d.NA2D_ALGO_MFMA, na2d.NA2D_ALGO_VALU
    sel = na2d.na2d_backward_select_algo
    assert sel(56, 56, 32, 7, na2d.NA2D_F16) == MFMA
    assert sel(56, 56, 32, 7, na2d.NA2D_BF16) == MFMA
    assert sel(56, 56, 32, 7, na2d.NA2D_F32) == VALU
    assert sel(56, 56, 64, 7, na2d.NA2D_F16) == VALU
    assert sel(128, 128, 32, 25, na2d.NA2D_F16) == MFMA
    assert sel(128, 128, 32, 27, na2d.NA2D_F16) == VALU
    # the largest map the matrix-core passes address, and the first past it
    assert 4096 * 4095 * 128 < 2 ** 31 <= 4096 * 4096 * 128
    assert sel(4096, 4095, 32, 7, na2d.NA2D_F16) == MFMA
    assert sel(4096, 4096, 32, 7, na2d.NA2D_F16) == VALU
    assert sel(16384, 1024, 32, 7, na2d.NA2D_BF16) == VALU
    assert sel(56, 56, 32, 8, na2d.NA2D_F16) == na2d.NA2D_ERR_KSIZE
    assert sel(56, 56, 48, 7, na2d.NA2D_F16) == na2d.NA2D_ERR_UNSUPPORTED
    assert sel(56, 56, 32, 7, 9) == na2d.NA2D_ERR_DTYPE


def test_occupancy_queries_start_at_zero():
    """No kernel has been launched on this CPU-only process, so the library
    has made no occupancy query."""
    assert na2d.na2d_occupancy_queries() == 0


def test_stream_reference_rejects_before_launch():
    ref = na2d.na_stream_reference
    assert ref(None, K, V, OUT, 64) == na2d.NA2D_ERR_NULL
    assert ref(Q, K, V, None, 64) == na2d.NA2D_ERR_NULL
    assert ref(Q, K, V, OUT, 0) == na2d.NA2D_ERR_SHAPE
    assert ref(Q, K, V, OUT, 60) == na2d.NA2D_ERR_SHAPE    # not a multiple of 8
    assert ref(Q + 8, K, V, OUT, 64) == na2d.NA2D_ERR_ALIGN
    assert ref(Q, K, V, OUT + 4, 64) == na2d.NA2D_ERR_ALIGN


def test_backward_noalloc_rejects_before_launch():
    """The allocation-free backward checks its arguments like na2d_backward
    (without a workspace) and refuses, before any HIP call, a problem whose
    workspace would not fit the fixed device array."""
    DQ, DK, DV, DRPB, DOUT = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xa0000000
    f = na2d.na2d_backward_noalloc
    args = (Q, K, V, RPB, OUT, None, DOUT, DQ, DK, DV, DRPB)
    assert f(*args, 2, 2, 14, 15, 32, 8, na2d.NA2D_F16, None) == na2d.NA2D_ERR_KSIZE
    assert f(Q, K, V, RPB, OUT, None, None, DQ, DK, DV, DRPB, 2, 2, 14, 15, 32, 7,
             na2d.NA2D_F16, None) == na2d.NA2D_ERR_NULL
    assert f(Q, K, V, RPB, OUT, None, DOUT, DQ, DK, DV, None, 2, 2, 14, 15, 32, 7,
             na2d.NA2D_F16, None) == na2d.NA2D_ERR_NULL
    assert f(Q, K, V, RPB, OUT, None, DOUT, Q, DK, DV, DRPB, 2, 2, 14, 15, 32, 7,
             na2d.NA2D_F16, None) == na2d.NA2D_ERR_ALIAS
    # 64 maps of 128 x 128 at k = 21: 8 + 41^2 * 4 / 64 bytes per query, past 64 MiB
    big = na2d.na2d_backward_workspace_bytes(16, 4, 128, 128, 21)
    assert big > na2d.NA2D_NOALLOC_SCRATCH_BYTES
    assert f(*args, 16, 4, 128, 128, 32, 21, na2d.NA2D_BF16, None) == na2d.NA2D_ERR_SCRATCH
    assert "scratch" in na2d.na2d_strerror(na2d.NA2D_ERR_SCRATCH)
    # the large-kernel workload fits: 8 maps of four heads at k = 21
    assert na2d.na2d_backward_workspace_bytes(8, 4, 128, 128, 21) <= na2d.NA2D_NOALLOC_SCRATCH_BYTES
