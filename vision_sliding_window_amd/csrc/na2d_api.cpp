// na2d_api.cpp -- host side of the C ABI declared in include/na2d.h:
// argument checks, kernel-family selection and launch.  No HIP call is made
// before every argument has been checked.
#include "na2d.h"
#include "na2d_launch.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

namespace {

thread_local std::string g_last_error;

constexpr int kVersion = 10100;  // 1.1.0

int elem_size(int dtype) { return dtype == NA2D_F32 ? 4 : 2; }

bool overlaps(const void *a, uint64_t abytes, const void *b, uint64_t bbytes)
{
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    const uint64_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bbytes && pb < pa + abytes;
}

// A grid of queries [B, heads, D, H, W] with a kd x kh x kw window.
struct Nd {
    int B, heads, D, H, W, d, kd, kh, kw, mode;
};

bool valu_supports(const Nd &n)
{
    return (n.d == 16 || n.d == 32 || n.d == 64 || n.d == 128) && n.kd <= NA2D_VALU_MAX_KSIZE &&
           n.kh <= NA2D_VALU_MAX_KSIZE && n.kw <= NA2D_VALU_MAX_KSIZE;
}

// The NA1D matrix-core kernel: a sequence (D = H = 1) with a 1 x 1 x kw NA window.
bool is_mfma_1d(const Nd &n)
{
    return n.D == 1 && n.H == 1 && n.kd == 1 && n.kh == 1 && n.mode == NA_WINDOW_NA &&
           n.kw >= 3 && n.kw <= NA1D_MFMA_MAX_KSIZE;
}

// The 2D matrix-core kernel (a K/V halo per tile in LDS): square windows, NA
// up to halo_max_na_k and SASA up to NA2D_MFMA_MAX_KSIZE.  Wider NA windows
// go to the wide-window kernel (na2d_large_mfma.hip), which streams the key
// blocks of a tile through LDS one block row at a time. For bf16 inputs that
// kernel, which multiplies fp16 weights by V converted to fp16 where the halo
// kernel splits the weights into two bf16 parts, measured faster from k = 11
// (k = 13: 79.5 against 82.1 us at 8 x 4 x 128^2); for fp16 inputs from k = 15.
int halo_max_na_k(int dtype) { return dtype == NA2D_BF16 ? 9 : 13; }

bool is_mfma_2d(const Nd &n, int dtype)
{
    return n.D == 1 && n.kd == 1 && n.kh == n.kw && n.kh >= 3 && n.kh <= NA2D_MFMA_MAX_KSIZE &&
           (n.mode == NA_WINDOW_SASA || n.kh <= halo_max_na_k(dtype));
}

// The wide-window kernel: square 2D NA windows past the halo kernel's range.
bool is_mfma_2d_large(const Nd &n, int dtype)
{
    return n.D == 1 && n.kd == 1 && n.kh == n.kw && n.mode == NA_WINDOW_NA && n.kh > halo_max_na_k(dtype) &&
           n.kh <= NA2D_MFMA_MAX_KSIZE;
}

// Both take 16-bit inputs with d = 32 and address one (b, h) map with 32-bit
// byte offsets.
// The streaming kernel: any other NA window with every axis small enough --
// 3D windows up to NA3D_MFMA_MAX_KSIZE per axis, 2D windows (kd = 1, square
// or rectangular) up to NA2D_MFMA_MAX_KSIZE.
bool is_mfma_3d(const Nd &n, int dtype)
{
    if (is_mfma_1d(n) || is_mfma_2d(n, dtype) || is_mfma_2d_large(n, dtype) || n.mode != NA_WINDOW_NA)
        return false;
    const int lim = n.kd == 1 ? NA2D_MFMA_MAX_KSIZE : NA3D_MFMA_MAX_KSIZE;
    return n.kd <= NA3D_MFMA_MAX_KSIZE && n.kh <= lim && n.kw <= lim;
}

bool mfma_supports(const Nd &n, int dtype)
{
    return (dtype == NA2D_F16 || dtype == NA2D_BF16) && n.d == 32 &&
           (is_mfma_1d(n) || is_mfma_2d(n, dtype) || is_mfma_2d_large(n, dtype) || is_mfma_3d(n, dtype)) &&
           (uint64_t)n.D * n.H * n.W * n.d * 4 <= 0x7fffffffull;
}

bool window_ok(int k, int L, int mode)
{
    return k >= 1 && (k % 2) == 1 && (mode == NA_WINDOW_SASA || k <= L);
}

// Size checks shared by every entry point.
int check_sizes(const Nd &n)
{
    if (n.B <= 0 || n.heads <= 0 || n.D <= 0 || n.H <= 0 || n.W <= 0 || n.d <= 0)
        return NA2D_ERR_SHAPE;
    const uint64_t queries = (uint64_t)n.B * n.heads * n.D * n.H * n.W;
    // element counts are 64-bit inside the kernels; keep the query count within
    // what a one-dimensional grid of 256-lane workgroups can cover
    if (queries > (uint64_t)0x7fffffff * 64ull || queries * (uint64_t)n.d > (1ull << 60))
        return NA2D_ERR_SHAPE;
    if (!window_ok(n.kd, n.D, n.mode) || !window_ok(n.kh, n.H, n.mode) ||
        !window_ok(n.kw, n.W, n.mode))
        return NA2D_ERR_KSIZE;
    return NA2D_OK;
}

int resolve_algo(const Nd &n, int dtype, int algo)
{
    if (algo == NA2D_ALGO_AUTO)
        return mfma_supports(n, dtype) ? NA2D_ALGO_MFMA : NA2D_ALGO_VALU;
    return algo;
}

int check_nd(const void *q, const void *k, const void *v, const float *rpb, const float *out,
             const Nd &n, int dtype, int algo, const float *lse = nullptr)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    if (algo != NA2D_ALGO_AUTO && algo != NA2D_ALGO_VALU && algo != NA2D_ALGO_MFMA)
        return NA2D_ERR_ALGO;
    if (n.mode != NA_WINDOW_NA && n.mode != NA_WINDOW_SASA) return NA2D_ERR_UNSUPPORTED;
    if (!q || !k || !v || !out) return NA2D_ERR_NULL;
    const int st = check_sizes(n);
    if (st != NA2D_OK) return st;
    const void *ptrs[6] = {q, k, v, out, rpb, lse};
    for (const void *p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return NA2D_ERR_ALIGN;
    const uint64_t queries = (uint64_t)n.B * n.heads * n.D * n.H * n.W;
    const uint64_t elems = queries * n.d;
    const uint64_t in_bytes = elems * elem_size(dtype), out_bytes = elems * 4;
    const uint64_t rpb_bytes =
        (uint64_t)n.heads * (2 * n.kd - 1) * (2 * n.kh - 1) * (2 * n.kw - 1) * 4;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, rpb, rpb_bytes))
        return NA2D_ERR_ALIAS;
    if (lse) {  // the log-sum-exp output: overlaps nothing
        const uint64_t lse_bytes = queries * 4;
        if (overlaps(lse, lse_bytes, q, in_bytes) || overlaps(lse, lse_bytes, k, in_bytes) ||
            overlaps(lse, lse_bytes, v, in_bytes) || overlaps(lse, lse_bytes, rpb, rpb_bytes) ||
            overlaps(lse, lse_bytes, out, out_bytes))
            return NA2D_ERR_ALIAS;
    }
    const int a = resolve_algo(n, dtype, algo);
    if (a == NA2D_ALGO_VALU && !valu_supports(n)) return NA2D_ERR_UNSUPPORTED;
    if (a == NA2D_ALGO_MFMA && !mfma_supports(n, dtype)) return NA2D_ERR_UNSUPPORTED;
    return NA2D_OK;
}

int forward_nd(const void *q, const void *k, const void *v, const float *rpb, float *out,
               const Nd &n, int dtype, int algo, void *stream, float *lse = nullptr)
{
    const int st = check_nd(q, k, v, rpb, out, n, dtype, algo, lse);
    if (st != NA2D_OK) return st;
    const na2d::Problem p{q,     k,      v,   rpb,  out,  n.B,  n.heads, n.H,
                          n.W,   n.d,    n.kh, dtype, n.D, n.kd, n.kh,    n.kw,
                          n.mode, lse};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (resolve_algo(n, dtype, algo) == NA2D_ALGO_MFMA)
        e = is_mfma_1d(n)         ? na2d::launch_mfma_1d(p, s)
            : is_mfma_2d(n, dtype)       ? na2d::launch_mfma(p, s)
            : is_mfma_2d_large(n, dtype) ? na2d::launch_mfma_large(p, s)
                                  : na2d::launch_mfma_3d(p, s);
    else
        e = na2d::launch_valu(p, s);
    if (e != hipSuccess) {
        g_last_error = hipGetErrorString(e);
        return NA2D_ERR_HIP;
    }
    return NA2D_OK;
}

Nd nd_2d(int B, int heads, int H, int W, int d, int ksize, int mode)
{
    return Nd{B, heads, 1, H, W, d, 1, ksize, ksize, mode};
}

}  // namespace

extern "C" int na2d_check_args(const void *q, const void *k, const void *v, const float *rpb,
                               const float *out, int B, int heads, int H, int W, int d,
                               int ksize, int dtype, int algo)
{
    return check_nd(q, k, v, rpb, out, nd_2d(B, heads, H, W, d, ksize, NA_WINDOW_NA), dtype,
                    algo);
}

extern "C" int na2d_select_algo(int H, int W, int d, int ksize, int dtype)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    const Nd n = nd_2d(1, 1, H, W, d, ksize, NA_WINDOW_NA);
    const int st = check_sizes(n);
    if (st != NA2D_OK) return st;
    const int a = resolve_algo(n, dtype, NA2D_ALGO_AUTO);
    if (a == NA2D_ALGO_VALU && !valu_supports(n)) return NA2D_ERR_UNSUPPORTED;
    return a;
}

extern "C" int na_select_algo_nd(int D, int H, int W, int d, int kd, int kh, int kw, int mode,
                                 int dtype)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    if (mode != NA_WINDOW_NA && mode != NA_WINDOW_SASA) return NA2D_ERR_UNSUPPORTED;
    const Nd n{1, 1, D, H, W, d, kd, kh, kw, mode};
    const int st = check_sizes(n);
    if (st != NA2D_OK) return st;
    const int a = resolve_algo(n, dtype, NA2D_ALGO_AUTO);
    if (a == NA2D_ALGO_VALU && !valu_supports(n)) return NA2D_ERR_UNSUPPORTED;
    return a;
}

extern "C" int na2d_forward_ex(const void *q, const void *k, const void *v, const float *rpb,
                               float *out, int B, int heads, int H, int W, int d, int ksize,
                               int dtype, int algo, void *stream)
{
    return forward_nd(q, k, v, rpb, out, nd_2d(B, heads, H, W, d, ksize, NA_WINDOW_NA), dtype,
                      algo, stream);
}

extern "C" int na2d_forward(const void *q, const void *k, const void *v, const float *rpb,
                            float *out, int B, int heads, int H, int W, int d, int ksize,
                            int dtype, void *stream)
{
    return na2d_forward_ex(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, NA2D_ALGO_AUTO,
                           stream);
}

extern "C" int na2d_forward_lse(const void *q, const void *k, const void *v, const float *rpb,
                                float *out, float *lse, int B, int heads, int H, int W, int d,
                                int ksize, int dtype, void *stream)
{
    if (!lse) return NA2D_ERR_NULL;
    return forward_nd(q, k, v, rpb, out, nd_2d(B, heads, H, W, d, ksize, NA_WINDOW_NA), dtype,
                      NA2D_ALGO_AUTO, stream, lse);
}

extern "C" int na_check_args_nd(const void *q, const void *k, const void *v, const float *rpb,
                                const float *out, int B, int heads, int D, int H, int W, int d,
                                int kd, int kh, int kw, int mode, int dtype, int algo)
{
    return check_nd(q, k, v, rpb, out, Nd{B, heads, D, H, W, d, kd, kh, kw, mode}, dtype, algo);
}

extern "C" int na_forward_nd(const void *q, const void *k, const void *v, const float *rpb,
                             float *out, int B, int heads, int D, int H, int W, int d, int kd,
                             int kh, int kw, int mode, int dtype, int algo, void *stream)
{
    return forward_nd(q, k, v, rpb, out, Nd{B, heads, D, H, W, d, kd, kh, kw, mode}, dtype, algo,
                      stream);
}

extern "C" int na1d_forward(const void *q, const void *k, const void *v, const float *rpb,
                            float *out, int B, int heads, int L, int d, int ksize, int dtype,
                            void *stream)
{
    return forward_nd(q, k, v, rpb, out, Nd{B, heads, 1, 1, L, d, 1, 1, ksize, NA_WINDOW_NA},
                      dtype, NA2D_ALGO_AUTO, stream);
}

extern "C" int na3d_forward(const void *q, const void *k, const void *v, const float *rpb,
                            float *out, int B, int heads, int D, int H, int W, int d, int ksize,
                            int dtype, void *stream)
{
    return forward_nd(q, k, v, rpb, out,
                      Nd{B, heads, D, H, W, d, ksize, ksize, ksize, NA_WINDOW_NA}, dtype,
                      NA2D_ALGO_AUTO, stream);
}

extern "C" int sasa2d_forward(const void *q, const void *k, const void *v, const float *rpb,
                              float *out, int B, int heads, int H, int W, int d, int ksize,
                              int dtype, void *stream)
{
    return forward_nd(q, k, v, rpb, out, nd_2d(B, heads, H, W, d, ksize, NA_WINDOW_SASA), dtype,
                      NA2D_ALGO_AUTO, stream);
}

namespace {

// The matrix-core backward: 16-bit inputs, d = 32, windows up to
// NA2D_BWD_MFMA_MAX_KSIZE, and one map's fp32 rows (dout: H * W * 128
// bytes) within the 32-bit byte offsets of its buffer addressing. Anything
// else runs on the VALU kernels, which use 64-bit element offsets.
bool bwd_mfma_supports(int H, int W, int d, int ksize, int dtype)
{
    return (dtype == NA2D_F16 || dtype == NA2D_BF16) && d == 32 &&
           ksize <= NA2D_BWD_MFMA_MAX_KSIZE && (uint64_t)H * W * d * 4 <= 0x7fffffffull;
}

int check_backward(const void *q, const void *k, const void *v, const float *rpb,
                   const float *out, const float *lse, const float *dout, const float *dq,
                   const float *dk, const float *dv, const float *drpb, const void *ws, int B,
                   int heads, int H, int W, int d, int ksize, int dtype, bool need_ws = true)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    if (!q || !k || !v || !out || !dout || !dq || !dk || !dv || (!ws && need_ws))
        return NA2D_ERR_NULL;
    if (!rpb != !drpb) return NA2D_ERR_NULL;  // a bias gradient exactly when there is a bias
    const Nd n = nd_2d(B, heads, H, W, d, ksize, NA_WINDOW_NA);
    const int st = check_sizes(n);
    if (st != NA2D_OK) return st;
    const void *ptrs[12] = {q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, ws};
    for (const void *p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return NA2D_ERR_ALIGN;
    const uint64_t queries = (uint64_t)B * heads * H * W, elems = queries * d;
    const uint64_t in_b = elems * elem_size(dtype), f_b = elems * 4;
    const uint64_t ws_b = na2d::bwd_workspace_bytes(B, heads, H, W, ksize);
    const uint64_t rpb_b = (uint64_t)heads * (2 * ksize - 1) * (2 * ksize - 1) * 4;
    struct Span { const void *p; uint64_t n; };
    const Span outs[5] = {{dq, f_b}, {dk, f_b}, {dv, f_b}, {drpb, rpb_b}, {ws, ws_b}};
    const Span ins[7] = {{q, in_b}, {k, in_b}, {v, in_b}, {rpb, rpb_b}, {out, f_b}, {dout, f_b},
                         {lse, queries * 4}};
    for (int i = 0; i < 5; ++i) {
        for (const Span &in : ins)
            if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return NA2D_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return NA2D_ERR_ALIAS;
    }
    if (!valu_supports(n)) return NA2D_ERR_UNSUPPORTED;
    return NA2D_OK;
}

}  // namespace

extern "C" int na2d_backward_check_args(const void *q, const void *k, const void *v,
                                        const float *rpb, const float *out, const float *lse,
                                        const float *dout, const float *dq, const float *dk,
                                        const float *dv, const float *drpb,
                                        const void *workspace, int B, int heads, int H, int W,
                                        int d, int ksize, int dtype)
{
    return check_backward(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, workspace, B, heads, H,
                          W, d, ksize, dtype);
}

extern "C" int na2d_backward_select_algo(int H, int W, int d, int ksize, int dtype)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    const Nd n = nd_2d(1, 1, H, W, d, ksize, NA_WINDOW_NA);
    const int st = check_sizes(n);
    if (st != NA2D_OK) return st;
    if (!valu_supports(n)) return NA2D_ERR_UNSUPPORTED;
    return bwd_mfma_supports(H, W, d, ksize, dtype) ? NA2D_ALGO_MFMA : NA2D_ALGO_VALU;
}

extern "C" long long na2d_backward_workspace_bytes(int B, int heads, int H, int W, int ksize)
{
    if (B <= 0 || heads <= 0 || H <= 0 || W <= 0 || ksize < 1 || ksize > NA2D_VALU_MAX_KSIZE)
        return 0;
    return (long long)na2d::bwd_workspace_bytes(B, heads, H, W, ksize);
}

extern "C" int na2d_backward(const void *q, const void *k, const void *v, const float *rpb,
                             const float *out, const float *lse, const float *dout, float *dq,
                             float *dk, float *dv, float *drpb, void *workspace, int B,
                             int heads, int H, int W, int d, int ksize, int dtype, void *stream)
{
    const int st = check_backward(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, workspace, B,
                                  heads, H, W, d, ksize, dtype);
    if (st != NA2D_OK) return st;
    const int algo =
        bwd_mfma_supports(H, W, d, ksize, dtype) ? NA2D_ALGO_MFMA : NA2D_ALGO_VALU;
    const na2d::BwdProblem p{q,  k,    v,         rpb, out, lse,   dout,  dq,   dk, dv,
                             drpb, workspace, B,   heads, H, W, d, ksize, dtype, algo};
    const hipError_t e = na2d::launch_backward(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_last_error = hipGetErrorString(e);
        return NA2D_ERR_HIP;
    }
    return NA2D_OK;
}

extern "C" int na2d_backward_noalloc(const void *q, const void *k, const void *v,
                                     const float *rpb, const float *out, const float *lse,
                                     const float *dout, float *dq, float *dk, float *dv,
                                     float *drpb, int B, int heads, int H, int W, int d,
                                     int ksize, int dtype, void *stream)
{
    const int st = check_backward(q, k, v, rpb, out, lse, dout, dq, dk, dv, drpb, nullptr, B,
                                  heads, H, W, d, ksize, dtype, false);
    if (st != NA2D_OK) return st;
    if (na2d::bwd_workspace_bytes(B, heads, H, W, ksize) > NA2D_NOALLOC_SCRATCH_BYTES)
        return NA2D_ERR_SCRATCH;
    void *ws = nullptr;
    hipError_t e = na2d::noalloc_scratch(&ws);
    if (e == hipSuccess) {
        const int algo =
            bwd_mfma_supports(H, W, d, ksize, dtype) ? NA2D_ALGO_MFMA : NA2D_ALGO_VALU;
        const na2d::BwdProblem p{q,  k,  v,  rpb,   out,   lse, dout, dq,    dk,    dv,
                                 drpb, ws, B,  heads, H, W, d,   ksize, dtype, algo};
        e = na2d::launch_backward(p, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) {
        g_last_error = hipGetErrorString(e);
        return NA2D_ERR_HIP;
    }
    return NA2D_OK;
}

extern "C" const char *na2d_strerror(int status)
{
    switch (status) {
    case NA2D_OK: return "success";
    case NA2D_ERR_NULL: return "q, k, v or out is NULL";
    case NA2D_ERR_SHAPE: return "a size is not positive, or the problem is too large";
    case NA2D_ERR_KSIZE: return "a window must be odd, >= 1 and (NA) no longer than its axis";
    case NA2D_ERR_DTYPE: return "dtype must be NA2D_F32, NA2D_F16 or NA2D_BF16";
    case NA2D_ERR_UNSUPPORTED:
        return "head dim, window or mode not supported by the selected kernel";
    case NA2D_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case NA2D_ERR_ALIAS: return "out overlaps q, k, v or rpb";
    case NA2D_ERR_HIP: return "HIP runtime error (see na2d_last_error)";
    case NA2D_ERR_ALGO: return "algo must be NA2D_ALGO_AUTO, NA2D_ALGO_VALU or NA2D_ALGO_MFMA";
    case NA2D_ERR_SCRATCH:
        return "the backward needs more workspace than the fixed device scratch array holds "
               "(NA2D_NOALLOC_SCRATCH_BYTES); call na2d_backward with a workspace";
    default: return "unknown status";
    }
}

extern "C" const char *na2d_last_error(void) { return g_last_error.c_str(); }

extern "C" int na2d_version(void) { return kVersion; }

extern "C" long long na2d_occupancy_queries(void) { return na2d::occupancy_queries(); }
