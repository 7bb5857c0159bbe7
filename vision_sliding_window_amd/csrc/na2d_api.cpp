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

constexpr int kVersion = 10000;  // 1.0.0

int elem_size(int dtype) { return dtype == NA2D_F32 ? 4 : 2; }

bool overlaps(const void *a, uint64_t abytes, const void *b, uint64_t bbytes)
{
    if (!a || !b || abytes == 0 || bbytes == 0) return false;
    const uint64_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bbytes && pb < pa + abytes;
}

bool valu_supports(int d, int ksize) {
    return (d == 16 || d == 32 || d == 64 || d == 128) && ksize <= NA2D_VALU_MAX_KSIZE;
}

// The MFMA kernel addresses one (b, h) map with 32-bit byte offsets.
bool mfma_supports(int H, int W, int d, int ksize, int dtype) {
    return (dtype == NA2D_F16 || dtype == NA2D_BF16) && d == 32 && ksize >= 3 &&
           ksize <= NA2D_MFMA_MAX_KSIZE && (uint64_t)H * W * d * 4 <= 0x7fffffffull;
}

// Size checks shared by every entry point.
int check_sizes(int B, int heads, int H, int W, int d, int ksize)
{
    if (B <= 0 || heads <= 0 || H <= 0 || W <= 0 || d <= 0) return NA2D_ERR_SHAPE;
    const uint64_t pixels = (uint64_t)B * heads * H * W;
    // element counts are 64-bit inside the kernels; keep the query count within
    // what a one-dimensional grid of 256-lane workgroups can cover
    if (pixels > (uint64_t)0x7fffffff * 64ull || pixels * (uint64_t)d > (1ull << 60))
        return NA2D_ERR_SHAPE;
    if (ksize < 1 || (ksize % 2) == 0 || ksize > H || ksize > W) return NA2D_ERR_KSIZE;
    return NA2D_OK;
}

int resolve_algo(int H, int W, int d, int ksize, int dtype, int algo)
{
    if (algo == NA2D_ALGO_AUTO)
        return mfma_supports(H, W, d, ksize, dtype) ? NA2D_ALGO_MFMA : NA2D_ALGO_VALU;
    return algo;
}

}  // namespace

extern "C" int na2d_check_args(const void *q, const void *k, const void *v, const float *rpb,
                               const float *out, int B, int heads, int H, int W, int d,
                               int ksize, int dtype, int algo)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    if (algo != NA2D_ALGO_AUTO && algo != NA2D_ALGO_VALU && algo != NA2D_ALGO_MFMA)
        return NA2D_ERR_ALGO;
    if (!q || !k || !v || !out) return NA2D_ERR_NULL;
    int st = check_sizes(B, heads, H, W, d, ksize);
    if (st != NA2D_OK) return st;
    const void *ptrs[5] = {q, k, v, out, rpb};
    for (const void *p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return NA2D_ERR_ALIGN;
    const uint64_t n = (uint64_t)B * heads * H * W * d;
    const uint64_t in_bytes = n * elem_size(dtype), out_bytes = n * 4;
    const uint64_t rpb_bytes = (uint64_t)heads * (2 * ksize - 1) * (2 * ksize - 1) * 4;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, rpb, rpb_bytes))
        return NA2D_ERR_ALIAS;
    const int a = resolve_algo(H, W, d, ksize, dtype, algo);
    if (a == NA2D_ALGO_VALU && !valu_supports(d, ksize)) return NA2D_ERR_UNSUPPORTED;
    if (a == NA2D_ALGO_MFMA && !mfma_supports(H, W, d, ksize, dtype)) return NA2D_ERR_UNSUPPORTED;
    return NA2D_OK;
}

extern "C" int na2d_select_algo(int H, int W, int d, int ksize, int dtype)
{
    if (dtype != NA2D_F32 && dtype != NA2D_F16 && dtype != NA2D_BF16) return NA2D_ERR_DTYPE;
    int st = check_sizes(1, 1, H, W, d, ksize);
    if (st != NA2D_OK) return st;
    const int a = resolve_algo(H, W, d, ksize, dtype, NA2D_ALGO_AUTO);
    if (a == NA2D_ALGO_VALU && !valu_supports(d, ksize)) return NA2D_ERR_UNSUPPORTED;
    return a;
}

extern "C" int na2d_forward_ex(const void *q, const void *k, const void *v, const float *rpb,
                               float *out, int B, int heads, int H, int W, int d, int ksize,
                               int dtype, int algo, void *stream)
{
    int st = na2d_check_args(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, algo);
    if (st != NA2D_OK) return st;
    const na2d::Problem p{q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = resolve_algo(H, W, d, ksize, dtype, algo) == NA2D_ALGO_MFMA
                             ? na2d::launch_mfma(p, s)
                             : na2d::launch_valu(p, s);
    if (e != hipSuccess) {
        g_last_error = hipGetErrorString(e);
        return NA2D_ERR_HIP;
    }
    return NA2D_OK;
}

extern "C" int na2d_forward(const void *q, const void *k, const void *v, const float *rpb,
                            float *out, int B, int heads, int H, int W, int d, int ksize,
                            int dtype, void *stream)
{
    return na2d_forward_ex(q, k, v, rpb, out, B, heads, H, W, d, ksize, dtype, NA2D_ALGO_AUTO,
                           stream);
}

extern "C" const char *na2d_strerror(int status)
{
    switch (status) {
    case NA2D_OK: return "success";
    case NA2D_ERR_NULL: return "q, k, v or out is NULL";
    case NA2D_ERR_SHAPE: return "B, heads, H, W or d is not positive, or the problem is too large";
    case NA2D_ERR_KSIZE: return "ksize must be odd, >= 1 and <= min(H, W)";
    case NA2D_ERR_DTYPE: return "dtype must be NA2D_F32, NA2D_F16 or NA2D_BF16";
    case NA2D_ERR_UNSUPPORTED: return "head dim or ksize not supported by the selected kernel";
    case NA2D_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case NA2D_ERR_ALIAS: return "out overlaps q, k, v or rpb";
    case NA2D_ERR_HIP: return "HIP runtime error (see na2d_last_error)";
    case NA2D_ERR_ALGO: return "algo must be NA2D_ALGO_AUTO, NA2D_ALGO_VALU or NA2D_ALGO_MFMA";
    default: return "unknown status";
    }
}

extern "C" const char *na2d_last_error(void) { return g_last_error.c_str(); }

extern "C" int na2d_version(void) { return kVersion; }
