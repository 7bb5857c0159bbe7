// na_valu.hip -- Neighborhood Attention forward, one query per lane, fp32
// vector arithmetic, over one, two or three axes.
//
// This is the plain kernel of the library: it serves float32 inputs, head
// dims 16/32/64/128, windows up to 63 per axis, NA1D/NA2D/NA3D and SASA
// windows.  Each lane owns one query (b, h, z, y, x) of a [B, heads, D, H, W]
// grid (2D: D = 1, 1D: D = H = 1).  It walks the query's kd x kh x kw window
// -- clamped inside the grid for NA (CSDN translation of "Neighborhood
// Attention Transformer", section 3.1 and the qiita article's border
// figure), centred on the query over a zero-padded input for SASA (CSDN
// page, section 3.1 after Eq. 4 and section 3.2) -- forms (q.k + bias) /
// sqrt(d) for each neighbour (Eq. 2 and Eq. 4), keeps a running softmax
// (max, sum) and accumulates the weighted values (Eq. 3-4) in registers.  A
// padded SASA neighbour is a zero key and a zero value: its logit is the bias
// alone and it adds to the softmax sum but not to the output.  Keys and
// values come straight from global memory; neighbouring lanes share most of
// their windows, so the L1/L2 caches absorb the re-reads.
//
// Numerics: products and sums in fp32 (fma), the logit is pre-multiplied by
// log2(e) so the exponential is exp2; the running max is subtracted before
// exponentiating, which changes no value exactly.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(_Float16 x) { return static_cast<float>(x); }
__device__ inline float to_f32(__bf16 x) { return static_cast<float>(x); }

// Start of the window of `ks` positions around i on an axis of length L: for
// NA the ks nearest positions, shifted inward at the borders; for SASA the
// window centred on i (it may reach past either end).
template <int MODE>
__device__ inline int window_start(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    if constexpr (MODE == NA_WINDOW_NA) {
        s = s < 0 ? 0 : s;
        s = s > L - ks ? L - ks : s;
    }
    return s;
}

// Load D consecutive elements (16-byte aligned) and widen them to fp32.
template <typename T, int D>
__device__ inline void load_row(const T *__restrict__ p, float (&dst)[D])
{
    constexpr int per = 16 / sizeof(T);  // elements per 16-byte load
    static_assert(D % per == 0, "row must be a whole number of 16-byte chunks");
    const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int c = 0; c < D / per; ++c) {
        const uint4 w = p4[c];
        const T *e = reinterpret_cast<const T *>(&w);
#pragma unroll
        for (int j = 0; j < per; ++j) dst[c * per + j] = to_f32(e[j]);
    }
}

struct Grid {
    int heads, L0, L1, L2;  // depth, height, width
    int k0, k1, k2;         // window per axis
};

template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void na_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ kk, const T *__restrict__ v,
    const float *__restrict__ rpb, float *__restrict__ out, float *__restrict__ lse, Grid g, float c,
    int64_t nq)
{
    // consecutive queries (neighbouring windows) stay on one XCD
    const int64_t gid =
        static_cast<int64_t>(xcd_tile(blockIdx.x, gridDim.x)) * blockDim.x + threadIdx.x;
    if (gid >= nq) return;
    int64_t t = gid;
    const int x = static_cast<int>(t % g.L2);
    t /= g.L2;
    const int y = static_cast<int>(t % g.L1);
    t /= g.L1;
    const int z = static_cast<int>(t % g.L0);
    t /= g.L0;  // t = b * heads + h
    const int h = static_cast<int>(t % g.heads);
    const int64_t map = t * g.L0 * g.L1 * g.L2;  // first position of this (b, h) grid

    float qf[D];
    load_row<T, D>(q + gid * D, qf);

    const int s0 = window_start<MODE>(z, g.k0, g.L0);
    const int s1 = window_start<MODE>(y, g.k1, g.L1);
    const int s2 = window_start<MODE>(x, g.k2, g.L2);
    const int nb0 = 2 * g.k0 - 1, nb1 = 2 * g.k1 - 1, nb2 = 2 * g.k2 - 1;
    const float *bias = rpb ? rpb + static_cast<int64_t>(h) * nb0 * nb1 * nb2 : nullptr;

    float m = -INFINITY, l = 0.f;
    float o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = 0.f;

    for (int a0 = 0; a0 < g.k0; ++a0) {
        const int kz = s0 + a0;
        const bool in0 = (unsigned)kz < (unsigned)g.L0;
        for (int a1 = 0; a1 < g.k1; ++a1) {
            const int ky = s1 + a1;
            const bool in01 = in0 && (unsigned)ky < (unsigned)g.L1;
            const int64_t row = map + (static_cast<int64_t>(kz) * g.L1 + ky) * g.L2;
            // bias row of this (kz, ky), indexed by kx - x + k2 - 1 below
            const float *brow =
                bias ? bias + ((kz - z + g.k0 - 1) * nb1 + (ky - y + g.k1 - 1)) * nb2 + (g.k2 - 1 - x)
                     : nullptr;
            for (int a2 = 0; a2 < g.k2; ++a2) {
                const int kx = s2 + a2;
                const bool inside = in01 && (unsigned)kx < (unsigned)g.L2;
                float dot = 0.f;
                if (inside) {
                    float kf[D];
                    load_row<T, D>(kk + (row + kx) * D, kf);
#pragma unroll
                    for (int e = 0; e < D; ++e) dot = fmaf(qf[e], kf[e], dot);
                }
                const float b = brow ? brow[kx] : 0.f;
                const float s = (dot + b) * c;  // (q.k + B) / sqrt(d), in log2 units
                if (s > m) {                    // new running max: rescale what we have
                    const float corr = exp2f(m - s);
                    l *= corr;
#pragma unroll
                    for (int e = 0; e < D; ++e) o[e] *= corr;
                    m = s;
                }
                const float p = exp2f(s - m);
                l += p;
                if (inside) {
                    float vf[D];
                    load_row<T, D>(v + (row + kx) * D, vf);
#pragma unroll
                    for (int e = 0; e < D; ++e) o[e] = fmaf(p, vf[e], o[e]);
                }
            }
        }
    }
    const float inv = 1.f / l;
    if (lse) lse[gid] = (m + log2f(l)) * 0.6931471805599453f;  // ln of the sum of exp(logits)
    float4 *dst = reinterpret_cast<float4 *>(out + gid * D);
#pragma unroll
    for (int e = 0; e < D / 4; ++e)
        dst[e] = make_float4(o[4 * e] * inv, o[4 * e + 1] * inv, o[4 * e + 2] * inv,
                             o[4 * e + 3] * inv);
}

template <typename T, int D, int MODE>
hipError_t launch_typed(const Problem &p, hipStream_t stream)
{
    const int64_t nq = static_cast<int64_t>(p.B) * p.heads * p.depth * p.H * p.W;
    const int threads = 256;
    const int64_t blocks = static_cast<int64_t>(xcd_grid((nq + threads - 1) / threads));
    const float c = 1.4426950408889634f / sqrtf(static_cast<float>(D));
    const Grid g{p.heads, p.depth, p.H, p.W, p.kd, p.kh, p.kw};
    hipLaunchKernelGGL((na_valu_kernel<T, D, MODE>), dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), 0, stream, static_cast<const T *>(p.q),
                       static_cast<const T *>(p.k), static_cast<const T *>(p.v), p.rpb, p.out, p.lse,
                       g, c, nq);
    return hipGetLastError();
}

template <typename T, int MODE>
hipError_t launch_dim(const Problem &p, hipStream_t stream)
{
    switch (p.d) {
    case 16: return launch_typed<T, 16, MODE>(p, stream);
    case 32: return launch_typed<T, 32, MODE>(p, stream);
    case 64: return launch_typed<T, 64, MODE>(p, stream);
    case 128: return launch_typed<T, 128, MODE>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_mode(const Problem &p, hipStream_t stream)
{
    return p.mode == NA_WINDOW_SASA ? launch_dim<T, NA_WINDOW_SASA>(p, stream)
                                    : launch_dim<T, NA_WINDOW_NA>(p, stream);
}

}  // namespace

hipError_t launch_valu(const Problem &p, hipStream_t stream)
{
    switch (p.dtype) {
    case NA2D_F32: return launch_mode<float>(p, stream);
    case NA2D_F16: return launch_mode<_Float16>(p, stream);
    case NA2D_BF16: return launch_mode<__bf16>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace na2d
