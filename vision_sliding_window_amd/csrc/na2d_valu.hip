// na2d_valu.hip -- NA2D forward, one query per lane, fp32 vector arithmetic.
//
// This is the plain kernel of the library: it serves float32 inputs, head
// dims 16/32/64/128 and kernel sizes up to 63, and it is the baseline the
// matrix-core kernel is measured against.  Each lane owns one query
// (b, h, y, x): it walks the ksize x ksize clamped window (CSDN translation of
// "Neighborhood Attention Transformer", section 3.1 and the qiita article's
// border figure), forms (q.k + bias) / sqrt(d) for each neighbour (Eq. 2 and
// Eq. 4), keeps a running softmax (max, sum) and accumulates the weighted
// values (Eq. 3-4) in registers.  Keys and values come straight from global
// memory; neighbouring lanes share most of their windows, so the L1/L2 caches
// absorb the re-reads.
//
// Numerics: products and sums in fp32 (fma), the logit is pre-multiplied by
// log2(e) so the exponential is exp2; the running max is subtracted before
// exponentiating, which changes no value exactly.
#include "na2d.h"
#include "na2d_launch.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(_Float16 x) { return static_cast<float>(x); }
__device__ inline float to_f32(__bf16 x) { return static_cast<float>(x); }

// Start of the window of `ks` pixels around i on an axis of length L: the ks
// nearest pixels, shifted inward at the borders.
__device__ inline int window_start(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
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

template <typename T, int D>
__global__ __launch_bounds__(256) void na2d_valu_kernel(
    const T *__restrict__ q, const T *__restrict__ kk, const T *__restrict__ v,
    const float *__restrict__ rpb, float *__restrict__ out, int heads, int H, int W, int ks,
    float c, int64_t nq)
{
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (gid >= nq) return;
    const int x = static_cast<int>(gid % W);
    int64_t t = gid / W;
    const int y = static_cast<int>(t % H);
    t /= H;  // t = b * heads + h
    const int h = static_cast<int>(t % heads);
    const int64_t map = t * H * W;  // first pixel of this (b, h) map

    float qf[D];
    load_row<T, D>(q + gid * D, qf);

    const int sy = window_start(y, ks, H);
    const int sx = window_start(x, ks, W);
    const int nb = 2 * ks - 1;
    const float *bias = rpb ? rpb + static_cast<int64_t>(h) * nb * nb : nullptr;

    float m = -INFINITY, l = 0.f;
    float o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = 0.f;

    for (int a = 0; a < ks; ++a) {
        const int ky = sy + a;
        const int64_t row = map + static_cast<int64_t>(ky) * W;
        const float *brow = bias ? bias + (ky - y + ks - 1) * nb + (ks - 1 - x) : nullptr;
        for (int cc = 0; cc < ks; ++cc) {
            const int kx = sx + cc;
            float kf[D];
            load_row<T, D>(kk + (row + kx) * D, kf);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) dot = fmaf(qf[e], kf[e], dot);
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
            float vf[D];
            load_row<T, D>(v + (row + kx) * D, vf);
#pragma unroll
            for (int e = 0; e < D; ++e) o[e] = fmaf(p, vf[e], o[e]);
        }
    }
    const float inv = 1.f / l;
    float4 *dst = reinterpret_cast<float4 *>(out + gid * D);
#pragma unroll
    for (int e = 0; e < D / 4; ++e)
        dst[e] = make_float4(o[4 * e] * inv, o[4 * e + 1] * inv, o[4 * e + 2] * inv,
                             o[4 * e + 3] * inv);
}

template <typename T, int D>
hipError_t launch_typed(const Problem &p, hipStream_t stream)
{
    const int64_t nq = static_cast<int64_t>(p.B) * p.heads * p.H * p.W;
    const int threads = 256;
    const int64_t blocks = (nq + threads - 1) / threads;
    const float c = 1.4426950408889634f / sqrtf(static_cast<float>(D));
    hipLaunchKernelGGL((na2d_valu_kernel<T, D>), dim3(static_cast<unsigned>(blocks)),
                       dim3(threads), 0, stream, static_cast<const T *>(p.q),
                       static_cast<const T *>(p.k), static_cast<const T *>(p.v), p.rpb, p.out,
                       p.heads, p.H, p.W, p.ksize, c, nq);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dim(const Problem &p, hipStream_t stream)
{
    switch (p.d) {
    case 16: return launch_typed<T, 16>(p, stream);
    case 32: return launch_typed<T, 32>(p, stream);
    case 64: return launch_typed<T, 64>(p, stream);
    case 128: return launch_typed<T, 128>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_valu(const Problem &p, hipStream_t stream)
{
    switch (p.dtype) {
    case NA2D_F32: return launch_dim<float>(p, stream);
    case NA2D_F16: return launch_dim<_Float16>(p, stream);
    case NA2D_BF16: return launch_dim<__bf16>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace na2d
