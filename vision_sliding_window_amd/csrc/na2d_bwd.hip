// na2d_bwd.hip -- gradients of the fused NA2D forward (fp32 vector arithmetic).
//
// Forward ("Neighborhood Attention Transformer", CSDN translation, section
// 3.1, Eq. 2-4), per query i of a (b, h) map and key j of its clamped window:
//   s_ij = (q_i . k_j + B[h][j - i + k - 1]) / sqrt(d),  p = softmax_j(s),
//   o_i = sum_j p_ij v_j.
// For the upstream gradient g_i = dL/do_i the chain rule gives
//   dS_ij = p_ij (g_i . v_j - g_i . o_i)
//   dq_i = sum_j dS_ij k_j / sqrt(d)              (query kernel)
//   dB[h][off] += dS_ij / sqrt(d)                  (query kernel)
//   dk_j = sum_{i : j in N(i)} dS_ij q_i / sqrt(d) (key kernel)
//   dv_j = sum_{i : j in N(i)} p_ij g_i            (key kernel)
// No k^2-wide tensor is stored: the query kernel keeps, per query, the
// log-sum-exp of its logits and D_i = g_i . o_i in a workspace (8 bytes per
// query), from which the key kernel recomputes p_ij and dS_ij for every query
// whose window holds its key.  Those queries form, on each axis, the
// contiguous range of positions whose clamped window start lies in
// [j - k + 1, j] (holders() gives its ends in closed form).
#include "na2d.h"
#include "na2d_launch.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace na2d {
namespace {

constexpr int kThreadsB = 256;
constexpr int kLdsBias = 4096;  // bias-gradient entries accumulated in LDS ((2k-1)^2 <= this)

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(_Float16 x) { return static_cast<float>(x); }
__device__ inline float to_f32(__bf16 x) { return static_cast<float>(x); }

__device__ inline int window_start(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
}

// The positions of an axis of length L whose clamped window of ks holds
// position j: [lo, hi].  The window start s(i) = clamp(i - r, 0, L - ks) is
// non-decreasing, so they are the i with j - ks + 1 <= s(i) <= j.  Low end:
// if j < ks every window starting at 0 holds j, so lo = 0; otherwise s(i) >= 1
// forces the unclamped branch s(i) = i - r, i >= j - r.  High end: if
// j >= L - ks every window start (at most L - ks) is <= j, so hi = L - 1;
// otherwise s(i) = i - r <= j, i <= j + r.
__device__ inline void holders(int j, int ks, int L, int &lo, int &hi)
{
    const int r = ks >> 1;
    lo = j < ks ? 0 : j - r;
    hi = j >= L - ks ? L - 1 : j + r;
}

template <typename T, int D>
__device__ inline void load_row(const T *__restrict__ p, float (&dst)[D])
{
    constexpr int per = 16 / sizeof(T);
    const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
#pragma unroll
    for (int c = 0; c < D / per; ++c) {
        const uint4 w = p4[c];
        const T *e = reinterpret_cast<const T *>(&w);
#pragma unroll
        for (int j = 0; j < per; ++j) dst[c * per + j] = to_f32(e[j]);
    }
}

struct BwdArgs {
    const void *q, *k, *v;
    const float *rpb, *out, *dout;
    const float *lse_in;  // the forward's per-query log-sum-exp (natural log), or null
    float *dq, *dk, *dv, *drpb;
    float2 *ws;  // per query: (log2-sum-exp of the log2-scaled logits, g . o)
    int heads, H, W, ks;
    int blocks_per_map;
    unsigned nblocks;
    float c;      // log2(e) / sqrt(d): logits in log2 units
    float scale;  // 1 / sqrt(d)
};

__global__ void zero_kernel(float *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// One query per lane; a workgroup never spans two (b, h) maps, so its bias
// gradient is one head's table.
template <typename T, int D>
__global__ __launch_bounds__(kThreadsB) void bwd_query_kernel(BwdArgs a)
{
    __shared__ float dbias[kLdsBias];
    const unsigned blk = xcd_tile(blockIdx.x, gridDim.x);  // neighbouring blocks share an L2
    if (blk >= a.nblocks) return;  // uniform per workgroup, before any barrier
    const int map = blk / a.blocks_per_map;  // b * heads + h
    const int h = map % a.heads;
    const int H = a.H, W = a.W, ks = a.ks, nb = 2 * ks - 1;
    const bool lds_bias = a.drpb && nb * nb <= kLdsBias;
    if (lds_bias)
        for (int e = threadIdx.x; e < nb * nb; e += kThreadsB) dbias[e] = 0.f;
    __syncthreads();

    const int pix = (blk - map * a.blocks_per_map) * kThreadsB + threadIdx.x;
    if (pix < H * W) {
        const int y = pix / W, x = pix - y * W;
        const int64_t base = (int64_t)map * H * W;
        const int64_t qi = base + pix;
        float qf[D], gf[D];
        load_row<T, D>(static_cast<const T *>(a.q) + qi * D, qf);
        load_row<float, D>(a.dout + qi * D, gf);
        float go = 0.f;
        {
            float of[D];
            load_row<float, D>(a.out + qi * D, of);
#pragma unroll
            for (int e = 0; e < D; ++e) go = fmaf(gf[e], of[e], go);
        }
        const int sy = window_start(y, ks, H), sx = window_start(x, ks, W);
        const float *bias = a.rpb ? a.rpb + (int64_t)h * nb * nb : nullptr;
        const T *kk = static_cast<const T *>(a.k);
        const T *vv = static_cast<const T *>(a.v);
        // pass 1: softmax statistics (online max and sum, log2 units), unless
        // the forward's log-sum-exp is given
        float lse;
        if (a.lse_in) {
            lse = a.lse_in[qi] * 1.4426950408889634f;  // to log2 units
        } else {
            float m = -INFINITY, l = 0.f;
            for (int ay = 0; ay < ks; ++ay) {
                const int64_t row = base + (int64_t)(sy + ay) * W;
                for (int ax = 0; ax < ks; ++ax) {
                    float kf[D];
                    load_row<T, D>(kk + (row + sx + ax) * D, kf);
                    float dot = 0.f;
#pragma unroll
                    for (int e = 0; e < D; ++e) dot = fmaf(qf[e], kf[e], dot);
                    const float b =
                        bias ? bias[(sy + ay - y + ks - 1) * nb + (sx + ax - x + ks - 1)] : 0.f;
                    const float s = (dot + b) * a.c;
                    if (s > m) {
                        l *= exp2f(m - s);
                        m = s;
                    }
                    l += exp2f(s - m);
                }
            }
            lse = m + log2f(l);
        }
        a.ws[qi] = make_float2(lse, go);
        // pass 2: dS_ij, dq_i and the bias gradient
        float dqf[D];
#pragma unroll
        for (int e = 0; e < D; ++e) dqf[e] = 0.f;
        for (int ay = 0; ay < ks; ++ay) {
            const int64_t row = base + (int64_t)(sy + ay) * W;
            for (int ax = 0; ax < ks; ++ax) {
                const int64_t kj = row + sx + ax;
                float kf[D], vf[D];
                load_row<T, D>(kk + kj * D, kf);
                load_row<T, D>(vv + kj * D, vf);
                float dot = 0.f, gv = 0.f;
#pragma unroll
                for (int e = 0; e < D; ++e) {
                    dot = fmaf(qf[e], kf[e], dot);
                    gv = fmaf(gf[e], vf[e], gv);
                }
                const int bi = (sy + ay - y + ks - 1) * nb + (sx + ax - x + ks - 1);
                const float b = bias ? bias[bi] : 0.f;
                const float p = exp2f((dot + b) * a.c - lse);
                const float ds = p * (gv - go);
#pragma unroll
                for (int e = 0; e < D; ++e) dqf[e] = fmaf(ds, kf[e], dqf[e]);
                if (a.drpb) {
                    if (lds_bias) atomicAdd(&dbias[bi], ds * a.scale);
                    else atomicAdd(&a.drpb[(int64_t)h * nb * nb + bi], ds * a.scale);
                }
            }
        }
        float4 *dst = reinterpret_cast<float4 *>(a.dq + qi * D);
#pragma unroll
        for (int e = 0; e < D / 4; ++e)
            dst[e] = make_float4(dqf[4 * e] * a.scale, dqf[4 * e + 1] * a.scale,
                                 dqf[4 * e + 2] * a.scale, dqf[4 * e + 3] * a.scale);
    }
    if (lds_bias) {
        __syncthreads();
        for (int e = threadIdx.x; e < nb * nb; e += kThreadsB)
            if (dbias[e] != 0.f) atomicAdd(&a.drpb[(int64_t)h * nb * nb + e], dbias[e]);
    }
}

// One key per lane: dk_j and dv_j from every query whose window holds j.
template <typename T, int D>
__global__ __launch_bounds__(kThreadsB) void bwd_key_kernel(BwdArgs a)
{
    const unsigned blk = xcd_tile(blockIdx.x, gridDim.x);
    if (blk >= a.nblocks) return;
    const int map = blk / a.blocks_per_map;
    const int h = map % a.heads;
    const int H = a.H, W = a.W, ks = a.ks, nb = 2 * ks - 1;
    const int pix = (blk - map * a.blocks_per_map) * kThreadsB + threadIdx.x;
    if (pix >= H * W) return;
    const int ky = pix / W, kx = pix - ky * W;
    const int64_t base = (int64_t)map * H * W;
    const int64_t kj = base + pix;
    float kf[D], vf[D];
    load_row<T, D>(static_cast<const T *>(a.k) + kj * D, kf);
    load_row<T, D>(static_cast<const T *>(a.v) + kj * D, vf);
    const float *bias = a.rpb ? a.rpb + (int64_t)h * nb * nb : nullptr;
    const T *qq = static_cast<const T *>(a.q);
    float dkf[D], dvf[D];
#pragma unroll
    for (int e = 0; e < D; ++e) dkf[e] = dvf[e] = 0.f;
    int y0, y1, x0, x1;
    holders(ky, ks, H, y0, y1);
    holders(kx, ks, W, x0, x1);
    for (int y = y0; y <= y1; ++y) {
        for (int x = x0; x <= x1; ++x) {
            const int64_t qi = base + (int64_t)y * W + x;
            float qf[D], gf[D];
            load_row<T, D>(qq + qi * D, qf);
            load_row<float, D>(a.dout + qi * D, gf);
            const float2 st = a.ws[qi];
            float dot = 0.f, gv = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) {
                dot = fmaf(qf[e], kf[e], dot);
                gv = fmaf(gf[e], vf[e], gv);
            }
            const float b = bias ? bias[(ky - y + ks - 1) * nb + (kx - x + ks - 1)] : 0.f;
            const float p = exp2f((dot + b) * a.c - st.x);
            const float ds = p * (gv - st.y);
#pragma unroll
            for (int e = 0; e < D; ++e) {
                dkf[e] = fmaf(ds, qf[e], dkf[e]);
                dvf[e] = fmaf(p, gf[e], dvf[e]);
            }
        }
    }
    float4 *dk4 = reinterpret_cast<float4 *>(a.dk + kj * D);
    float4 *dv4 = reinterpret_cast<float4 *>(a.dv + kj * D);
#pragma unroll
    for (int e = 0; e < D / 4; ++e) {
        dk4[e] = make_float4(dkf[4 * e] * a.scale, dkf[4 * e + 1] * a.scale, dkf[4 * e + 2] * a.scale,
                             dkf[4 * e + 3] * a.scale);
        dv4[e] = make_float4(dvf[4 * e], dvf[4 * e + 1], dvf[4 * e + 2], dvf[4 * e + 3]);
    }
}

template <typename T, int D>
hipError_t launch_bwd_typed(const BwdProblem &p, hipStream_t stream)
{
    BwdArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
    a.lse_in = p.lse;
    a.dout = p.dout;
    a.dq = p.dq;
    a.dk = p.dk;
    a.dv = p.dv;
    a.drpb = p.drpb;
    a.ws = reinterpret_cast<float2 *>(p.workspace);
    a.heads = p.heads;
    a.H = p.H;
    a.W = p.W;
    a.ks = p.ksize;
    a.blocks_per_map = (p.H * p.W + kThreadsB - 1) / kThreadsB;
    a.c = 1.4426950408889634f / sqrtf((float)D);
    a.scale = 1.f / sqrtf((float)D);
    const uint64_t blocks = (uint64_t)p.B * p.heads * a.blocks_per_map;
    if (blocks == 0 || xcd_grid(blocks) > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.nblocks = (unsigned)blocks;
    // both passes run on the matrix cores where they apply
    if (p.algo == NA2D_ALGO_MFMA) return launch_backward_mfma(p, stream);
    if (p.drpb) {  // the bias gradient accumulates: clear it first (a kernel, not a memset)
        const int n = p.heads * (2 * p.ksize - 1) * (2 * p.ksize - 1);
        hipLaunchKernelGGL(zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p.drpb, n);
    }
    const dim3 grid((unsigned)xcd_grid(blocks));
    hipLaunchKernelGGL((bwd_query_kernel<T, D>), grid, dim3(kThreadsB), 0, stream, a);
    hipLaunchKernelGGL((bwd_key_kernel<T, D>), grid, dim3(kThreadsB), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dim(const BwdProblem &p, hipStream_t stream)
{
    switch (p.d) {
    case 16: return launch_bwd_typed<T, 16>(p, stream);
    case 32: return launch_bwd_typed<T, 32>(p, stream);
    case 64: return launch_bwd_typed<T, 64>(p, stream);
    case 128: return launch_bwd_typed<T, 128>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_backward(const BwdProblem &p, hipStream_t stream)
{
    switch (p.dtype) {
    case NA2D_F32: return launch_bwd_dim<float>(p, stream);
    case NA2D_F16: return launch_bwd_dim<_Float16>(p, stream);
    case NA2D_BF16: return launch_bwd_dim<__bf16>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace na2d
