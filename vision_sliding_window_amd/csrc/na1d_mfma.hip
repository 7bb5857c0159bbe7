// na1d_mfma.hip -- NA1D forward for fp16/bf16 inputs on the gfx950 matrix cores.
//
// The operation is Neighborhood Attention over a sequence ("Neighborhood
// Attention Transformer", CSDN translation, section 3.1, Eq. 2-4, with the
// 1D module of section 3.2): query x attends to the k positions
// [sx, sx + k), sx = clamp(x - k/2, 0, L - k), with logits
// (q.k + B[key - x + k - 1]) / sqrt(d), a softmax over the window and the
// weighted sum of the values.
//
// How.  A workgroup of four waves takes 64 consecutive queries of one
// (b, h) sequence.
//  1. Staging.  The K and V halo -- 64 + NC positions from the window start
//     of the tile's first query, enough for every wave's candidates -- goes
//     to LDS as [position][4 x 16-byte d-slices], slice s of position p at
//     slot s ^ ((p >> 2) & 3).  Positions past the sequence load as zeros.
//  2. Logits.  A wave owns 16 queries; their windows together span at most
//     15 + k positions, read as NCB blocks of 16 from the window start of the
//     wave's first query.  S^T = K_block Q^T is one v_mfma_f32_16x16x32 per
//     block (d = 32 is the contraction): lane (g, i) then holds query i and
//     keys 4 g .. 4 g + 3 of the block.  The bias of a key inside the query's
//     window comes from the scaled (2k-1) table in LDS; a key outside it reads
//     the table's trailing -inf, which masks it exactly.
//  3. Softmax over the wave's candidates in one pass: row max and sum over
//     the 4 lanes of a query (v_permlane16/32_swap), p = exp2(s - m).
//  4. O^T = V^T P^T by v_mfma_f32_16x16x32 over pairs of key blocks, V^T
//     fragments from ds_read_b64_tr_b16; P is fp16 for fp16 inputs and a
//     bf16 hi + lo pair for bf16 inputs.
//  5. out = O / sum, fp32, 16-byte buffer stores; positions past the
//     sequence are dropped by the range check.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_mfma_util.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

constexpr int kW1 = 4;          // waves per workgroup
constexpr int kT1 = 64 * kW1;   // threads per workgroup
constexpr int kTQ = 16 * kW1;   // queries per tile
constexpr int kMaxRaw = 2 * NA1D_MFMA_MAX_KSIZE;  // (2k-1) bias values + the -inf slot

struct Args1 {
    const void *q, *k, *v;
    const float *rpb;
    float *out;
    int heads, L, ks;
    int tiles_per_seq;
    unsigned ntiles;
    float c;  // log2(e) / sqrt(d)
};

__device__ inline int window_start_1d(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
}

// LDS byte offset of d-slice `s` of halo position `p`.
__device__ inline unsigned slot_offset(int p, int s)
{
    return (unsigned)p * 64u + 16u * (unsigned)(s ^ ((p >> 2) & 3));
}

template <typename T, int NCB>
__global__ __launch_bounds__(kT1) void na1d_mfma_kernel(Args1 a)
{
    using FragT = typename Frag<T>::type;
    constexpr int NC = 16 * NCB;        // candidate keys per wave
    constexpr int HP = (kTQ + NC + 63) / 64 * 64;  // halo positions held in LDS (>= 64 + NC)
    static_assert(NCB % 2 == 0, "P.V consumes key blocks in pairs");
    __shared__ __align__(16) unsigned char kh[HP * 64];
    __shared__ __align__(16) unsigned char vh[HP * 64];
    __shared__ float braw[kMaxRaw];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);  // neighbouring tiles share an L2
    if (tile >= a.ntiles) return;
    const int seq = tile / a.tiles_per_seq;                 // b * heads + h
    const int x0 = (tile - seq * a.tiles_per_seq) * kTQ;    // first query of the tile
    const int h = seq % a.heads;
    const int ks = a.ks, L = a.L;
    const int64_t base = (int64_t)seq * L;
    const unsigned seq_bytes = (unsigned)L * 64u;
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, base, 64, seq_bytes);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, base, 64, seq_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, base, 64, seq_bytes);

    // 1. halo [hx0, hx0 + HP) -> LDS (zeros past the sequence), bias -> LDS
    const int hx0 = window_start_1d(x0, ks, L);
    constexpr int CHUNKS = HP * 4;  // 16-byte chunks per tensor
    static_assert(CHUNKS % kT1 == 0, "whole chunks per thread");
    u32x4 kr[CHUNKS / kT1], vr[CHUNKS / kT1];
#pragma unroll
    for (int e = 0; e < CHUNKS / kT1; ++e) {
        const int ch = e * kT1 + tid, p = ch >> 2, s = ch & 3;
        const int gx = hx0 + p;
        const unsigned off = gx < L ? (unsigned)gx * 64u + 16u * s : kOutOfRange;
        kr[e] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        vr[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
    // this lane's query fragment: slice g of query i (the B operand of S^T)
    const int g = lane >> 4, qi = lane & 15;
    const int x = x0 + 16 * wave + qi;
    const u32x4 qv =
        __builtin_amdgcn_raw_buffer_load_b128(rq, x < L ? (unsigned)x * 64u + 16u * g : kOutOfRange, 0, 0);
    const int nb = 2 * ks - 1;
    float bv = 0.f;
    if (a.rpb && tid < nb) bv = a.rpb[(int64_t)h * nb + tid];
#pragma unroll
    for (int e = 0; e < CHUNKS / kT1; ++e) {
        const int ch = e * kT1 + tid, p = ch >> 2, s = ch & 3;
        *reinterpret_cast<u32x4 *>(kh + slot_offset(p, s)) = kr[e];
        *reinterpret_cast<u32x4 *>(vh + slot_offset(p, s)) = vr[e];
    }
    if (tid < nb) braw[tid] = bv * a.c;
    if (tid == nb) braw[tid] = -__builtin_inff();
    __syncthreads();

    // 2. logits of the wave's 16 queries against its NC candidates
    const FragT qf = __builtin_bit_cast(FragT, qv);
    const int xc = min(x, L - 1);                 // queries past the end compute a copy
    const int sx = window_start_1d(xc, ks, L);
    const int cw = window_start_1d(min(x0 + 16 * wave, L - 1), ks, L);  // wave's first candidate
    const int pb = cw - hx0;                      // its halo position
    lds_cu8 *kp = (lds_cu8 *)(kh + slot_offset(pb + qi, g));
    const int pv = pb + 4 * g + (qi >> 2);        // the position this lane feeds to the V^T read
    const int sv = (qi >> 1) & 1;
    lds_cu8 *vp0 = (lds_cu8 *)(vh + slot_offset(pv, sv) + 8u * (qi & 1));
    lds_cu8 *vp1 = (lds_cu8 *)(vh + slot_offset(pv, 2 + sv) + 8u * (qi & 1));
    opaque(kp);
    opaque(vp0);
    opaque(vp1);

    float sc[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const FragT kf = __builtin_bit_cast(FragT, *(lds_cu4 *)(kp + cb * 1024));
        const floatx4 acc = mfma16x16x32(kf, qf, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = cw + 16 * cb + 4 * g + j;
            const int bi = (unsigned)(key - sx) < (unsigned)ks ? key - xc + ks - 1 : nb;
            sc[cb][j] = fmaf(acc[j], a.c, braw[bi]);
        }
    }
    // 3. softmax
    float m = -__builtin_inff();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, sc[cb][j]);
    m = quad_max(m);  // every query has k >= 1 keys in range, so m is finite
    floatx4 o[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    float lsum = 0.f;
    // 4. O^T = V^T P^T over pairs of key blocks
#pragma unroll
    for (int cb = 0; cb < NCB; cb += 2) {
        FragT vf[2];
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) {
            lds_cu8 *vp = dh ? vp1 : vp0;
            const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vp + cb * 1024));
            const v4i16 vb =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vp + (cb + 1) * 1024));
            vf[dh] = __builtin_bit_cast(FragT, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = __builtin_amdgcn_exp2f(sc[cb][j] - m);
            p[4 + j] = __builtin_amdgcn_exp2f(sc[cb + 1][j] - m);
        }
        if constexpr (__is_same(T, _Float16)) {
            half8 pf;
#pragma unroll
            for (int j = 0; j < 8; ++j) pf[j] = static_cast<_Float16>(p[j]);
            // the sum takes the rounded weights, so it matches what multiplies V
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                lsum = __builtin_amdgcn_fdot2(half2{pf[j], pf[j + 1]}, half2{1, 1}, lsum, false);
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) o[dh] = mfma16x16x32(vf[dh], pf, o[dh]);
        } else {
            bf16x8 ph, pl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                ph[j] = static_cast<__bf16>(p[j]);
                pl[j] = static_cast<__bf16>(p[j] - static_cast<float>(ph[j]));
                lsum += p[j];
            }
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                o[dh] = mfma16x16x32(vf[dh], ph, o[dh]);
                o[dh] = mfma16x16x32(vf[dh], pl, o[dh]);
            }
        }
    }
    // 5. normalise and store: lane (g, i) holds dims 16 dh + 4 g + j of query i
    const float inv = __builtin_amdgcn_rcpf(quad_sum(lsum));
    const __amdgpu_buffer_rsrc_t ro = map_rsrc(a.out, base, 128, (unsigned)L * 128u);
    const unsigned off = x < L ? (unsigned)x * 128u + 16u * g : kOutOfRange;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
        const floatx4 r = o[dh] * inv;
        // non-temporal: nothing reads the output again
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r), ro, off + 64u * dh, 0,
                                               kNonTemporal);
    }
}

template <typename T, int NCB>
hipError_t launch_ncb(const Problem &p, hipStream_t stream)
{
    Args1 a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
    a.heads = p.heads;
    a.L = p.W;
    a.ks = p.kw;
    a.tiles_per_seq = (p.W + kTQ - 1) / kTQ;
    a.c = 1.4426950408889634f / sqrtf(32.f);
    const uint64_t blocks = (uint64_t)p.B * p.heads * a.tiles_per_seq;
    if (blocks == 0 || xcd_grid(blocks) > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.ntiles = (unsigned)blocks;
    hipLaunchKernelGGL((na1d_mfma_kernel<T, NCB>), dim3((unsigned)xcd_grid(blocks)), dim3(kT1), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const Problem &p, hipStream_t stream)
{
    // a wave's candidates: 15 + k positions, in an even number of 16-key blocks
    const int ks = p.kw;
    if (15 + ks <= 32) return launch_ncb<T, 2>(p, stream);
    if (15 + ks <= 64) return launch_ncb<T, 4>(p, stream);
    return launch_ncb<T, 6>(p, stream);
}

}  // namespace

hipError_t launch_mfma_1d(const Problem &p, hipStream_t stream)
{
    if (p.d != 32 || p.depth != 1 || p.H != 1 || p.kd != 1 || p.kh != 1 || p.mode != NA_WINDOW_NA ||
        p.kw < 3 || p.kw > NA1D_MFMA_MAX_KSIZE || (uint64_t)p.W * 128u > 0x7fffffffull || p.lse)
        return hipErrorInvalidValue;
    if (p.dtype == NA2D_F16) return launch_typed<_Float16>(p, stream);
    if (p.dtype == NA2D_BF16) return launch_typed<__bf16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace na2d
