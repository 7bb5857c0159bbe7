// na2d_bwd_mfma.hip -- gradients of the NA2D forward on the gfx950 matrix
// cores (fp16/bf16 inputs, d = 32).
//
// The chain rule through "Neighborhood Attention Transformer" (CSDN
// translation, section 3.1, Eq. 2-4), for query i, key j of its clamped
// window and upstream gradient g_i:
//   p_ij  = exp(s_ij - lse_i),  s_ij = (q_i . k_j + B[j - i + k - 1]) / sqrt(d)
//   dS_ij = p_ij (g_i . v_j - g_i . o_i)
//   dq_i = sum_j dS_ij k_j / sqrt(d),  dB[off] += dS_ij / sqrt(d)   (query pass)
//   dk_j = sum_i dS_ij q_i / sqrt(d),  dv_j = sum_i p_ij g_i         (key pass)
// Both passes give each wave 16 "own" positions (a 2 x 8 patch) and stream
// the 16-wide blocks of the other side that its windows (query pass) or
// window holders (key pass) touch, straight from L2; no k^2 tensor exists.
//
// Matrix products (v_mfma_f32_16x16x32 / 16x16x16, fp32 accumulate):
//  - logits and g.v: the streamed block as the A operand (rows = its 16
//    positions, one 16-byte d-slice per lane) against the wave's own
//    fragments as B, so lane (g, c) holds the 4 streamed positions 4g..4g+3
//    for own position c;
//  - dv^T += g^T P, dk^T += q^T dS (key pass) and dq^T += k^T dS^T (query
//    pass): the transposed operand comes from a per-wave LDS copy of the
//    streamed block read back with ds_read_b64_tr_b16.
// fp32 operands (g, P, dS) enter the 16-bit products as a high part plus a
// scaled low part (x = hi + lo to ~22 bits for fp16, ~16 for bf16; see
// split), which keeps the gradients at fp32-like accuracy.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_mfma_util.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

constexpr int kBW = 4;         // waves per workgroup (independent: no barrier in the loops)
constexpr int kBT = 64 * kBW;  // threads per workgroup
constexpr int kBMaxRaw = (2 * NA2D_BWD_MFMA_MAX_KSIZE - 1) * (2 * NA2D_BWD_MFMA_MAX_KSIZE - 1);

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

__device__ inline floatx4 mfma16x16x16(const v4i16 &a, const v4i16 &b, const floatx4 &c, _Float16)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4, a),
                                                 __builtin_bit_cast(half4, b), c, 0, 0, 0);
}
__device__ inline floatx4 mfma16x16x16(const v4i16 &a, const v4i16 &b, const floatx4 &c, __bf16)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// x = hi + lo / kLoScale<T> in the 16-bit type T.  The low part is stored
// scaled up by the rounding step of T (2^11 for fp16, 2^8 for bf16) so that it
// stays a normal number even for small x (an fp16 remainder would otherwise
// fall into the subnormal range, which the products do not keep); the
// products of low parts are accumulated apart and scaled back in fp32.
template <typename T> struct LoScale;
template <> struct LoScale<_Float16> { static constexpr float up = 2048.f, down = 1.f / 2048.f; };
template <> struct LoScale<__bf16> { static constexpr float up = 256.f, down = 1.f / 256.f; };

// x is pinned to one fp32 value first: were a product folded into the
// conversions, hi could be rounded once from the exact product where lo is
// formed and twice (via fp32) where hi is kept, and differ by one step.
template <typename T>
__device__ inline void split(float x, T &hi, T &lo)
{
    asm volatile("" : "+v"(x));
    hi = static_cast<T>(x);
    lo = static_cast<T>((x - static_cast<float>(hi)) * LoScale<T>::up);
}

template <typename T>
__device__ inline short bits(T x)
{
    return __builtin_bit_cast(short, x);
}

__device__ inline int wstart(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
}

// positions of an axis whose window holds j (see na2d_bwd.hip)
__device__ inline void holders(int j, int ks, int L, int &lo, int &hi)
{
    const int r = ks >> 1;
    lo = j < ks ? 0 : j - r;
    hi = j >= L - ks ? L - 1 : j + r;
}

struct BArgs {
    const void *q, *k, *v;
    const float *rpb, *out, *dout;
    float *dq, *dk, *dv, *drpb;
    float2 *ws;
    int heads, H, W, ks;
    int tiles_x, tiles_per_map;
    unsigned ntiles;
    float c, scale;
};

struct Patch {  // a workgroup's 8 x 8 own positions
    int map, h, y0, x0;
    int64_t base;
};

__device__ inline Patch patch_of(const BArgs &a, unsigned tile)
{
    Patch p;
    p.map = tile / a.tiles_per_map;
    const int t = tile - p.map * a.tiles_per_map;
    const int ty = t / a.tiles_x;
    p.y0 = ty * 8;
    p.x0 = (t - ty * a.tiles_x) * 8;
    p.h = p.map % a.heads;
    p.base = (int64_t)p.map * a.H * a.W;
    return p;
}

// the head's (2k-1)^2 bias table, scaled to log2 units, into LDS
__device__ inline void stage_raw_bias(const BArgs &a, int h, float *raw)
{
    const int nb = 2 * a.ks - 1;
    for (int e = threadIdx.x; e < nb * nb; e += kBT)
        raw[e] = a.rpb ? a.rpb[(int64_t)h * nb * nb + e] * a.c : 0.f;
}

// slice g of the 16-bit row at (y, x) (lane (g, i) of a block takes x = x0 + i),
// zeros past the map
__device__ inline u32x4 load_slice(__amdgpu_buffer_rsrc_t r, int y, int x, int W, int g)
{
    return __builtin_amdgcn_raw_buffer_load_b128(
        r, x < W ? (unsigned)(y * W + x) * 64u + 16u * (unsigned)g : kOutOfRange, 0, 0);
}

// ---------------------------------------------------------------------------
// Key pass: dk, dv of 16 own keys per wave from every query holding them.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_kv_mfma_kernel(BArgs a)
{
    using FragT = typename Frag<T>::type;
    __shared__ float raw[kBMaxRaw];
    __shared__ __align__(16) unsigned char qbuf[kBW][16 * 64];    // streamed q block [pos][d], 16-bit
    __shared__ __align__(16) unsigned char gbuf[kBW][2][16 * 64]; // streamed g block, hi and lo
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= a.ntiles) return;
    const Patch P = patch_of(a, tile);
    stage_raw_bias(a, P.h, raw);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int H = a.H, W = a.W, ks = a.ks, nb = 2 * ks - 1;
    const int ky1 = P.y0 + 2 * wave;                 // the wave's key rows ky1, ky1 + 1
    if (ky1 >= H) return;
    const int ky = min(ky1 + (c >> 3), H - 1), kx = min(P.x0 + (c & 7), W - 1);
    const bool own_valid = ky1 + (c >> 3) < H && P.x0 + (c & 7) < W;
    const unsigned map_bytes = (unsigned)H * W * 64u;
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, P.base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, P.base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, P.base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rg = map_rsrc(a.dout, P.base, 128, (unsigned)H * W * 128u);
    const __amdgpu_buffer_rsrc_t rw = map_rsrc(a.ws, P.base, 8, (unsigned)H * W * 8u);
    // the wave's own keys as B operands: lane (g, c) holds slice g of key c
    const unsigned own_off = (unsigned)(ky * W + kx) * 64u + 16u * g;
    const FragT kf = __builtin_bit_cast(FragT, __builtin_amdgcn_raw_buffer_load_b128(rk, own_off, 0, 0));
    const FragT vf = __builtin_bit_cast(FragT, __builtin_amdgcn_raw_buffer_load_b128(rv, own_off, 0, 0));

    // the queries holding any of the wave's keys
    int ylo, yhi, xlo, xhi, t0, t1;
    holders(ky1, ks, H, ylo, t0);
    holders(min(ky1 + 1, H - 1), ks, H, t1, yhi);
    holders(P.x0, ks, W, xlo, t0);
    holders(min(P.x0 + 7, W - 1), ks, W, t1, xhi);
    const int nblk = (xhi - xlo + 16) >> 4;

    // main and low-part accumulators (see split)
    floatx4 dk[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
    floatx4 dv[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
    floatx4 dkl[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
    floatx4 dvl[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
    unsigned char *qb = qbuf[wave];
    unsigned char *gbh = gbuf[wave][0], *gbl = gbuf[wave][1];
    // transposed reads: lane (g, i) takes dims 16 dh + 4 (i & 3) .. + 3 of
    // position 4 g + (i >> 2) and receives dim 16 dh + i of positions 4 g .. 4 g + 3
    const unsigned tr_off = (unsigned)(4 * g + (c >> 2)) * 64u + 8u * (unsigned)(c & 3);

    for (int y = ylo; y <= yhi; ++y) {
        const int sy = wstart(y, ks, H);
        for (int b = 0; b < nblk; ++b) {
            const int xb = xlo + 16 * b;
            // streamed block: q and g rows of queries (y, xb + i)
            const u32x4 qv = load_slice(rq, y, xb + c, W, g);
            const unsigned goff = xb + c < W ? (unsigned)(y * W + xb + c) * 128u + 32u * g : kOutOfRange;
            const u32x4 g0 = __builtin_amdgcn_raw_buffer_load_b128(rg, goff, 0, 0);
            const u32x4 g1 = __builtin_amdgcn_raw_buffer_load_b128(rg, goff + 16u, 0, 0);
            // softmax statistics of queries xb + 4 g + r (r = 0..3), zeros past the map
            const unsigned woff = xb + 4 * g < W ? (unsigned)(y * W + xb + 4 * g) * 8u : kOutOfRange;
            const u32x4 w01 = __builtin_amdgcn_raw_buffer_load_b128(rw, woff, 0, 0);
            const u32x4 w23 = __builtin_amdgcn_raw_buffer_load_b128(rw, woff + 16u, 0, 0);
            // q as A operand (the block's positions as rows), its copy for q^T
            *reinterpret_cast<u32x4 *>(qb + (unsigned)c * 64u + 16u * g) = qv;
            FragT gh, gl;
            {
                const floatx4 ga = __builtin_bit_cast(floatx4, g0), gb = __builtin_bit_cast(floatx4, g1);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    T h, l;
                    split<T>(ga[e], h, l);
                    gh[e] = h;
                    gl[e] = l;
                    split<T>(gb[e], h, l);
                    gh[4 + e] = h;
                    gl[4 + e] = l;
                }
            }
            *reinterpret_cast<FragT *>(gbh + (unsigned)c * 64u + 16u * g) = gh;
            *reinterpret_cast<FragT *>(gbl + (unsigned)c * 64u + 16u * g) = gl;
            const FragT qa = __builtin_bit_cast(FragT, qv);
            floatx4 s = mfma16x16x32(qa, kf, floatx4{0, 0, 0, 0});
            const floatx4 gvh = mfma16x16x32(gh, vf, floatx4{0, 0, 0, 0});
            const floatx4 gvl = mfma16x16x32(gl, vf, floatx4{0, 0, 0, 0});
            const floatx4 gv = gvh + gvl * LoScale<T>::down;
            const float lse[4] = {__uint_as_float(w01[0]), __uint_as_float(w01[2]),
                                  __uint_as_float(w23[0]), __uint_as_float(w23[2])};
            const float dd[4] = {__uint_as_float(w01[1]), __uint_as_float(w01[3]),
                                 __uint_as_float(w23[1]), __uint_as_float(w23[3])};
            // p and dS for queries (y, xb + 4 g + r) and key c
            v4i16 ph, pl, sh, sl;
            const bool rowin = own_valid && (unsigned)(ky - sy) < (unsigned)ks;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int x = xb + 4 * g + r;
                const bool in = rowin && x < W && (unsigned)(kx - wstart(min(x, W - 1), ks, W)) < (unsigned)ks;
                // key inside the query's window: the offset indexes the table
                const float bias = raw[in ? (ky - y + ks - 1) * nb + (kx - x + ks - 1) : 0];
                const float p = in ? __builtin_amdgcn_exp2f(s[r] * a.c + bias - lse[r]) : 0.f;
                const float ds = p * (gv[r] - dd[r]);
                T h, l;
                split<T>(p, h, l);
                ph[r] = bits(h);
                pl[r] = bits(l);
                split<T>(ds, h, l);
                sh[r] = bits(h);
                sl[r] = bits(l);
            }
            // dv^T += g^T P and dk^T += q^T dS (16x16x16: 4 queries per lane)
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                const v4i16 qt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(qb + tr_off + 32u * dh));
                const v4i16 gth = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(gbh + tr_off + 32u * dh));
                const v4i16 gtl = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(gbl + tr_off + 32u * dh));
                dv[dh] = mfma16x16x16(gth, ph, dv[dh], T{});
                dvl[dh] = mfma16x16x16(gth, pl, dvl[dh], T{});
                dvl[dh] = mfma16x16x16(gtl, ph, dvl[dh], T{});
                dk[dh] = mfma16x16x16(qt, sh, dk[dh], T{});
                dkl[dh] = mfma16x16x16(qt, sl, dkl[dh], T{});
            }
        }
    }
    // lane (g, c): dims 16 dh + 4 g + j of key c
    if (own_valid) {
        const int64_t kj = P.base + (int64_t)ky * W + kx;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) {
            const floatx4 dkt = dk[dh] + dkl[dh] * LoScale<T>::down;
            const floatx4 dvt = dv[dh] + dvl[dh] * LoScale<T>::down;
            *reinterpret_cast<floatx4 *>(a.dk + kj * 32 + 16 * dh + 4 * g) = dkt * a.scale;
            *reinterpret_cast<floatx4 *>(a.dv + kj * 32 + 16 * dh + 4 * g) = dvt;
        }
    }
}

}  // namespace

// Gradients with the key pass on the matrix cores; the query pass (dq, the
// bias gradient and the workspace) is run by `query_pass` first.
hipError_t launch_backward_kv_mfma(const BwdProblem &p, hipStream_t stream)
{
    BArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
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
    a.tiles_x = (p.W + 7) / 8;
    a.tiles_per_map = a.tiles_x * ((p.H + 7) / 8);
    a.c = 1.4426950408889634f / sqrtf(32.f);
    a.scale = 1.f / sqrtf(32.f);
    const uint64_t tiles = (uint64_t)p.B * p.heads * a.tiles_per_map;
    if (tiles == 0 || xcd_grid(tiles) > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.ntiles = (unsigned)tiles;
    const dim3 grid((unsigned)xcd_grid(tiles));
    if (p.dtype == NA2D_F16)
        hipLaunchKernelGGL(bwd_kv_mfma_kernel<_Float16>, grid, dim3(kBT), 0, stream, a);
    else if (p.dtype == NA2D_BF16)
        hipLaunchKernelGGL(bwd_kv_mfma_kernel<__bf16>, grid, dim3(kBT), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace na2d
