// na2d_mfma.hip -- NA2D forward for fp16/bf16 inputs on the gfx950 matrix cores.
//
// What is computed is Neighborhood Attention ("Neighborhood Attention
// Transformer", CSDN translation, section 3.1, Eq. 2-4): per query the
// clamped ksize x ksize window, logits (q.k + B) / sqrt(d), softmax over the
// window, weighted sum of the values.
//
// How (one workgroup = 4 waves = a TY x TX query tile, TY = 4 * QY, TX = QX):
//  1. The tile's key/value halo -- the union of its queries' windows, at most
//     (TY + ksize - 1) rows by 16 * NCB columns -- is copied once from HBM to
//     LDS with 16-byte loads: K as [row][col][d] (16-byte d-slices swizzled
//     against bank conflicts), V transposed as [d][row][col], plus this head's
//     bias table scaled by log2(e)/sqrt(d) with a row and a column of -inf
//     appended (used for keys outside a query's window).  This is the tiled
//     design of the paperlayer summary's appendix A.4 (a query tile plus a key
//     tile of side tq + k - 1 in on-chip memory), re-shaped for 64-lane waves.
//  2. Each wave owns a QY x QX = 16-query subtile.  Its candidate keys are NR
//     halo rows by 16 * NCB columns, cut into blocks of 16 keys (one row, 16
//     consecutive columns).  For a block, S^T = K_block Q^T is one
//     v_mfma_f32_16x16x32 (d = 32 is the contraction); in the result each lane
//     holds one query (lane % 16) and four consecutive keys (4 * (lane / 16)
//     + j).  Keys outside the query's own window get the -inf bias, so the
//     result is exactly the masked window.
//  3. Softmax is single-pass over chunks of RPC block rows: chunk max across
//     the 4 lanes holding a query (two xor-shuffles), running max / sum with
//     rescale, p = exp2(s - m).
//  4. O^T = V^T P^T, again v_mfma_f32_16x16x32: the S^T layout above is
//     exactly the B-operand layout of P^T for 32 keys (two blocks), and V^T
//     comes from the transposed LDS copy with one 8-byte read per block.  P
//     is fp16 for fp16 inputs; for bf16 inputs it is split into bf16 hi + lo
//     parts (two products) so the weights keep ~16 bits.
//  5. out = O / sum, written as fp32 with 16-byte stores.
// No ksize^2-wide tensor ever leaves the chip.
#include "na2d.h"
#include "na2d_launch.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kD = 32;        // head dim handled here
constexpr int kWaves = 4;     // waves per workgroup, stacked vertically
constexpr int kThreads = 64 * kWaves;

template <typename T> struct Frag;
template <> struct Frag<_Float16> { typedef half8 type; };
template <> struct Frag<__bf16> { typedef bf16x8 type; };

__device__ inline floatx4 mfma16x16x32(const half8 &a, const half8 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Start of the window of ks pixels around i on an axis of length L.
__device__ inline int window_start(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
}

struct Args {
    const void *q, *k, *v;
    const float *rpb;
    float *out;
    int heads, H, W, ks;
    int tiles_x, tiles_y;  // tiles per map
    unsigned ntiles;       // maps * tiles_y * tiles_x
    int lr;                // halo rows held in LDS
    int ds;                // LDS stride (in elements) between two d-rows of V^T
    float c;               // log2(e) / sqrt(d)
};

template <int QY, int QX, int NCB, int RPC>
struct Shape {
    static constexpr int TY = QY * kWaves;          // tile rows
    static constexpr int TX = QX;                   // tile cols
    static constexpr int NC = 16 * NCB;             // halo cols held in LDS
    static constexpr int BPC = RPC * NCB;           // key blocks per chunk
    static_assert(QY * QX == 16, "a wave owns 16 queries");
    static_assert(BPC % 2 == 0, "P.V consumes key blocks in pairs");
};

// Rows of candidate keys per wave: QY + ks - 1 rounded up to whole chunks.
__host__ __device__ inline int wave_rows(int QY, int RPC, int ks)
{
    const int n = QY + ks - 1;
    return (n + RPC - 1) / RPC * RPC;
}

template <typename T, int QY, int QX, int NCB, int RPC>
__global__ __launch_bounds__(kThreads) void na2d_mfma_kernel(Args a)
{
    using S = Shape<QY, QX, NCB, RPC>;
    using FragT = typename Frag<T>::type;
    extern __shared__ __align__(16) unsigned char smem[];

    const int ks = a.ks, H = a.H, W = a.W;
    const int lr = a.lr, ds = a.ds;
    const int nr = wave_rows(QY, RPC, ks);
    const int tw = 2 * ks;  // bias table row width (2k-1 entries + one -inf column)

    uint4 *ks_lds = reinterpret_cast<uint4 *>(smem);                          // [lr][NC][4]
    T *vt_lds = reinterpret_cast<T *>(smem + (size_t)lr * S::NC * kD * sizeof(T));  // [kD][ds]
    float *b_lds = reinterpret_cast<float *>(smem + (size_t)lr * S::NC * kD * sizeof(T) +
                                             (size_t)kD * ds * sizeof(T));    // [tw][tw]

    // ---- which tile: consecutive tiles of a map go to the same XCD (the 8
    // XCDs receive workgroups round-robin and each has its own L2, which then
    // serves the halo overlap between neighbouring tiles).
    unsigned tile;
    {
        const unsigned n = a.ntiles, bid = blockIdx.x;
        const unsigned xcd = bid & 7u, slot = bid >> 3;
        const unsigned per = n >> 3, rem = n & 7u;
        tile = xcd * per + (xcd < rem ? xcd : rem) + slot;
    }
    const unsigned tiles_per_map = (unsigned)a.tiles_x * a.tiles_y;
    const unsigned map = tile / tiles_per_map;
    const unsigned tr = tile - map * tiles_per_map;
    const int ty = (int)(tr / a.tiles_x), tx = (int)(tr % a.tiles_x);
    const int h = (int)(map % (unsigned)a.heads);
    const int64_t map_base = (int64_t)map * H * W;  // first pixel of this (b, h) map

    const int y0 = ty * S::TY, x0 = tx * S::TX;
    // halo rows [hy0, hy0 + lr): every window of the tile's rows lies in
    // [hy0, hy0 + min(TY + ks - 1, H)); rows at or beyond H are zero-filled.
    const int hr = min(S::TY + ks - 1, H);
    const int hy0 = min(window_start(y0, ks, H), H - hr);
    // halo cols [cx, cx + NC): covers the windows of columns x0 .. x0 + QX - 1
    const int cx = W >= S::NC ? min(window_start(x0, ks, W), W - S::NC) : 0;

    const int tid = threadIdx.x;
    // ---- stage K: 16-byte d-slices, slot swizzled by column
    {
        const uint4 *kg = reinterpret_cast<const uint4 *>(a.k);
        const int units = lr * S::NC * 4;
        for (int u = tid; u < units; u += kThreads) {
            const int r = u / (S::NC * 4), rem = u - r * (S::NC * 4);
            const int j = rem >> 2, s = rem & 3;
            const int gy = hy0 + r, gx = cx + j;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (gy < H && gx < W) val = kg[((map_base + (int64_t)gy * W + gx) * kD) / 8 + s];
            ks_lds[(r * S::NC + j) * 4 + (s ^ ((j >> 2) & 3))] = val;
        }
    }
    // ---- stage V transposed: a thread takes one d-slice of 4 consecutive columns
    {
        const uint4 *vg = reinterpret_cast<const uint4 *>(a.v);
        const int units = lr * S::NC;  // lr rows * NC/4 column groups * 4 slices
        for (int u = tid; u < units; u += kThreads) {
            const int r = u / S::NC, rem = u - r * S::NC;
            const int jg = rem >> 2, s = rem & 3;
            const int gy = hy0 + r;
            uint4 px[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gx = cx + 4 * jg + i;
                px[i] = make_uint4(0, 0, 0, 0);
                if (gy < H && gx < W) px[i] = vg[((map_base + (int64_t)gy * W + gx) * kD) / 8 + s];
            }
            const unsigned short *e0 = reinterpret_cast<const unsigned short *>(&px[0]);
            const unsigned short *e1 = reinterpret_cast<const unsigned short *>(&px[1]);
            const unsigned short *e2 = reinterpret_cast<const unsigned short *>(&px[2]);
            const unsigned short *e3 = reinterpret_cast<const unsigned short *>(&px[3]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint2 w;
                w.x = (unsigned)e0[e] | ((unsigned)e1[e] << 16);
                w.y = (unsigned)e2[e] | ((unsigned)e3[e] << 16);
                *reinterpret_cast<uint2 *>(vt_lds + (size_t)(8 * s + e) * ds + r * S::NC + 4 * jg) = w;
            }
        }
    }
    // ---- bias table of this head, times c; last row and last column -inf
    {
        const int nb = 2 * ks - 1;
        const float *rb = a.rpb ? a.rpb + (int64_t)h * nb * nb : nullptr;
        for (int u = tid; u < tw * tw; u += kThreads) {
            const int r = u / tw, cc = u - r * tw;
            float val = -__builtin_inff();
            if (r < nb && cc < nb) val = rb ? rb[r * nb + cc] * a.c : 0.f;
            b_lds[u] = val;
        }
    }
    __syncthreads();

    // ---- per-wave work
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, qi = lane & 15;
    int y = y0 + QY * w + qi / QX;
    int x = x0 + qi % QX;
    const bool store_ok = y < H && x < W;
    y = min(y, H - 1);
    x = min(x, W - 1);
    const int sy = window_start(y, ks, H), sx = window_start(x, ks, W);
    const int y1 = min(y0 + QY * w, H - 1);
    const int ry = max(hy0, min(window_start(y1, ks, H), hy0 + hr - nr));  // wave's first key row
    const int rrel = ry - hy0;
    const int64_t qoff = map_base + (int64_t)y * W + x;

    const FragT qf = *reinterpret_cast<const FragT *>(static_cast<const T *>(a.q) + qoff * kD + 8 * g);

    // bias column (per lane, per held key column) or the -inf column when the
    // key column is outside this query's window
    int coloff[NCB][4];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = cx + 16 * cb + 4 * g + j;
            coloff[cb][j] = (unsigned)(col - sx) < (unsigned)ks ? col - x + ks - 1 : 2 * ks - 1;
        }

    float m = -__builtin_inff(), lsum = 0.f;
    floatx4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int kslot = g ^ ((qi >> 2) & 3);  // swizzled d-slice this lane reads from K

    for (int c0 = 0; c0 < nr; c0 += RPC) {
        float sc[RPC][NCB][4];
        // logits S^T for this chunk's blocks
#pragma unroll
        for (int rr = 0; rr < RPC; ++rr) {
            const int i = c0 + rr;
            const int krow = ry + i;
            const int rowb = (unsigned)(krow - sy) < (unsigned)ks ? (krow - y + ks - 1) * tw
                                                                   : (2 * ks - 1) * tw;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const uint4 kv = ks_lds[((rrel + i) * S::NC + 16 * cb + qi) * 4 + kslot];
                const FragT kf = *reinterpret_cast<const FragT *>(&kv);
                const floatx4 acc = mfma16x16x32(kf, qf, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sc[rr][cb][j] = fmaf(acc[j], a.c, b_lds[rowb + coloff[cb][j]]);
            }
        }
        // running max over the chunk and the 4 lanes that hold this query
        float mc = -__builtin_inff();
#pragma unroll
        for (int rr = 0; rr < RPC; ++rr)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) mc = fmaxf(mc, sc[rr][cb][j]);
        mc = fmaxf(mc, __shfl_xor(mc, 16));
        mc = fmaxf(mc, __shfl_xor(mc, 32));
        const float mnew = fmaxf(m, mc);
        const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
        const float corr = __builtin_amdgcn_exp2f(m - muse);
        m = mnew;
        lsum *= corr;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[dh][j] *= corr;

        // weights and P.V, two key blocks (32 keys) per product
#pragma unroll
        for (int bp = 0; bp < S::BPC; bp += 2) {
            const int rA = bp / NCB, cbA = bp % NCB;
            const int rB = (bp + 1) / NCB, cbB = (bp + 1) % NCB;
            float p[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[j] = __builtin_amdgcn_exp2f(sc[rA][cbA][j] - muse);
                p[4 + j] = __builtin_amdgcn_exp2f(sc[rB][cbB][j] - muse);
            }
            FragT vf[2];
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                const T *base = vt_lds + (size_t)(16 * dh + qi) * ds + 4 * g;
                const uint2 va = *reinterpret_cast<const uint2 *>(base + (rrel + c0 + rA) * S::NC + 16 * cbA);
                const uint2 vb = *reinterpret_cast<const uint2 *>(base + (rrel + c0 + rB) * S::NC + 16 * cbB);
                uint4 vv = make_uint4(va.x, va.y, vb.x, vb.y);
                vf[dh] = *reinterpret_cast<const FragT *>(&vv);
            }
            if constexpr (sizeof(T) == 2 && __is_same(T, _Float16)) {
                half8 pf;
#pragma unroll
                for (int j = 0; j < 8; ++j) pf[j] = static_cast<_Float16>(p[j]);
#pragma unroll
                for (int j = 0; j < 8; ++j) lsum += static_cast<float>(pf[j]);
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
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (store_ok) {
        const float inv = 1.f / lsum;
        float *dst = a.out + qoff * kD + 4 * g;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)
            *reinterpret_cast<float4 *>(dst + 16 * dh) =
                make_float4(o[dh][0] * inv, o[dh][1] * inv, o[dh][2] * inv, o[dh][3] * inv);
    }
}

template <typename T, int QY, int QX, int NCB, int RPC>
hipError_t launch_cfg(const Problem &p, hipStream_t stream)
{
    using S = Shape<QY, QX, NCB, RPC>;
    Args a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
    a.heads = p.heads;
    a.H = p.H;
    a.W = p.W;
    a.ks = p.ksize;
    a.tiles_x = (p.W + S::TX - 1) / S::TX;
    a.tiles_y = (p.H + S::TY - 1) / S::TY;
    const uint64_t ntiles = (uint64_t)p.B * p.heads * a.tiles_x * a.tiles_y;
    if (ntiles == 0 || ntiles > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.ntiles = (unsigned)ntiles;
    const int nr = wave_rows(QY, RPC, p.ksize);
    a.lr = max(S::TY + p.ksize - 1, nr);
    // V^T row stride in elements: lr * NC, padded so that the 16 d-rows read
    // by one 16-lane group start in different LDS banks (stride = 2 mod 32 dwords)
    int dsw = a.lr * S::NC / 2;
    dsw += (2 - dsw % 32 + 32) % 32;
    a.ds = 2 * dsw;
    a.c = 1.4426950408889634f / sqrtf((float)kD);
    const size_t lds = (size_t)a.lr * S::NC * kD * sizeof(T) + (size_t)kD * a.ds * sizeof(T) +
                       (size_t)(2 * p.ksize) * (2 * p.ksize) * sizeof(float);
    auto kern = na2d_mfma_kernel<T, QY, QX, NCB, RPC>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(a.ntiles), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const Problem &p, hipStream_t stream)
{
    const int ks = p.ksize;
    if (ks == 7) return launch_cfg<T, 2, 8, 1, 8>(p, stream);
    if (ks <= 9) return launch_cfg<T, 2, 8, 1, 2>(p, stream);
    if (ks <= 13) return launch_cfg<T, 4, 4, 1, 8>(p, stream);
    return launch_cfg<T, 2, 8, 2, 2>(p, stream);
}

}  // namespace

hipError_t launch_mfma(const Problem &p, hipStream_t stream)
{
    if (p.d != kD || p.ksize < 3 || p.ksize > NA2D_MFMA_MAX_KSIZE) return hipErrorInvalidValue;
    if (p.dtype == NA2D_F16) return launch_typed<_Float16>(p, stream);
    if (p.dtype == NA2D_BF16) return launch_typed<__bf16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace na2d
