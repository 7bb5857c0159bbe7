// na3d_mfma.hip -- NA3D forward (fp16/bf16 inputs, d = 32) on the gfx950
// matrix cores.
//
// Neighborhood Attention over a D x H x W volume (the NA definition of
// "Neighborhood Attention Transformer", CSDN translation, section 3.1,
// Eq. 2-4, applied per axis; NATTEN's 3D form, qiita article, section
// "NATTEN"): per query the kd x kh x kw window clamped into the volume on
// every axis, logits (q.k + B[dz, dy, dx]) / sqrt(d), softmax over the
// window, weighted sum of the values.
//
// How.  A workgroup owns an 8 x 8 patch of queries at one depth z; each of
// its four waves owns a QY x QX = 16-query subtile.  All of a wave's queries
// share z and so the depth slices of their windows; the wave walks the
// 16-key blocks (BR key rows x 16/BR consecutive columns) that cover the
// union of their windows, straight from L2, two blocks at a time.  Three
// shapes -- 2 x 8 queries against 1 x 16 key blocks, 4 x 4 queries against
// 2 x 8 or 4 x 4 blocks -- and each launch takes the one with the fewest
// blocks per slice for its window (at k = 5: 4 instead of 6; at k = 21: 36
// instead of 44).  Per pair of blocks:
//  - S^T = K_block Q^T, one v_mfma_f32_16x16x32 per block: lane (g, c)
//    holds query c against keys 4g..4g+3 of the block (one key row);
//  - the bias (times log2(e)/sqrt(d)) comes from an LDS copy of the head's
//    table; keys outside a query's window are masked to -inf;
//  - online softmax over the pair: one max over the four lanes of a query
//    (v_permlane16/32_swap), rescale of the running sum and output;
//  - O^T += V^T P^T as one v_mfma_f32_16x16x32 per 16 dims: the two blocks'
//    S^T layouts together are the B-operand layout of P^T for 32 keys, and
//    ds_read_b64_tr_b16 from a per-wave LDS copy of each V block gives the
//    matching A operand.  P is fp16 for fp16 inputs; for bf16 it is split
//    into bf16 hi + lo parts (two products), so the weights keep ~16 bits.
// Each pair's K and V are loaded one pair ahead into one of two register
// sets taken in turn.  out = O / sum in fp32.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_mfma_util.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

constexpr int kW3 = 4;          // waves per workgroup
constexpr int kT3 = 64 * kW3;   // threads per workgroup
// the largest bias table: a 3D window of NA3D_MFMA_MAX_KSIZE per axis, or a 2D
// one of NA2D_MFMA_MAX_KSIZE
constexpr int kTable3 =
    (2 * NA3D_MFMA_MAX_KSIZE - 1) * (2 * NA3D_MFMA_MAX_KSIZE - 1) * (2 * NA3D_MFMA_MAX_KSIZE - 1);
constexpr int kTable2 = (2 * NA2D_MFMA_MAX_KSIZE - 1) * (2 * NA2D_MFMA_MAX_KSIZE - 1);
constexpr int kMaxTable = kTable3 > kTable2 ? kTable3 : kTable2;
constexpr int kPad = 16;  // floats of margin before and after the bias table

struct Args3 {
    const void *q, *k, *v;
    const float *rpb;
    float *out;
    float *lse;  // per-query log-sum-exp of the logits, or null
    int heads, D, H, W, kd, kh, kw;
    int tiles_x, tiles_yx, tiles_per_map;
    unsigned ntiles;
    float c;  // log2(e) / sqrt(d)
};

__device__ inline int wstart3(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    s = s < 0 ? 0 : s;
    return s > L - ks ? L - ks : s;
}

// The 16-byte d-slice g of the 16-bit row of pixel (z, y, x) of the map;
// zeros for a pixel past the map's last row or column.
__device__ inline u32x4 load_slice3(__amdgpu_buffer_rsrc_t r, int z, int y, int x, int H, int W, int g)
{
    return __builtin_amdgcn_raw_buffer_load_b128(
        r, x < W && y < H ? (unsigned)((z * H + y) * W + x) * 64u + 16u * (unsigned)g : kOutOfRange,
        0, 0);
}

// Walks the key blocks of a wave one at a time: slices z0..zlast, block rows
// y0, y0 + BR, .. up to y1, nblk column blocks of width BC from x0; past the
// last block it stays on the last.
template <int BR, int BC>
struct Walk3 {
    int z, y, b;
    int zlast;
    const int y0, y1, x0, nblk;
    __device__ Walk3(int z0, int zl, int y0_, int y1_, int x0_, int nblk_)
        : z(z0), y(y0_), b(0), zlast(zl), y0(y0_), y1(y1_), x0(x0_), nblk(nblk_) {}
    __device__ int xb() const { return x0 + BC * b; }
    __device__ void advance()
    {
        if (++b < nblk) return;
        b = 0;
        if (y + BR <= y1) {
            y += BR;
        } else if (z < zlast) {
            ++z;
            y = y0;
        } else {
            b = nblk - 1;  // stay on the last block
        }
    }
};

struct Pos {
    int z, y, xb;
};

// QY x QX: a wave's queries; BR x BC (= 16): a key block.
template <typename T, int QY, int QX, int BR>
__global__ __launch_bounds__(kT3) void na3d_mfma_kernel(Args3 a)
{
    constexpr int BC = 16 / BR;
    static_assert(QY * QX == 16 && BR * BC == 16 && 4 % BR == 0 && 8 % QX == 0, "shape");
    using FragT = typename Frag<T>::type;
    __shared__ float table[kPad + kMaxTable + kPad];              // bias table, times c, with margins
    float *const raw = table + kPad;
    __shared__ __align__(16) unsigned char vbuf[kW3][2][16 * 64];  // a pair's V blocks [pos][d]
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= a.ntiles) return;
    const int H = a.H, W = a.W, D = a.D, kd = a.kd, kh = a.kh, kw = a.kw;
    const int nbd = 2 * kd - 1, nbh = 2 * kh - 1, nbw = 2 * kw - 1;
    const int map = tile / a.tiles_per_map;
    const int rem = tile - map * a.tiles_per_map;
    const int z = rem / a.tiles_yx;
    const int t2 = rem - z * a.tiles_yx;
    const int ty = t2 / a.tiles_x;
    const int y0 = ty * 8, x0 = (t2 - ty * a.tiles_x) * 8;
    const int h = map % a.heads;
    {
        const int n = nbd * nbh * nbw;
        const float *bias = a.rpb ? a.rpb + (int64_t)h * n : nullptr;
        for (int e = threadIdx.x; e < n; e += kT3) raw[e] = bias ? bias[e] * a.c : 0.f;
        if (threadIdx.x < 2 * kPad) table[threadIdx.x < kPad ? threadIdx.x : kPad + n + threadIdx.x - kPad] = 0.f;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    // the wave's subtile: rows qy1 .. qy1 + QY - 1, columns qx1 .. qx1 + QX - 1
    const int qy1 = y0 + QY * (wave / (8 / QX)), qx1 = x0 + QX * (wave % (8 / QX));
    if (qy1 >= H || qx1 >= W) return;
    const int qy = min(qy1 + c / QX, H - 1), qx = min(qx1 + c % QX, W - 1);
    const bool own_valid = qy1 + c / QX < H && qx1 + c % QX < W;
    const int sy = wstart3(qy, kh, H), sx = wstart3(qx, kw, W), sz = wstart3(z, kd, D);
    const int64_t base = (int64_t)map * D * H * W;
    const unsigned map_bytes = (unsigned)D * H * W * 64u;
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, base, 64, map_bytes);
    // the wave's own queries as B operands: lane (g, c) holds slice g of query c
    const FragT qf = __builtin_bit_cast(
        FragT, __builtin_amdgcn_raw_buffer_load_b128(rq, (unsigned)((z * H + qy) * W + qx) * 64u + 16u * g, 0, 0));

    // key blocks the wave's windows touch
    const int kylo = wstart3(qy1, kh, H), kyhi = wstart3(min(qy1 + QY - 1, H - 1), kh, H) + kh - 1;
    const int kxlo = wstart3(qx1, kw, W), kxhi = wstart3(min(qx1 + QX - 1, W - 1), kw, W) + kw - 1;
    const int nblk = (kxhi - kxlo + BC) / BC;
    const int nblocks = kd * ((kyhi - kylo + BR) / BR) * nblk;
    const int npairs = (nblocks + 1) >> 1;

    float m = -1e30f, l = 0.f;  // running max (shared by a query's 4 lanes) and this lane's sum
    floatx4 o[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
    unsigned char *vb0 = vbuf[wave][0], *vb1 = vbuf[wave][1];
    const unsigned tr_off0 = tr_read_off(g, c, 0), tr_off1 = tr_read_off(g, c, 1);
    const unsigned st_off = stage_off(g, c);
    const int zoff = z - (kd - 1);  // key slice minus this, times the row stride, indexes the table

    // logits of block (p.z, p.y, p.xb) for query c, keys 4g + r, in log2 units:
    // key 4g + r of the block is (row p.y + 4g / BC, column p.xb + 4g % BC + r).
    // The four bias entries are read unconditionally from a base clamped into
    // the padded table (a masked key's entry is never used), so the reads
    // need no branches.
    const int nmax = nbd * nbh * nbw;
    const int krow = 4 * g / BC, kcol = 4 * g % BC;  // this lane's keys within a block
    auto logits = [&](const floatx4 &s, const Pos &p, bool real, float *t) {
        const int ky = p.y + krow;
        const bool rowin = real && own_valid && (unsigned)(ky - sy) < (unsigned)kh;
        const int base = ((p.z - zoff) * nbh + (ky - qy + kh - 1)) * nbw + p.xb + kcol - qx + kw - 1;
        const float *bp = raw + min(max(base, -kPad), nmax + kPad - 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kx = p.xb + kcol + r;
            const bool in = rowin && (unsigned)(kx - sx) < (unsigned)kw;
            float b = bp[r];
            asm volatile("" : "+v"(b));  // keeps the read out of a branch on `in`
            t[r] = in ? s[r] * a.c + b : -INFINITY;
        }
    };
    struct Pair {
        u32x4 k0, v0, k1, v1;
    };
    Walk3<BR, BC> walk(sz, sz + kd - 1, kylo, kyhi, kxlo, nblk);
    // lane (g, c) loads slice g of key c of a block: (row + c / BC, column + c % BC)
    const int lrow = c / BC, lcol = c % BC;
    auto load_pair = [&](Pos &p0, Pos &p1) {
        Pair t;
        p0 = Pos{walk.z, walk.y, walk.xb()};
        t.k0 = load_slice3(rk, p0.z, p0.y + lrow, p0.xb + lcol, H, W, g);
        t.v0 = load_slice3(rv, p0.z, p0.y + lrow, p0.xb + lcol, H, W, g);
        walk.advance();
        p1 = Pos{walk.z, walk.y, walk.xb()};
        t.k1 = load_slice3(rk, p1.z, p1.y + lrow, p1.xb + lcol, H, W, g);
        t.v1 = load_slice3(rv, p1.z, p1.y + lrow, p1.xb + lcol, H, W, g);
        walk.advance();
        return t;
    };
    auto process = [&](const Pair &pr, const Pos &p0, const Pos &p1, int pair) {
        *reinterpret_cast<u32x4 *>(vb0 + st_off) = pr.v0;
        *reinterpret_cast<u32x4 *>(vb1 + st_off) = pr.v1;
        const floatx4 s0 = mfma16x16x32(__builtin_bit_cast(FragT, pr.k0), qf, floatx4{0, 0, 0, 0});
        const floatx4 s1 = mfma16x16x32(__builtin_bit_cast(FragT, pr.k1), qf, floatx4{0, 0, 0, 0});
        float t[8];
        logits(s0, p0, true, t);
        logits(s1, p1, 2 * pair + 1 < nblocks, t + 4);  // an odd count leaves the last pair half empty
        float mx = t[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, t[e]);
        const float mn = fmaxf(m, quad_max(mx));
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(t[e] - mn);
            ps += p[e];
        }
        l = l * alpha + ps;
        FragT ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph[e] = static_cast<T>(p[e]);
            if constexpr (!std::is_same<T, _Float16>::value) pl[e] = static_cast<T>(p[e] - static_cast<float>(ph[e]));
        }
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) {
            const unsigned to = dh ? tr_off1 : tr_off0;
            const v4i16 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb0 + to));
            const v4i16 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb1 + to));
            const v8i16 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const FragT vt = __builtin_bit_cast(FragT, av);
            o[dh] = mfma16x16x32(vt, ph, o[dh] * alpha);
            if constexpr (!std::is_same<T, _Float16>::value) o[dh] = mfma16x16x32(vt, pl, o[dh]);
        }
    };
    // pairs in two register sets taken in turn, each loaded one pair ahead
    Pos pa0, pa1;
    Pair sa = load_pair(pa0, pa1);
    for (int j = 0; j + 1 < npairs; j += 2) {
        Pos pb0, pb1;
        const Pair sb = load_pair(pb0, pb1);
        process(sa, pa0, pa1, j);
        sa = load_pair(pa0, pa1);
        process(sb, pb0, pb1, j + 1);
    }
    if (npairs & 1) process(sa, pa0, pa1, npairs - 1);

    // lane (g, c): dims 16 dh + 4 g + r of query c
    const float lq = quad_sum(l);
    const float inv = 1.f / lq;
    if (own_valid) {
        const int64_t qi = base + (int64_t)(z * H + qy) * W + qx;
        if (a.lse && g == 0) a.lse[qi] = (m + __builtin_amdgcn_logf(lq)) * 0.6931471805599453f;
        float *dst = a.out + qi * 32 + 4 * g;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh)  // non-temporal: nothing reads the output again
            __builtin_nontemporal_store(o[dh] * inv, reinterpret_cast<floatx4 *>(dst + 16 * dh));
    }
}

}  // namespace

namespace {

// shape 0: 2 x 8 queries, 1 x 16 key blocks; 1: 4 x 4 queries, 2 x 8 blocks;
// 2: 4 x 4 queries, 4 x 4 blocks
template <typename T>
void launch_shape(int shape, dim3 grid, const Args3 &a, hipStream_t stream)
{
    if (shape == 0)
        hipLaunchKernelGGL((na3d_mfma_kernel<T, 2, 8, 1>), grid, dim3(kT3), 0, stream, a);
    else if (shape == 1)
        hipLaunchKernelGGL((na3d_mfma_kernel<T, 4, 4, 2>), grid, dim3(kT3), 0, stream, a);
    else
        hipLaunchKernelGGL((na3d_mfma_kernel<T, 4, 4, 4>), grid, dim3(kT3), 0, stream, a);
}

}  // namespace

hipError_t launch_mfma_3d(const Problem &p, hipStream_t stream)
{
    if (p.d != 32 || p.mode != NA_WINDOW_NA ||
        (2 * p.kd - 1) * (2 * p.kh - 1) * (2 * p.kw - 1) > kMaxTable)
        return hipErrorInvalidValue;
    Args3 a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
    a.lse = p.lse;
    a.heads = p.heads;
    a.D = p.depth;
    a.H = p.H;
    a.W = p.W;
    a.kd = p.kd;
    a.kh = p.kh;
    a.kw = p.kw;
    a.tiles_x = (p.W + 7) / 8;
    a.tiles_yx = a.tiles_x * ((p.H + 7) / 8);
    a.tiles_per_map = a.tiles_yx * p.depth;
    a.c = 1.4426950408889634f / sqrtf(32.f);
    const uint64_t tiles = (uint64_t)p.B * p.heads * a.tiles_per_map;
    if (tiles == 0 || xcd_grid(tiles) > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.ntiles = (unsigned)tiles;
    const dim3 grid((unsigned)xcd_grid(tiles));
    // the subtile / block shape with the fewest key blocks per wave and depth
    // slice: ceil((QY + kh - 1) / BR) * ceil((QX + kw - 1) / BC)
    auto blocks = [&](int qy, int qx, int br) {
        const int bc = 16 / br;
        return ((qy + p.kh - 1 + br - 1) / br) * ((qx + p.kw - 1 + bc - 1) / bc);
    };
    const int nA = blocks(2, 8, 1), nB = blocks(4, 4, 2), nD = blocks(4, 4, 4);
    const int shape = nA <= nB && nA <= nD ? 0 : nB <= nD ? 1 : 2;
    if (p.dtype == NA2D_F16)
        launch_shape<_Float16>(shape, grid, a, stream);
    else if (p.dtype == NA2D_BF16)
        launch_shape<__bf16>(shape, grid, a, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace na2d
