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

// Entry i (row-major offset from entry (0, 0)) of a padded LDS bias table
// (stage_padded_bias), read whether or not the caller will use it: the
// empty asm keeps the read out of a branch on the caller's mask, so the
// reads of a block issue together.
__device__ inline float padded_at(const float *t, int i)
{
    float b = t[i];
    asm volatile("" : "+v"(b));
    return b;
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
    const float *lse_in;  // the forward's per-query log-sum-exp (natural log), or null
    float *dq, *dk, *dv, *drpb;
    float2 *ws;
    float *part;  // per-tile bias-gradient tables, (2k-1)^2 floats each
    int B, heads, H, W, ks;
    unsigned red_jobs;  // bias-table reduction jobs (see reduce_bias_tables)
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
// The head's (2k-1)^2 bias table times log2(e)/sqrt(d), in LDS with one
// zero row above and below and pl / pr zero columns left / right, row stride
// 2k - 1 + pl + pr. Every entry a pass reads, masked keys included, then lies
// inside it, so the reads need no clamp: over all windows up to 25 and all
// map sizes, the query pass reads rows 0 .. 2k-2 and columns -6 .. 2k+14,
// and the key pass rows -1 .. 2k-1 and columns -22 .. 2k+5. Returns entry
// (0, 0).
constexpr int kQPadL = 8, kQPadR = 24, kKvPadL = 24, kKvPadR = 8;

__host__ __device__ constexpr int padded_floats(int ks, int pl, int pr)
{
    return (2 * ks + 1) * (2 * ks - 1 + pl + pr);
}

__device__ inline const float *stage_padded_bias(const BArgs &a, int h, float *t, int pl, int pr)
{
    const int nb = 2 * a.ks - 1, rs = nb + pl + pr;
    for (int e = threadIdx.x; e < (nb + 2) * rs; e += kBT) {
        const int row = e / rs, i = row - 1, j = e - row * rs - pl;
        const bool in = a.rpb && (unsigned)i < (unsigned)nb && (unsigned)j < (unsigned)nb;
        t[e] = in ? a.rpb[(int64_t)h * nb * nb + i * nb + j] * a.c : 0.f;
    }
    return t + rs + pl;
}

// slice g of the 16-bit row at (y, x) (lane (g, i) of a block takes x = x0 + i),
// zeros past the map
__device__ inline u32x4 load_slice(__amdgpu_buffer_rsrc_t r, int y, int x, int W, int g)
{
    return __builtin_amdgcn_raw_buffer_load_b128(
        r, x < W ? (unsigned)(y * W + x) * 64u + 16u * (unsigned)g : kOutOfRange, 0, 0);
}

// Walks the 16-wide column blocks of rows y0..y1 (nblk a row from column x0)
// one ahead: (ny, nxb) is the next block; past the last it stays on the last
// row (a spare in-range load).
struct BlockWalk {
    int ny, nxb, b;
    const int y1, x0, nblk;
    __device__ BlockWalk(int y0_, int y1_, int x0_, int nblk_)
        : ny(y0_), nxb(x0_), b(0), y1(y1_), x0(x0_), nblk(nblk_) {}
    __device__ void advance()
    {
        if (++b == nblk) {
            b = 0;
            ny = min(ny + 1, y1);
        }
        nxb = x0 + 16 * b;
    }
};

// Runs body(data, y, xb) over the blocks of `bw` in order, each block's data
// (load(y, xb)) loaded one block ahead of its use into one of two register
// sets taken in turn, so no copy waits on a load in flight.  Past the last
// block the walk stays in range, so the spare loads are harmless.
template <typename Load, typename Body>
__device__ inline void pipelined_walk(BlockWalk bw, int nblocks, Load load, Body body)
{
    int ya = bw.ny, xa = bw.nxb;
    auto sa = load(ya, xa);
    bw.advance();
    for (int j = 0; j + 1 < nblocks; j += 2) {
        const int yb = bw.ny, xb = bw.nxb;
        const auto sb = load(yb, xb);
        bw.advance();
        body(sa, ya, xa);
        ya = bw.ny;
        xa = bw.nxb;
        sa = load(ya, xa);
        bw.advance();
        body(sb, yb, xb);
    }
    if (nblocks & 1) body(sa, ya, xa);
}

// The per-block bias gradient.  Lane (g, c) holds dS of query c (row c >> 3,
// column c & 7 of the wave's 2 x 8 queries) against keys 4g..4g+3 of the
// block, and the bias entry of a pair depends on (key row - query row,
// key column - query column): within a query row the entries are the
// diagonals of the 8 x 16 (query, key) block, which several lanes share.  The
// block is staged in LDS and each of 2 x 23 lanes sums one diagonal, so one
// conflict-free LDS atomic per block adds it to the workgroup's table.
// dy0 = key row - first query row, dx0 = first key column - first query column.
constexpr int kDsRow = 16 + 4;              // a query's 16 keys (+ padding)
constexpr int kDsRows = 16;                 // 2 x 8 queries
constexpr int kDiag = 23;                   // key - query column: -7..15
constexpr int kRedRows = 32;                // tiles per workgroup of the bias reduction

__device__ inline void add_bias_grad(const floatx4 &db, float *buf, float *dbias, int lane, int g,
                                     int c, int dy0, int dx0, int ks, float scale)
{
    *reinterpret_cast<floatx4 *>(buf + c * kDsRow + 4 * g) = db;
    if (lane < 2 * kDiag) {
        const int hq = lane >= kDiag, dl = lane - kDiag * hq - 7;  // dl = key col - query col in the block
        float sum = 0.f;
#pragma unroll
        for (int c7 = 0; c7 < 8; ++c7) {
            const int kc = dl + c7;
            float v = buf[(8 * hq + c7) * kDsRow + min(max(kc, 0), 15)];
            asm volatile("" : "+v"(v));  // read on every lane, no branch
            sum += (unsigned)kc < 16u ? v : 0.f;
        }
        const int nb = 2 * ks - 1;
        const int row = dy0 - hq + ks - 1, col = dx0 + dl + ks - 1;
        if (sum != 0.f && (unsigned)row < (unsigned)nb && (unsigned)col < (unsigned)nb)
            atomicAdd(&dbias[row * nb + col], sum * scale);
    }
}

// Write one fp32 gradient of a wave's 16 positions (2 rows of 8, 32 floats
// each). In the MFMA fragments, lane (g, c) holds dims 16 dh + 4 g .. + 3 of
// position c. The values pass through a 1 KB LDS area of the wave, one row
// of 8 positions per round, so that each store instruction writes 8 whole
// 128-byte rows instead of half of 16. Chunk k of the round's position j sits
// at 8 j + (k ^ j), so any 8 consecutive lanes reach 8 different bank groups.
// Lanes of the wave trade data through the area, hence the code-motion
// fences. The stores are non-temporal: the gradients are not read again.
// Every lane of the wave must take part; positions outside the map are not
// stored.
__device__ inline void store_rows(float *map, int y0, int x0, int H, int W, const floatx4 (&v)[2],
                                  float *stage, int lane)
{
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        __builtin_amdgcn_wave_barrier();
        if ((c >> 3) == r) {
            const int j = c & 7;
#pragma unroll
            for (int dh = 0; dh < 2; ++dh)
                *reinterpret_cast<floatx4 *>(stage + 4 * (8 * j + ((4 * dh + g) ^ j))) = v[dh];
        }
        __builtin_amdgcn_wave_barrier();
        const int j = lane >> 3, k = lane & 7;
        const floatx4 x = *reinterpret_cast<const floatx4 *>(stage + 4 * (8 * j + (k ^ j)));
        const int y = y0 + r, xx = x0 + j;
        if (y < H && xx < W)
            __builtin_nontemporal_store(x, reinterpret_cast<floatx4 *>(map + ((int64_t)y * W + xx) * 32 + 4 * k));
    }
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Query pass: softmax statistics, g . o, dq and the bias gradient of 16 own
// queries per wave, from the key blocks that their windows touch.  Writes the
// per-query (log2-sum-exp, g . o) pair the key pass reads.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_q_mfma_kernel(BArgs a)
{
    using FragT = typename Frag<T>::type;
    __shared__ __align__(16) unsigned char kbuf[kBW][16 * 64];    // streamed k block [pos][d], 16-bit
    __shared__ __align__(16) float dsbuf[kBW][kDsRows * kDsRow];  // a block's dS by (query, key)
    extern __shared__ float bias_lds[];  // the padded bias table, then the workgroup's bias gradient
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= a.ntiles) return;
    const Patch P = patch_of(a, tile);
    const int H = a.H, W = a.W, ks = a.ks, nb = 2 * ks - 1, rs = nb + kQPadL + kQPadR;
    const float *raw = stage_padded_bias(a, P.h, bias_lds, kQPadL, kQPadR);
    float *dbias = bias_lds + padded_floats(ks, kQPadL, kQPadR);
    if (a.drpb) {
        for (int e = threadIdx.x; e < nb * nb; e += kBT) dbias[e] = 0.f;
        // the key pass, which runs after this kernel, adds the tables into drpb
        if (tile == 0)
            for (int e = threadIdx.x; e < a.heads * nb * nb; e += kBT) a.drpb[e] = 0.f;
    }
    __syncthreads();

    // the wave index is uniform: in a scalar register, loop bounds built on it stay scalar
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int qy1 = P.y0 + 2 * wave;  // the wave's query rows qy1, qy1 + 1
    if (qy1 < H) {
        const int qy = min(qy1 + (c >> 3), H - 1), qx = min(P.x0 + (c & 7), W - 1);
        const bool own_valid = qy1 + (c >> 3) < H && P.x0 + (c & 7) < W;
        const int sy = wstart(qy, ks, H), sx = wstart(qx, ks, W);
        const unsigned map_bytes = (unsigned)H * W * 64u;
        const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, P.base, 64, map_bytes);
        const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, P.base, 64, map_bytes);
        const int64_t qi = P.base + (int64_t)qy * W + qx;
        // the wave's own queries as B operands: lane (g, c) holds slice g of query c
        const FragT qf = __builtin_bit_cast(
            FragT, *reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.q) + qi * 32 + 8 * g));
        FragT gh, gl;
        float go = 0.f;  // this lane's share of g . o
        {
            const float *gp = a.dout + qi * 32 + 8 * g, *op = a.out + qi * 32 + 8 * g;
            const floatx4 g0 = *reinterpret_cast<const floatx4 *>(gp);
            const floatx4 g1 = *reinterpret_cast<const floatx4 *>(gp + 4);
            const floatx4 o0 = *reinterpret_cast<const floatx4 *>(op);
            const floatx4 o1 = *reinterpret_cast<const floatx4 *>(op + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                T h, l;
                split<T>(g0[e], h, l);
                gh[e] = h;
                gl[e] = l;
                split<T>(g1[e], h, l);
                gh[4 + e] = h;
                gl[4 + e] = l;
                go = fmaf(g0[e], o0[e], go);
                go = fmaf(g1[e], o1[e], go);
            }
        }
        const float dd = quad_sum(go);

        // keys the wave's windows touch: rows kylo..kyhi, 16-wide column blocks from kxlo
        const int kylo = wstart(qy1, ks, H), kyhi = wstart(min(qy1 + 1, H - 1), ks, H) + ks - 1;
        const int kxlo = wstart(P.x0, ks, W), kxhi = wstart(min(P.x0 + 7, W - 1), ks, W) + ks - 1;
        const int nblk = (kxhi - kxlo + 16) >> 4;
        const int nblocks = (kyhi - kylo + 1) * nblk;

        // the softmax statistics: the forward's log-sum-exp when given, else
        // pass 1 below recomputes them
        float lse = 0.f;
        if (a.lse_in) {
            if (own_valid) lse = a.lse_in[qi] * 1.4426950408889634f;  // to log2 units
        } else {
            // pass 1: online max and sum of the log2-scaled logits, per lane over
            // its keys 4g..4g+3 of each block, then over the four lane groups.
            // Blocks run row by row.
            float m = -1e30f, l = 0.f;
            pipelined_walk(
                BlockWalk(kylo, kyhi, kxlo, nblk), nblocks,
                [&](int ky, int kxb) { return load_slice(rk, ky, kxb + c, W, g); },
                [&](const u32x4 &kv, int ky, int kxb) {
                    const FragT ka = __builtin_bit_cast(FragT, kv);
                    const bool rowin = own_valid && (unsigned)(ky - sy) < (unsigned)ks;
                    const int brow = (ky - qy + ks - 1) * rs;
                    const floatx4 s = mfma16x16x32(ka, qf, floatx4{0, 0, 0, 0});
                    float t[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kx = kxb + 4 * g + r;
                        const bool in = rowin && (unsigned)(kx - sx) < (unsigned)ks;
                        const float b = padded_at(raw, brow + kx - qx + ks - 1);
                        t[r] = in ? s[r] * a.c + b : -INFINITY;
                    }
                    const float mn = fmaxf(fmaxf(m, fmaxf(t[0], t[1])), fmaxf(t[2], t[3]));
                    l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(t[0] - mn) +
                        __builtin_amdgcn_exp2f(t[1] - mn) + __builtin_amdgcn_exp2f(t[2] - mn) +
                        __builtin_amdgcn_exp2f(t[3] - mn);
                    m = mn;
                });
            const float mq = quad_max(m);
            const float lq = quad_sum(l * __builtin_amdgcn_exp2f(m - mq));
            lse = own_valid ? mq + __builtin_amdgcn_logf(lq) : 0.f;
        }

        // pass 2: P, dS, dq^T += k^T dS^T and the bias gradient
        floatx4 dq[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
        floatx4 dql[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
        unsigned char *kb = kbuf[wave];
        const unsigned tr_off0 = tr_read_off(g, c, 0), tr_off1 = tr_read_off(g, c, 1);
        const unsigned st_off = stage_off(g, c);
        struct KV {
            u32x4 k, v;
        };
        pipelined_walk(
            BlockWalk(kylo, kyhi, kxlo, nblk), nblocks,
            [&](int ky, int kxb) {
                return KV{load_slice(rk, ky, kxb + c, W, g), load_slice(rv, ky, kxb + c, W, g)};
            },
            [&](const KV &blk, int ky, int kxb) {
                const u32x4 kv = blk.k, vv = blk.v;
                const bool rowin = own_valid && (unsigned)(ky - sy) < (unsigned)ks;
                const int brow = (ky - qy + ks - 1) * rs;
                *reinterpret_cast<u32x4 *>(kb + st_off) = kv;
                const FragT ka = __builtin_bit_cast(FragT, kv), va = __builtin_bit_cast(FragT, vv);
                const floatx4 s = mfma16x16x32(ka, qf, floatx4{0, 0, 0, 0});
                const floatx4 gvh = mfma16x16x32(va, gh, floatx4{0, 0, 0, 0});
                const floatx4 gvl = mfma16x16x32(va, gl, floatx4{0, 0, 0, 0});
                const floatx4 gv = gvh + gvl * LoScale<T>::down;
                v4i16 sh, sl;
                floatx4 db;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kx = kxb + 4 * g + r;
                    const bool in = rowin && (unsigned)(kx - sx) < (unsigned)ks;
                    const float b = padded_at(raw, brow + kx - qx + ks - 1);
                    const float e = __builtin_amdgcn_exp2f(s[r] * a.c + b - lse);
                    const float p = in ? e : 0.f;
                    const float ds = p * (gv[r] - dd);
                    db[r] = ds;
                    T h, lo;
                    split<T>(ds, h, lo);
                    sh[r] = bits(h);
                    sl[r] = bits(lo);
                }
                if (a.drpb) add_bias_grad(db, dsbuf[wave], dbias, lane, g, c, ky - qy1, kxb - P.x0, ks, a.scale);
#pragma unroll
                for (int dh = 0; dh < 2; ++dh) {
                    const v4i16 kt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(kb + (dh ? tr_off1 : tr_off0)));
                    dq[dh] = mfma16x16x16(kt, sh, dq[dh], T{});
                    dql[dh] = mfma16x16x16(kt, sl, dql[dh], T{});
                }
            });
        if (own_valid && g == 0) a.ws[qi] = make_float2(lse, dd);
        // the wave's k block area is free once its last block is consumed
        const floatx4 dqs[2] = {(dq[0] + dql[0] * LoScale<T>::down) * a.scale,
                                (dq[1] + dql[1] * LoScale<T>::down) * a.scale};
        store_rows(a.dq + P.base * 32, qy1, P.x0, H, W, dqs, reinterpret_cast<float *>(kbuf[wave]), lane);
    }
    if (a.drpb) {  // the tile's table, summed over tiles by reduce_bias_tables
        __syncthreads();
        float *dst = a.part + (int64_t)tile * nb * nb;
        for (int e = threadIdx.x; e < nb * nb; e += kBT) dst[e] = dbias[e];
    }
}

// drpb[h] += the tables of tiles [chunk * kRedRows, ...) of head h, for
// job = chunk * heads + h (tiles are numbered map-major, map = b * heads + h).
// Run by the first workgroups of the key pass, after the query pass wrote the
// tables and cleared drpb.  The 32 reads of an entry are issued together (one
// memory latency before those workgroups start on their own tiles).
__device__ inline void reduce_bias_tables(const BArgs &a, unsigned job)
{
    const int nbb = (2 * a.ks - 1) * (2 * a.ks - 1);
    const int h = job % a.heads, chunk = job / a.heads;
    const int rows = a.B * a.tiles_per_map;
    const int r0 = chunk * kRedRows;
    for (int e = threadIdx.x; e < nbb; e += kBT) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kRedRows; ++i) {
            const int r = min(r0 + i, rows - 1);  // a row past the end is read but not added
            const int b = r / a.tiles_per_map, t = r - b * a.tiles_per_map;
            const float v = a.part[((int64_t)(b * a.heads + h) * a.tiles_per_map + t) * nbb + e];
            acc += r0 + i < rows ? v : 0.f;
        }
        unsafeAtomicAdd(&a.drpb[(int64_t)h * nbb + e], acc);
    }
}

// ---------------------------------------------------------------------------
// Key pass: dk, dv of 16 own keys per wave from every query holding them.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_kv_mfma_kernel(BArgs a)
{
    using FragT = typename Frag<T>::type;
    __shared__ __align__(16) unsigned char qbuf[kBW][16 * 64];    // streamed q block [pos][d], 16-bit
    __shared__ __align__(16) unsigned char gbuf[kBW][2][16 * 64]; // streamed g block, hi and lo
    extern __shared__ float bias_lds[];                           // the padded bias table
    if (a.drpb && blockIdx.x < a.red_jobs) reduce_bias_tables(a, blockIdx.x);
    const unsigned tile = xcd_tile(blockIdx.x, gridDim.x);
    if (tile >= a.ntiles) return;
    const Patch P = patch_of(a, tile);
    // the wave index is uniform: in a scalar register, loop bounds built on it stay scalar
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c = lane & 15;
    const int H = a.H, W = a.W, ks = a.ks, rs = 2 * ks - 1 + kKvPadL + kKvPadR;
    const int ky1 = P.y0 + 2 * wave;                 // the wave's key rows ky1, ky1 + 1
    // this lane's key (clamped into the map) and its k and v fragments, issued
    // before the bias table is staged so that the two latencies overlap
    const int ky = min(ky1 + (c >> 3), H - 1), kx = min(P.x0 + (c & 7), W - 1);
    const unsigned map_bytes = (unsigned)H * W * 64u;
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, P.base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, P.base, 64, map_bytes);
    const unsigned own_off = (unsigned)(ky * W + kx) * 64u + 16u * g;
    const FragT kf = __builtin_bit_cast(FragT, __builtin_amdgcn_raw_buffer_load_b128(rk, own_off, 0, 0));
    const FragT vf = __builtin_bit_cast(FragT, __builtin_amdgcn_raw_buffer_load_b128(rv, own_off, 0, 0));
    const float *raw = stage_padded_bias(a, P.h, bias_lds, kKvPadL, kKvPadR);
    __syncthreads();
    if (ky1 >= H) return;
    const bool own_valid = ky1 + (c >> 3) < H && P.x0 + (c & 7) < W;
    // the queries whose windows hold this lane's key: rows hy0 .. hy1, columns hx0 .. hx1
    int hy0, hy1, hx0, hx1;
    holders(ky, ks, H, hy0, hy1);
    holders(kx, ks, W, hx0, hx1);
    const unsigned hyn = (unsigned)(hy1 - hy0), hxn = (unsigned)(hx1 - hx0);
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, P.base, 64, map_bytes);
    const __amdgpu_buffer_rsrc_t rg = map_rsrc(a.dout, P.base, 128, (unsigned)H * W * 128u);
    const __amdgpu_buffer_rsrc_t rw = map_rsrc(a.ws, P.base, 8, (unsigned)H * W * 8u);
    // (kf, vf above: the wave's own keys as B operands, lane (g, c) holding slice g of key c)

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
    const unsigned tr_off0 = tr_read_off(g, c, 0), tr_off1 = tr_read_off(g, c, 1);
    const unsigned st_off = stage_off(g, c);

    // streamed block at (y, xb): q and g rows of queries (y, xb + i), and the
    // softmax statistics of queries xb + 4 g + r (r = 0..3); zeros past the map
    struct Streamed {
        u32x4 q, g0, g1;
        unsigned w;
    };
    auto load_block = [&](int y, int xb) {
        Streamed t;
        t.q = load_slice(rq, y, xb + c, W, g);
        const unsigned goff = xb + c < W ? (unsigned)(y * W + xb + c) * 128u + 32u * g : kOutOfRange;
        t.g0 = __builtin_amdgcn_raw_buffer_load_b128(rg, goff, 0, 0);
        t.g1 = __builtin_amdgcn_raw_buffer_load_b128(rg, goff + 16u, 0, 0);
        // lane (g, c < 8) fetches word c & 7 of queries xb + 4 g .. + 3 (their
        // log-sum-exp and g . o pairs); process() broadcasts them across the row
        const unsigned woff = xb + 4 * g < W ? (unsigned)(y * W + xb + 4 * g) * 8u + 4u * (c & 7) : kOutOfRange;
        t.w = __builtin_amdgcn_raw_buffer_load_b32(rw, woff, 0, 0);
        return t;
    };
    auto process = [&](const Streamed &cur, int y, int xb) {
        {
            const u32x4 qv = cur.q, g0 = cur.g0, g1 = cur.g1;
            // q as A operand (the block's positions as rows), its copy for q^T
            *reinterpret_cast<u32x4 *>(qb + st_off) = qv;
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
            *reinterpret_cast<FragT *>(gbh + st_off) = gh;
            *reinterpret_cast<FragT *>(gbl + st_off) = gl;
            const FragT qa = __builtin_bit_cast(FragT, qv);
            floatx4 s = mfma16x16x32(qa, kf, floatx4{0, 0, 0, 0});
            const floatx4 gvh = mfma16x16x32(gh, vf, floatx4{0, 0, 0, 0});
            const floatx4 gvl = mfma16x16x32(gl, vf, floatx4{0, 0, 0, 0});
            const floatx4 gv = gvh + gvl * LoScale<T>::down;
            // row_newbcast:n (DPP control 0x150 + n): every lane of a 16-lane row takes lane n's word
            const int wv = (int)cur.w;
            const float lse[4] = {__int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x150, 0xf, 0xf, false)),
                                  __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x152, 0xf, 0xf, false)),
                                  __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x154, 0xf, 0xf, false)),
                                  __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x156, 0xf, 0xf, false))};
            const float dd[4] = {__int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x151, 0xf, 0xf, false)),
                                 __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x153, 0xf, 0xf, false)),
                                 __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x155, 0xf, 0xf, false)),
                                 __int_as_float(__builtin_amdgcn_update_dpp(0, wv, 0x157, 0xf, 0xf, false))};
            // p and dS for queries (y, xb + 4 g + r) and key c
            v4i16 ph, pl, sh, sl;
            const bool rowin = own_valid && (unsigned)(y - hy0) <= hyn;
            const int brow = (ky - y + ks - 1) * rs + kx + ks - 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int x = xb + 4 * g + r;
                // the key lies in the window of query (y, x) exactly when the query holds it
                const bool in = rowin && (unsigned)(x - hx0) <= hxn;
                const float bias = padded_at(raw, brow - x);
                const float e = __builtin_amdgcn_exp2f(s[r] * a.c + bias - lse[r]);
                const float p = in ? e : 0.f;
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
                const unsigned to = dh ? tr_off1 : tr_off0;
                const v4i16 qt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(qb + to));
                const v4i16 gth = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(gbh + to));
                const v4i16 gtl = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(gbl + to));
                dv[dh] = mfma16x16x16(gth, ph, dv[dh], T{});
                dvl[dh] = mfma16x16x16(gth, pl, dvl[dh], T{});
                dvl[dh] = mfma16x16x16(gtl, ph, dvl[dh], T{});
                dk[dh] = mfma16x16x16(qt, sh, dk[dh], T{});
                dkl[dh] = mfma16x16x16(qt, sl, dkl[dh], T{});
            }
        }
    };
    // blocks row by row
    pipelined_walk(BlockWalk(ylo, yhi, xlo, nblk), (yhi - ylo + 1) * nblk, load_block, process);
    // the wave's q block area is free once its last block is consumed
    const floatx4 dks[2] = {(dk[0] + dkl[0] * LoScale<T>::down) * a.scale,
                            (dk[1] + dkl[1] * LoScale<T>::down) * a.scale};
    const floatx4 dvs[2] = {dv[0] + dvl[0] * LoScale<T>::down, dv[1] + dvl[1] * LoScale<T>::down};
    float *stage = reinterpret_cast<float *>(qbuf[wave]);
    store_rows(a.dk + P.base * 32, ky1, P.x0, H, W, dks, stage, lane);
    store_rows(a.dv + P.base * 32, ky1, P.x0, H, W, dvs, stage, lane);
}

}  // namespace

// Both passes on the matrix cores: the query pass (dq, the bias gradient and
// the per-query statistics), then the key pass that reads those statistics.
// The bias gradient must already be cleared.
hipError_t launch_backward_mfma(const BwdProblem &p, hipStream_t stream)
{
    BArgs a;
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
    a.part = reinterpret_cast<float *>(static_cast<char *>(p.workspace) +
                                       bwd_stats_bytes(p.B, p.heads, p.H, p.W));
    a.B = p.B;
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
    a.red_jobs = (unsigned)(((uint64_t)p.B * a.tiles_per_map + kRedRows - 1) / kRedRows * p.heads);
    const dim3 grid((unsigned)xcd_grid(tiles));
    if (a.red_jobs > grid.x) return hipErrorInvalidConfiguration;  // cannot happen: a job spans >= 32 tiles
    const int nb = 2 * p.ksize - 1;
    const size_t q_lds = (size_t)(padded_floats(p.ksize, kQPadL, kQPadR) + nb * nb) * 4;
    const size_t kv_lds = (size_t)padded_floats(p.ksize, kKvPadL, kKvPadR) * 4;
    if (p.dtype == NA2D_F16) {
        hipLaunchKernelGGL(bwd_q_mfma_kernel<_Float16>, grid, dim3(kBT), q_lds, stream, a);
        hipLaunchKernelGGL(bwd_kv_mfma_kernel<_Float16>, grid, dim3(kBT), kv_lds, stream, a);
    } else if (p.dtype == NA2D_BF16) {
        hipLaunchKernelGGL(bwd_q_mfma_kernel<__bf16>, grid, dim3(kBT), q_lds, stream, a);
        hipLaunchKernelGGL(bwd_kv_mfma_kernel<__bf16>, grid, dim3(kBT), kv_lds, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace na2d
