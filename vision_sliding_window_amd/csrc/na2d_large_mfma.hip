// na2d_large_mfma.hip -- NA2D forward for wide windows (fp16/bf16 inputs,
// d = 32) on the gfx950 matrix cores.
//
// The operation is Neighborhood Attention ("Neighborhood Attention
// Transformer", CSDN translation, section 3.1, Eq. 2-4): per query the
// clamped ksize x ksize window, logits (q.k + B) / sqrt(d), softmax over the
// window, weighted sum of the values.
//
// How.  Persistent workgroups of four waves walk a list of query tiles:
// 4 x 16 while the union of a tile's windows fits 32 staged columns (k <= 17;
// every block row of such a tile serves all four waves), else 8 x 8. Wave w
// owns the 4 x 4 subtile (w / WX, w % WX), WX = 4 or 2 waves across. The
// union of the tile's windows -- at most 15 + ksize columns -- is cut into
// 4 x 4 key blocks; for a 4 x 4 subtile 4 x 4 blocks cover the window union
// most tightly (at ksize = 21, 36 blocks against 44 for 16-key rows).
//  1. Staging.  The tile's key blocks go through LDS one block row (four key
//     rows) at a time, double buffered: while the waves work on block row i,
//     the loads of row i + 1 (or of the next tile's first row) are in flight
//     in registers, and are written to the other buffer afterwards.  All four
//     waves read each staged block, so each key and value leaves L2 once per
//     tile (this is the tiled design of the paperlayer summary's appendix
//     A.4 -- a query tile and the key tile its windows need on chip -- with
//     the key tile streamed in rows so that it fits for wide windows).  A
//     block is stored as 16 keys x 64 bytes, the 16-byte d-slice s of key p
//     at slot s ^ bswz(p) (see bswz).
//  2. Logits.  Per block, S^T = K_block Q^T is one v_mfma_f32_16x16x32 (d =
//     32 is the contraction); lane (g, c) then holds query c against the
//     four keys of block row g.  For a subtile whose queries are all
//     unclamped, the bias enters as the MFMA's accumulator, read from a
//     table over key-minus-query offsets that holds -inf outside the
//     window; other subtiles add the bias from the head's table and mask by
//     each query's clamped window.
//  3. Softmax, single pass over the block rows: per row the max over the
//     four lanes of a query (v_permlane16/32_swap); the weights are
//     p = exp2(c (q.k + B) - m), c = log2(e)/sqrt(d), against a reference m
//     that is moved (rescaling the running sum and output) only when a
//     query's max passes it by more than 8.
//  4. O^T += V^T P^T on the matrix cores, two blocks (32 keys) per
//     v_mfma_f32_16x16x32: the S^T layouts of two blocks side by side are the
//     B operand, and ds_read_b64_tr_b16 of the two blocks supplies V^T. P and
//     V are fp16: bf16 values of V are converted when staged (exactly for
//     magnitudes in [2^-14, 2^16); a tile whose V holds a larger value is
//     run again with V scaled down by a power of two, and its output scaled
//     back). The softmax
//     sum is one more product, with an all-ones operand.
//  5. out = O / sum in fp32, non-temporal stores.
// No ksize^2-wide tensor ever leaves the chip.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_geometry.h"
#include "na_mfma_util.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kLWaves = 4;
constexpr int kLThreads = 64 * kLWaves;
// widest rows (NBW) that take 4 x 16 tiles (see launch_large_nbw)
constexpr int kWideTileMaxNBW = 6;
constexpr int kLMaxBlocks = kLargeMaxBlocks;   // block rows / columns of a tile's union (ksize <= 25)
constexpr int kLRowBytes = kLMaxBlocks * 1024;  // one block row of K (or V): blocks x 16 keys x 64 B
// slices of a block row a thread stages: 4 rows x 4 kLMaxBlocks columns x 4
// slices = 512 for K, as many for V, over 256 threads
constexpr int kLSlices = 4 * 4 * kLMaxBlocks * 4 / kLThreads;

struct LArgs {
    const void *q, *k, *v;
    const float *rpb;
    float *out;
    float *lse;  // per-query log-sum-exp of the logits, or null
    int B, heads, H, W, ks;
    int tiles_x, tiles_y;
    unsigned ntiles;
    int xcd_split;
    float c;  // log2(e) / sqrt(d)
};

// The bias tables `col` and `raw`, the column mask and their paddings are
// described in na_geometry.h.

// A staged block: 16 keys x 64 bytes, the 16-byte d-slice s of key p at
// slot s ^ bswz(p). The K reads (lane (g, c): slice g of key c, 16 bytes) are
// conflict-free under any slot swizzle; the transposing V reads (lane (g, i):
// 8 bytes of key 4 g + i / 4) measured 22% faster with this one than with the
// swizzle of the halo kernels' copies (copy_swz).
__device__ inline unsigned bswz(unsigned p) { return ((p >> 1) & 3u) ^ ((p >> 3) & 1u); }
__device__ inline unsigned bstage_off(int g, int c)
{
    return (unsigned)c * 64u + 16u * ((unsigned)g ^ bswz((unsigned)c));
}
// where lane (g, i) reads V^T for dims 16 dh .. 16 dh + 15: dims 16 dh +
// 4 (i & 3) .. + 3 of key 4 g + (i >> 2); the lane then holds dim 16 dh + i of
// keys 4 g .. 4 g + 3
__device__ inline unsigned btr_read_off(int g, int i, int dh)
{
    const unsigned p = 4u * g + ((unsigned)i >> 2);
    const unsigned s = 2u * dh + ((unsigned)(i & 3) >> 1);
    return p * 64u + 16u * (s ^ bswz(p)) + 8u * (unsigned)(i & 1);
}

// Where one tile sits (uniform values).
struct LTile {
    int h;
    int64_t map_base;
    int y0, x0;    // first query
    int uy0, ux0;  // first key row / column of the union of the tile's windows
    int nbr, nbc;  // block rows / columns of the union
};

template <int WX>
__device__ inline LTile ltile(const LArgs &a, unsigned t)
{
    constexpr int TY = 16 / WX, TX = 4 * WX;
    const unsigned tpm = (unsigned)a.tiles_x * a.tiles_y;
    const unsigned per_head = tpm * (unsigned)a.B;
    LTile g;
    g.h = (int)(t / per_head);
    const unsigned rem = t - (unsigned)g.h * per_head;
    const unsigned b = rem / tpm, tr = rem - b * tpm;
    const int ty = (int)(tr / a.tiles_x), tx = (int)(tr - (unsigned)ty * a.tiles_x);
    g.map_base = ((int64_t)b * a.heads + g.h) * a.H * a.W;
    g.y0 = TY * ty;
    g.x0 = TX * tx;
    const LargeTileGeom u = large_tile_geometry(g.y0, g.x0, TY, TX, a.ks, a.H, a.W);
    g.uy0 = u.uy0;
    g.ux0 = u.ux0;
    g.nbr = u.nbr;
    g.nbc = u.nbc;
    return g;
}

// This thread's share of staging one block row: slices tid and tid + 256
// of K and V. The block row is laid out as 4 key rows x 32 columns (8
// blocks, the widest union) of four 16-byte d-slices: slice s is d-slice
// s % 4 of pixel s / 4, at row (s / 4) / 32 and column (s / 4) % 32; columns
// past the union (or the map) load as zeros and fill unused blocks.
struct LSlices {
    unsigned goff[kLSlices];  // global byte offset in block row 0, or kOutOfRange
};

__device__ inline int lslice_lds(int tid, int e)
{
    const int s = tid + kLThreads * e;
    const int px = s >> 2, g = s & 3;
    const int ri = px >> 5, cj = px & 31;
    return (int)((unsigned)(cj >> 2) * 1024u + bstage_off(g, 4 * ri + (cj & 3)));
}

__device__ inline void lslices(const LArgs &a, const LTile &t, int tid, LSlices &sl)
{
#pragma unroll
    for (int e = 0; e < kLSlices; ++e) {
        const int s = tid + kLThreads * e;
        const int px = s >> 2, g = s & 3;
        const int ri = px >> 5, cj = px & 31;
        const int gy = t.uy0 + ri, gx = t.ux0 + cj;
        // rows past the map fall past the buffer's end in any block row; a
        // column past the map would wrap into the next row, so it is cut here
        sl.goff[e] = cj < 4 * t.nbc && gx < a.W ? (unsigned)(gy * a.W + gx) * 64u + 16u * g : kOutOfRange;
    }
}

struct LStage {
    u32x4 k[kLSlices], v[kLSlices];
};

// Block row rb: the offsets of block row 0 plus 4 rb map rows (an
// out-of-range offset stays out of range: it and the addition are both
// below 2^31).
__device__ inline void lstage_load(const LArgs &a, const LTile &t, const LSlices &sl, int rb, LStage &st)
{
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, t.map_base, kD * 2, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, t.map_base, kD * 2, map_bytes);
    const unsigned drow = (unsigned)(4 * rb * a.W) * 64u;
#pragma unroll
    for (int e = 0; e < kLSlices; ++e) {
        st.k[e] = __builtin_amdgcn_raw_buffer_load_b128(rk, sl.goff[e] + drow, 0, 0);
        st.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, sl.goff[e] + drow, 0, 0);
    }
}

// Write a staged block row to LDS. For bf16 inputs the values of V go in
// as fp16, so that the weights multiply them in fp16 (one product instead
// of a bf16 hi + lo pair): every bf16 value below 2^16 in magnitude
// converts exactly, except that those below 2^-14 lose low bits (an
// absolute error under 2^-25). A thread that meets a larger one (or an
// infinity) raises `ovf` to (tile sequence number << 8 | the largest
// exponent), and the workgroup then runs the tile again with V scaled by a
// power of two (SCALED, by vs) that brings it into range; the output is
// scaled back. Only values below 2^-24 of the tile's largest are then lost.
template <typename T, bool SCALED>
__device__ inline void lstage_write(const int (&lds)[kLSlices], const LStage &st, unsigned char *kbuf,
                                    unsigned char *vbuf, unsigned *ovf, unsigned seq, float vs)
{
    float big = 0.f;
#pragma unroll
    for (int e = 0; e < kLSlices; ++e) {
        *reinterpret_cast<u32x4 *>(kbuf + lds[e]) = st.k[e];
        u32x4 y = st.v[e];
        if constexpr (!__is_same(T, _Float16)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float lo = __uint_as_float(st.v[e][i] << 16), hi = __uint_as_float(st.v[e][i] & 0xffff0000u);
                if constexpr (SCALED) {
                    lo *= vs;
                    hi *= vs;
                } else {
                    // big = max(big, |lo|, |hi|) in one instruction (NaNs need no
                    // flag: they stay NaN in fp16)
                    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(big) : "v"(big), "v"(lo), "v"(hi));
                }
                y[i] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, half2));
            }
        }
        *reinterpret_cast<u32x4 *>(vbuf + lds[e]) = y;
    }
    if constexpr (!__is_same(T, _Float16) && !SCALED)
        if (big >= 65520.f)  // rounds to infinity in fp16
            __hip_atomic_fetch_max(ovf, seq << 8 | __float_as_uint(big) >> 23, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Fill the head's two bias tables (see col_extent).
__device__ inline void lstage_bias(const LArgs &a, int h, float *raw, float *col, int tid)
{
    const int ks = a.ks, nb = 2 * ks - 1, n = nb * nb;
    const float *rb = a.rpb ? a.rpb + (int64_t)h * n : nullptr;
    // the kRawPad floats before the table are read too (and masked): -inf, so
    // that no stale LDS value (a NaN) meets the mask
    if (tid < kRawPad) raw[tid - kRawPad] = -__builtin_inff();
    for (int u = tid; u < raw_floats(ks); u += kLThreads) raw[u] = u < n ? (rb ? rb[u] : 0.f) : -__builtin_inff();
    for (int u = tid; u < col_floats(ks); u += kLThreads) {
        const int src = col_entry_source(u, ks);
        col[u] = src < 0 ? -__builtin_inff() : (rb ? rb[src] : 0.f);
    }
}

// Work of one wave on one tile, carried across the block rows.
struct LWave {
    bool active, colclamp;
    int rb0, rb1, cb0, ncb;  // its block rows [rb0, rb1] and columns [cb0, cb0 + ncb)
    int qy, qx, sy;          // this lane's query and its window's first row
    int cxw;                 // first column of the wave's blocks minus the window's first
    int bcol;                // this lane's bias column base (in `col` or `raw`)
    float m, lex;
    floatx4 l;               // softmax sum of the query, in each of its four rows
    floatx4 o[2];
};

template <int WX>
__device__ inline void lwave_begin(const LArgs &a, const LTile &t, int wave, int lane, LWave &w)
{
    const LargeTileGeom tg{t.uy0, t.ux0, t.nbr, t.nbc};
    const LargeWaveGeom g = large_wave_geometry(tg, t.y0, t.x0, wave, WX, a.ks, a.H, a.W);
    w.active = g.active;
    w.colclamp = g.colclamp;
    w.rb0 = g.rb0;
    w.rb1 = g.rb1;
    w.cb0 = g.cb0;
    w.ncb = g.ncb;
    const LargeLaneGeom l = large_lane_geometry(tg, g, lane & 15, a.ks, a.H, a.W);
    w.qy = l.qy;
    w.qx = l.qx;
    w.sy = l.sy;
    w.cxw = l.cxw;
    w.bcol = l.bcol;
    w.m = -__builtin_inff();
    w.lex = 0.f;
    w.l = floatx4{0.f, 0.f, 0.f, 0.f};
    w.o[0] = floatx4{0.f, 0.f, 0.f, 0.f};
    w.o[1] = floatx4{0.f, 0.f, 0.f, 0.f};
}

// Four weights as fp16, the P^T fragment of one 16-key block.
__device__ inline half4 p_half4(const float *p)
{
    return half4{static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]), static_cast<_Float16>(p[2]),
                 static_cast<_Float16>(p[3])};
}

// One block row of one wave over NB column blocks: logits, the softmax
// update, and the products with V (fp16 in LDS). CLAMP: the wave has fewer
// than NB blocks (ncb < NB); blocks past its last read its last block's keys
// and values and get a -inf bias. COLCLAMP: the wave's queries' windows are
// clamped on the column axis; each query's window columns are masked by
// adding `cmask` (0 inside the window, -inf outside) to the bias.
template <typename T, int NB, bool CLAMP, bool COLCLAMP, bool LSE>
__device__ inline void lwave_row(const LArgs &a, const LTile &t, int rb, int lane,
                                 const typename Frag<T>::type &qf, const unsigned char *kbuf,
                                 const unsigned char *vbuf, const float *table, const float *cmask,
                                 LWave &w)
{
    using FragT = typename Frag<T>::type;
    const int ks = a.ks, nb = 2 * ks - 1;
    const int g = lane >> 4, c = lane & 15;
    const int ky = t.uy0 + 4 * rb + g;  // this lane's key row
    lds_cf32 *bp = (lds_cf32 *)table + large_bias_row(COLCLAMP, ky, w.qy, w.sy, ks) + w.bcol;
    lds_cf32 *mp = (lds_cf32 *)cmask + kMaskPad + w.cxw;
    const unsigned char *kb = kbuf + (unsigned)w.cb0 * 1024u + bstage_off(g, c);
    const unsigned char *vb = vbuf + (unsigned)w.cb0 * 1024u;
    float sc[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int jj = CLAMP ? min(j, w.ncb - 1) : j;
        const FragT kf = __builtin_bit_cast(FragT, *(lds_cu4 *)(kb + (unsigned)jj * 1024u));
        floatx4 bias;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bias[e] = bp[4 * j + e];
            if constexpr (COLCLAMP) bias[e] += mp[4 * j + e];
        }
        // q.k + B, -inf outside the query's window
        const floatx4 acc = mfma16x16x32(kf, qf, bias);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[j][e] = acc[e];
    }
    // online softmax over this row's blocks (log2 units; the scores are not
    // yet scaled, and c > 0 makes the scaled max the max of the scaled ones)
    float mc = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mc = fmaxf(mc, sc[j][e]);
    mc = quad_max(mc) * a.c;
    // The weights are taken against a reference m that trails the running
    // max by at most 8 (so they stay <= 2^8): the sum and output are rescaled
    // only when some query's max passes its reference by more than that,
    // which after a query's first window row is rare. The result is the same
    // for any reference; m = -inf (no key of the query seen yet) always moves.
    if (__builtin_amdgcn_ballot_w64(mc > w.m + 8.f)) {
        const float mnew = max_f32(w.m, mc);
        const float corr = __builtin_amdgcn_exp2f(w.m - (mnew == -__builtin_inff() ? 0.f : mnew));
        w.l = w.l * corr;  // corr = 0 while m = -inf: nothing accumulated yet
        if constexpr (LSE) w.lex *= corr;
#pragma unroll
        for (int dh = 0; dh < 2; ++dh) w.o[dh] = w.o[dh] * corr;
        w.m = mnew;
    }
    const float muse = w.m == -__builtin_inff() ? 0.f : w.m;
    // weights and products with V, two blocks (32 keys) per 16 x 16 x 32
    // product: the S^T layouts of blocks j and j + 1 side by side are the B
    // operand of P^T for the pair (lane (g, c): keys 4g .. 4g + 3 of each),
    // and the transposing reads of the two blocks, side by side, the matching
    // A operand V^T; the all-ones A operand sums the weights as they multiply
    // V (fp16-rounded). An odd last block takes 16 x 16 x 16 products.
    const half8 ones8 = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int j = 0; j < NB; j += 2) {
        const bool pair = j + 1 < NB;
        float p[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(sc[j][e], a.c, -muse));
            if (pair) p[4 + e] = __builtin_amdgcn_exp2f(fmaf(sc[j + 1 < NB ? j + 1 : j][e], a.c, -muse));
        }
        if constexpr (LSE) {  // the log-sum-exp takes the fp32 weights
            w.lex += (p[0] + p[1]) + (p[2] + p[3]);
            if (pair) w.lex += (p[4] + p[5]) + (p[6] + p[7]);
        }
        const int ja = CLAMP ? min(j, w.ncb - 1) : j;
        const int jb = CLAMP ? min(j + 1, w.ncb - 1) : j + 1;
        if (pair) {
            const half4 pa = p_half4(p), pb = p_half4(p + 4);
            const half8 ph = __builtin_shufflevector(pa, pb, 0, 1, 2, 3, 4, 5, 6, 7);
            w.l = mfma16x16x32(ones8, ph, w.l);
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(vb + (unsigned)ja * 1024u + btr_read_off(g, c, dh)));
                const v4i16 vbb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(vb + (unsigned)jb * 1024u + btr_read_off(g, c, dh)));
                const half8 vt = __builtin_bit_cast(half8, __builtin_shufflevector(va, vbb, 0, 1, 2, 3, 4, 5, 6, 7));
                w.o[dh] = mfma16x16x32(vt, ph, w.o[dh]);
            }
        } else {
            const half4 pa = p_half4(p);
            w.l = mfma16x16x16(half4{1, 1, 1, 1}, pa, w.l);
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                const v4i16 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16 *)(vb + (unsigned)ja * 1024u + btr_read_off(g, c, dh)));
                w.o[dh] = mfma16x16x16(__builtin_bit_cast(half4, vt), pa, w.o[dh]);
            }
        }
    }
}

// The kind of a wave's row loop: NB blocks per row, CLAMP and COLCLAMP as
// in lwave_row.
template <int NB, bool CLAMP, bool COLCLAMP>
struct RowKind {
    static constexpr int nb = NB;
    static constexpr bool clamp = CLAMP, colclamp = COLCLAMP;
};

// out = O / sum for the wave's queries (lane (g, c): dims 16 dh + 4 g + j of
// query c), non-temporal; with LSE, lane g == 0 also writes ln(sum of
// exp(logits)) of its query.
template <typename T, int WX, bool LSE>
__device__ inline void lwave_store(const LArgs &a, const LTile &t, int wave, int lane, const LWave &w, float os)
{
    const float l = w.l[0];
    const float inv = __builtin_amdgcn_rcpf(l) * os;
    const int g = lane >> 4, c = lane & 15;
    const QueryPos qp = large_query(t.y0, t.x0, wave, WX, c);
    const int y = qp.y, x = qp.x;
    const __amdgpu_buffer_rsrc_t ro =
        map_rsrc(a.out, t.map_base, kD * 4, (unsigned)a.H * a.W * (kD * 4));
    const bool in = y < a.H && x < a.W;
#pragma unroll
    for (int dh = 0; dh < 2; ++dh) {
        const unsigned off = in ? (unsigned)(y * a.W + x) * 128u + 64u * dh + 16u * g : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w.o[dh] * inv), ro, off, 0,
                                               kNonTemporal);
    }
    if constexpr (LSE) {
        const float le = quad_sum(w.lex);
        if (g == 0 && in)
            a.lse[t.map_base + (int64_t)y * a.W + x] = (w.m + __builtin_amdgcn_logf(le)) * 0.6931471805599453f;
    }
}

template <typename T, int NBW, int WX, bool LSE>
__global__ __launch_bounds__(kLThreads) void na2d_large_kernel(LArgs a)
{
    using FragT = typename Frag<T>::type;
    constexpr int kRawMax = raw_floats(NA2D_MFMA_MAX_KSIZE);
    constexpr int kColMax = col_floats(NA2D_MFMA_MAX_KSIZE);
    __shared__ __align__(16) unsigned char kbuf[2][kLRowBytes];
    __shared__ __align__(16) unsigned char vbuf[2][kLRowBytes];
    // the raw table starts kRawPad floats in: a row's first columns may lie
    // a few entries before a table row (they are masked, but read)
    __shared__ float raw_area[kRawPad + kRawMax];
    float *const raw = raw_area + kRawPad;
    __shared__ float col[kColMax];
    __shared__ float cmask[kMaskFloats];
    // per tile parity, the sequence number of a tile whose V holds values too
    // large for fp16 (bf16 inputs)
    __shared__ unsigned ovf[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    unsigned tile, step, end;
    if (a.xcd_split) {
        const unsigned xcd = blockIdx.x & 7u;
        tile = (unsigned)(((uint64_t)a.ntiles * xcd) >> 3) + (blockIdx.x >> 3);
        end = (unsigned)(((uint64_t)a.ntiles * (xcd + 1)) >> 3);
        step = gridDim.x >> 3;
    } else {
        tile = blockIdx.x;
        end = a.ntiles;
        step = gridDim.x;
    }
    if (tile >= end) return;

    if (tid < 2) ovf[tid] = 0u;
    if (tid < kMaskFloats)
        cmask[tid] = (unsigned)(tid - kMaskPad) < (unsigned)a.ks ? 0.f : -__builtin_inff();
    LTile t = ltile<WX>(a, tile);
    int bias_head = t.h;
    lstage_bias(a, t.h, raw, col, tid);
    LSlices sl;
    lslices(a, t, tid, sl);
    LStage st;
    lstage_load(a, t, sl, 0, st);
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    auto load_q = [&](const LTile &tt) {
        const int c = lane & 15, g = lane >> 4;
        const QueryPos qp = large_query(tt.y0, tt.x0, wave, WX, c);
        const int y = min(qp.y, a.H - 1), x = min(qp.x, a.W - 1);
        const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, tt.map_base, kD * 2, map_bytes);
        return __builtin_amdgcn_raw_buffer_load_b128(rq, (unsigned)(y * a.W + x) * 64u + 16u * g, 0,
                                                     kNonTemporal);
    };
    u32x4 qraw = load_q(t);
    int lds_off[kLSlices];
#pragma unroll
    for (int e = 0; e < kLSlices; ++e) lds_off[e] = lslice_lds(tid, e);
    unsigned seq = 1;  // this WG's tiles so far (below 2^24); `ovf` starts at 0
    // a second run of a tile whose V is past the fp16 range: V times vs = 2^-S,
    // the output times 2^S
    bool redo = false;
    float vs = 1.f, os = 1.f;
    auto stage = [&](int b) {
        if (redo)
            lstage_write<T, true>(lds_off, st, kbuf[b], vbuf[b], nullptr, 0u, vs);
        else
            lstage_write<T, false>(lds_off, st, kbuf[b], vbuf[b], &ovf[seq & 1], seq, 1.f);
    };
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // `ovf` is cleared
    stage(0);
    __syncthreads();
    int buf = 0;
    while (true) {
        work_priority(end, tile, step);
        LWave w;
        lwave_begin<WX>(a, t, wave, lane, w);
        const FragT qf = __builtin_bit_cast(FragT, qraw);
        const unsigned next = tile + step;
        const bool more = next < end;
        LTile tn = t;
        LSlices sn = sl;
        // The row loop, compiled once per kind of wave (blocks per row, column
        // clamping: uniform over the wave and fixed for the tile), so that its
        // accumulators stay in place from row to row.
        auto rows = [&](auto kind) {
            using K = decltype(kind);
            const float *table = K::colclamp ? raw : col;
            for (int rb = 0; rb < t.nbr; ++rb) {
                // The next block row, or the next tile's first with its queries,
                // loads while this one is used. The loads are issued on every row
                // (past the end: out of range, which reads nothing) so that they
                // always land in the same registers: loads issued on two paths
                // would be merged by copies that wait for them at once.
                const bool last = rb + 1 == t.nbr;
                if (last && more) {
                    tn = ltile<WX>(a, next);
                    lslices(a, tn, tid, sn);
                }
                {
                    const int64_t base = last ? tn.map_base : t.map_base;
                    const unsigned drow = last ? 0u : (unsigned)(4 * (rb + 1) * a.W) * 64u;
                    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, base, kD * 2, map_bytes);
                    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, base, kD * 2, map_bytes);
#pragma unroll
                    for (int e = 0; e < kLSlices; ++e) {
                        const unsigned off = last ? (more ? sn.goff[e] : kOutOfRange) : sl.goff[e] + drow;
                        st.k[e] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
                        st.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
                    }
                    if (last) {  // the next tile's queries (uniform branch, one load)
                        const int c = lane & 15, g = lane >> 4;
                        const QueryPos qp = large_query(tn.y0, tn.x0, wave, WX, c);
                        const int y = min(qp.y, a.H - 1), x = min(qp.x, a.W - 1);
                        const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, base, kD * 2, map_bytes);
                        qraw = __builtin_amdgcn_raw_buffer_load_b128(
                            rq, more ? (unsigned)(y * a.W + x) * 64u + 16u * g : kOutOfRange, 0, kNonTemporal);
                    }
                }
                if (w.active && rb >= w.rb0 && rb <= w.rb1)
                    lwave_row<T, K::nb, K::clamp, K::colclamp, LSE>(a, t, rb, lane, qf, kbuf[buf], vbuf[buf],
                                                                    table, cmask, w);
                if (last) break;
                // the other buffer was last read before the barrier that ended the previous row
                __builtin_amdgcn_s_waitcnt(0);
                stage(buf ^ 1);
                __syncthreads();
                buf ^= 1;
            }
        };
        // NBW blocks cover any alignment of the wave's windows in the block
        // grid, NBW - 1 the aligned case; fewer (at the map's borders) run the
        // NBW - 1 loop with its last blocks masked
        if (w.colclamp) {
            if (w.ncb == NBW)
                rows(RowKind<NBW, false, true>{});
            else if (w.ncb == NBW - 1)
                rows(RowKind<NBW - 1, false, true>{});
            else
                rows(RowKind<NBW - 1, true, true>{});
        } else {
            if (w.ncb == NBW)
                rows(RowKind<NBW, false, false>{});
            else if (w.ncb == NBW - 1)
                rows(RowKind<NBW - 1, false, false>{});
            else
                rows(RowKind<NBW - 1, true, false>{});
        }
        if constexpr (!__is_same(T, _Float16)) {
            // Uniform over the workgroup: every row of the tile was staged before
            // the last barrier, and the word is next raised two tiles on.
            const unsigned f = __builtin_amdgcn_readfirstlane(ovf[seq & 1]);
            if (!redo && f >> 8 == seq) {
                // Rare: run the tile again with V times 2^-S, S = (largest
                // exponent) - 14, so that every |v| 2^-S < 2^15.
                const int S = (int)(f & 0xffu) - 127 - 14;
                vs = __builtin_ldexpf(1.f, -S);
                os = __builtin_ldexpf(1.f, S);
                redo = true;
                // the other buffer was last read before the last barrier
                __builtin_amdgcn_s_waitcnt(0);
                lstage_load(a, t, sl, 0, st);
                qraw = load_q(t);
                __builtin_amdgcn_s_waitcnt(0);
                stage(buf ^ 1);
                __syncthreads();
                buf ^= 1;
                continue;
            }
        }
        if (w.active) lwave_store<T, WX, LSE>(a, t, wave, lane, w, os);
        redo = false;
        os = 1.f;
        if (!more) break;
        __builtin_amdgcn_s_waitcnt(0);
        if (tn.h != bias_head) {  // rare: the tile list is head-major
            __syncthreads();      // every wave is done with this head's tables
            lstage_bias(a, tn.h, raw, col, tid);
            bias_head = tn.h;
        }
        ++seq;
        stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
        t = tn;
        sl = sn;
        tile = next;
    }
}

template <typename T, int NBW, int WX, bool LSE>
hipError_t launch_large_typed(const LArgs &a0, hipStream_t stream)
{
    LArgs a = a0;
    constexpr int TY = 16 / WX, TX = 4 * WX;
    a.tiles_x = (a.W + TX - 1) / TX;
    a.tiles_y = (a.H + TY - 1) / TY;
    const uint64_t ntiles = (uint64_t)a.B * a.heads * a.tiles_x * a.tiles_y;
    if (ntiles == 0 || ntiles > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.ntiles = (unsigned)ntiles;
    const auto kern = na2d_large_kernel<T, NBW, WX, LSE>;
    int per_cu = 0;
    const hipError_t e = occupancy(reinterpret_cast<const void *>(kern), kLThreads, 0, per_cu);
    if (e != hipSuccess) return e;
    const int cus = device_cus();
    if (per_cu <= 0 || cus <= 0) return hipErrorInvalidConfiguration;
    uint64_t grid = (uint64_t)cus * per_cu;
    if (grid > a.ntiles) grid = a.ntiles;
    // a workgroup numbers its tiles in 24 bits (the V range check)
    if (a.ntiles / grid + 2 >= (1u << 24)) return hipErrorInvalidConfiguration;
    a.xcd_split = 0;
    if (grid >= 64) {
        grid &= ~7ull;
        a.xcd_split = 1;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kLThreads), 0, stream, a);
    return hipGetLastError();
}

// Tiles of 4 x 16 queries while their union of windows fits the 32 staged
// columns (16 + k - 1 <= 32: k <= 17): every block row of such a tile is used
// by all four waves. Wider windows take 8 x 8 tiles, whose first and last
// block rows only two waves use.
template <typename T, bool LSE>
hipError_t launch_large_nbw(const LArgs &a, hipStream_t stream)
{
    // blocks a wave's windows touch per block row: (3 + k) columns, aligned
    // anywhere in the tile's block grid
    switch ((a.ks + 9) / 4) {
    case 4: return launch_large_typed<T, 4, kWideTileMaxNBW >= 4 ? 4 : 2, LSE>(a, stream);
    case 5: return launch_large_typed<T, 5, kWideTileMaxNBW >= 5 ? 4 : 2, LSE>(a, stream);
    case 6: return launch_large_typed<T, 6, kWideTileMaxNBW >= 6 ? 4 : 2, LSE>(a, stream);
    case 7: return launch_large_typed<T, 7, 2, LSE>(a, stream);
    case 8: return launch_large_typed<T, 8, 2, LSE>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mfma_large(const Problem &p, hipStream_t stream)
{
    if (p.d != kD || p.mode != NA_WINDOW_NA || p.depth != 1 || p.kd != 1 || p.kh != p.kw ||
        p.ksize < 7 || p.ksize > NA2D_MFMA_MAX_KSIZE)
        return hipErrorInvalidValue;
    // byte offsets inside one map are 32-bit (buffer addressing)
    if ((uint64_t)p.H * p.W * (kD * 4) > 0x7fffffffull) return hipErrorInvalidValue;
    LArgs a;
    a.q = p.q;
    a.k = p.k;
    a.v = p.v;
    a.rpb = p.rpb;
    a.out = p.out;
    a.lse = p.lse;
    a.B = p.B;
    a.heads = p.heads;
    a.H = p.H;
    a.W = p.W;
    a.ks = p.ksize;
    a.tiles_x = a.tiles_y = 0;  // per tile shape (launch_large_typed)
    a.ntiles = 0;
    a.xcd_split = 0;
    a.c = 1.4426950408889634f / sqrtf((float)kD);
    if (p.dtype == NA2D_F16)
        return p.lse ? launch_large_nbw<_Float16, true>(a, stream) : launch_large_nbw<_Float16, false>(a, stream);
    if (p.dtype == NA2D_BF16)
        return p.lse ? launch_large_nbw<__bf16, true>(a, stream) : launch_large_nbw<__bf16, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace na2d
