// na2d_mfma.hip -- NA2D forward for fp16/bf16 inputs on the gfx950 matrix cores.
//
// What is computed is Neighborhood Attention ("Neighborhood Attention
// Transformer", CSDN translation, section 3.1, Eq. 2-4): per query the
// clamped ksize x ksize window, logits (q.k + B) / sqrt(d), softmax over the
// window, weighted sum of the values.
//
// How.  Persistent workgroups of NW waves walk a list of query tiles of
// TY x TX = (NW QY) x QX queries; each wave owns one QY x QX = 16-query subtile.
//  1. Staging.  The tile's key/value halo -- the union of its queries'
//     windows, at most TY + ksize - 1 rows by NC = 16 NCB columns -- goes to
//     LDS as [row][col][d] for both K and V.  The 16-byte d-slice s of pixel
//     column c sits at slot s ^ ((c >> 1) & 3) (halo_slot) so the reads below
//     are free of bank conflicts: 16-byte reads are served 8 lanes (128
//     bytes) at a time, 8-byte transposing reads 16 lanes at a time.  Pixels outside the map get an out-of-range buffer
//     offset and so arrive as zeros.  This is the tiled design of the
//     paperlayer summary's appendix A.4 (a query tile plus a key tile of side
//     tq + k - 1 in on-chip memory), re-shaped for 64-lane waves.
//  2. Logits.  The wave's candidate keys are NR halo rows by NC columns, in
//     blocks of 16 (one row, 16 consecutive columns).  For a block,
//     S^T = K_block Q^T is one v_mfma_f32_16x16x32 (d = 32 is the
//     contraction); each lane then holds one query (lane % 16) and four
//     consecutive keys (4 (lane / 16) + j).  The bias comes from an LDS
//     table holding -inf for keys outside the query's window, so the masked
//     window is exact; with 8-row chunks it enters as the MFMA's accumulator,
//     which then returns q.k + B (bias_in_acc).
//  3. Softmax, single pass over chunks of RPC block rows: the chunk max over
//     the 4 lanes of a query (v_permlane16/32_swap, no LDS) in log2 units
//     (c = log2(e)/sqrt(d)); running max and sum with rescale;
//     p = exp2(c (q.k + B) - m).
//  4. O^T = V^T P^T, again v_mfma_f32_16x16x32: the S^T layout above is
//     exactly the B-operand layout of P^T for 32 keys (two blocks), and
//     ds_read_b64_tr_b16 hands each lane the 4 keys' values of its d from the
//     [row][col][d] copy of V.  P is fp16 for fp16 inputs; for bf16 inputs it
//     is split into bf16 hi + lo parts (two products), so the weights keep
//     ~16 bits either way.
//  5. out = O / sum in fp32 with 16-byte buffer stores (out-of-map lanes get
//     an out-of-range offset and are dropped).  The k = 7 kernels first pass
//     a wave's outputs through LDS, so that each store writes whole rows.
// Three kernels share steps 2-5.  na2d_mfma_kernel (any kernel size) copies
// the halo HBM -> LDS with buffer_load ... lds (no VGPRs) and then waits for
// it; na2d_mfma_pipe_kernel (a compile-time kernel size) loads the next
// tile's halo into registers while the current tile is computed, and writes
// it to LDS between two barriers; na2d_mfma_ring_kernel walks a column of
// tiles and loads only the halo rows that enter.  Each iteration drains the
// vector memory counter completely: loads and stores may retire out of order
// against each other, so a partial count would not prove the halo had landed.
// No ksize^2-wide tensor ever leaves the chip.
#include "na2d.h"
#include "na2d_launch.h"
#include "na_geometry.h"
#include "na_mfma_util.h"
#include "na_xcd.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <vector>

namespace na2d {

int device_cus()
{
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

// Resident workgroups per CU of kernel `f` with `threads` threads and `lds`
// bytes of dynamic LDS on the current device. The occupancy query -- and,
// above 64 KB of LDS, the attribute that allows it -- runs once per kernel,
// device and LDS size; later calls read the answer from a process-wide
// table, so a forward call makes no HIP call besides its launch.
namespace {
struct OccEntry {
    const void *f;
    int dev, threads;
    size_t lds;
    int per_cu;
};
std::mutex g_occ_mutex;
std::vector<OccEntry> g_occ;
std::atomic<long long> g_occ_queries{0};
}  // namespace

hipError_t occupancy(const void *f, int threads, size_t lds, int &per_cu)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_occ_mutex);
    for (const OccEntry &o : g_occ)
        if (o.f == f && o.dev == dev && o.threads == threads && o.lds == lds) {
            per_cu = o.per_cu;
            return hipSuccess;
        }
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, threads, lds);
    g_occ_queries.fetch_add(1);
    if (e != hipSuccess) return e;
    g_occ.push_back(OccEntry{f, dev, threads, lds, per_cu});
    return hipSuccess;
}

namespace {

constexpr int kWaves = 4;     // waves per workgroup of the general kernel, stacked vertically
constexpr int kThreads = 64 * kWaves;

struct Args {
    const void *q, *k, *v;
    const float *rpb;
    float *out;
    float *lse;            // per-query log-sum-exp of the logits, or null
    int B, heads, H, W, ks;
    int tiles_x, tiles_y;  // tiles per map
    unsigned ntiles;       // heads * B * tiles_y * tiles_x
    int lr;                // halo rows held in LDS
    int xcd_split;         // 1: tiles split into 8 contiguous ranges, one per XCD
    float c;               // log2(e) / sqrt(d)
    // column runs (na2d_mfma_ring_kernel): run r covers tile rows
    // [part * run_len, ...) of tile column r / runs_per_col, part = r % runs_per_col
    unsigned nruns;
    int runs_per_col, run_len;
};

// Row pitch of a bias table that a wave reads from QY rows at once (its
// queries' rows): at least `need` floats, and congruent to 32 / QY modulo 32.
// A b32 LDS read serves 32 lanes per cycle from 32 four-byte banks; with this
// pitch the QY rows' column ranges fall in disjoint banks instead of two rows
// meeting in a bank.
__host__ __device__ constexpr int bias_pitch(int need, int qy)
{
    return need + ((32 / qy - need) % 32 + 32) % 32;
}

// With chunks of 8 block rows, every bias read of a chunk issues up front,
// and the bias enters the QK MFMA as its accumulator (the MFMA returns
// q.k + B; the logit scale is applied inside the exp's fma): -1 us at k = 7.
// With short chunks the MFMA would wait on each read; there the tables hold
// the bias times the scale and it is added by one fma after the MFMA, which
// measured 0.5 us faster at k = 5 and 9.
__host__ __device__ constexpr bool bias_in_acc(int rpc) { return rpc >= 8; }

template <int QY, int QX, int NCB, int RPC, int NW = kWaves, bool CT = true>
struct Shape {
    static constexpr int NT = 64 * NW;              // threads per workgroup
    static constexpr int TY = QY * NW;              // tile rows
    static constexpr int TX = QX;                   // tile cols
    static constexpr int NC = 16 * NCB;             // halo cols held in LDS
    static constexpr int BPC = RPC * NCB;           // key blocks per chunk
    static constexpr int P = bias_pitch(NC + QX - 1, QY);  // interior bias table pitch
    static constexpr int PC = 2 * NC - 1;           // class table pitch
    // class tables (one per column class, see stage_bias) for one 16-column
    // block of 8-query-wide subtiles when CT allows them; otherwise a general
    // table plus an interior table
    static constexpr bool CLS = CT && NCB == 1 && QX == 8;
    static_assert(QY * QX == 16, "a wave owns 16 queries");
    static_assert(BPC % 2 == 0, "P.V consumes key blocks in pairs");
};

// LDS layout: K and V halos as [lr][NC pixels][4 x 16-byte d-slices], then
// the head's bias tables (see stage_bias):
//  - class layout: k tables [2k-1][PC] floats, then a -inf strip of
//    RPC * PC + NC floats;
//  - split layout: the general table [2k + 1][2k] (a -inf row, then the
//    general rows), then the interior table [NR + QY - 1][P].
__host__ __device__ inline unsigned halo_bytes(int lr, int nc) { return (unsigned)lr * nc * 64u; }
// LDS slot (16 bytes) of d-slice s of halo column c, and, the XOR being its
// own inverse, the d-slice held by slot s
__host__ __device__ constexpr int halo_slot(int s, int c) { return s ^ ((c >> 1) & 3); }
__host__ __device__ inline unsigned b_offset(int lr, int nc) { return 2u * halo_bytes(lr, nc); }
__host__ __device__ constexpr unsigned class_floats(int ks, int pc) { return (unsigned)ks * (2 * ks - 1) * pc; }
__host__ __device__ constexpr unsigned bias_floats(bool cls, int ks, int nr, int qy, int qx, int nc, int rpc)
{
    if (cls) return class_floats(ks, 2 * nc - 1) + (unsigned)(rpc * (2 * nc - 1) + nc);
    return (unsigned)((2 * ks + 1) * bias_pitch(2 * ks, qy)) +
           (unsigned)((nr + qy - 1) * bias_pitch(nc + qx - 1, qy));
}
__host__ __device__ inline unsigned lds_bytes(int lr, int nc, unsigned bfloats)
{
    return (b_offset(lr, nc) + bfloats * 4u + 15u) & ~15u;
}

// Where one query tile sits (uniform across the workgroup).
struct Tile {
    int h, y0, x0, hy0, hr, cx;
    int64_t map_base;  // first pixel of the (b, h) map
};

template <int TY, int TX, int NC, int WM>
__device__ inline Tile tile_geometry(const Args &a, unsigned t)
{
    // tiles are numbered head-major (head, batch, tile row, tile col), so that a
    // run of consecutive tiles shares one head and one bias table
    const unsigned tpm = (unsigned)a.tiles_x * a.tiles_y;
    const unsigned per_head = tpm * (unsigned)a.B;
    Tile g;
    g.h = (int)(t / per_head);
    const unsigned rem = t - (unsigned)g.h * per_head;
    const unsigned b = rem / tpm, tr = rem - b * tpm;
    const int ty = (int)(tr / a.tiles_x), tx = (int)(tr - (unsigned)ty * a.tiles_x);
    g.map_base = ((int64_t)b * a.heads + g.h) * a.H * a.W;
    g.y0 = ty * TY;
    g.x0 = tx * TX;
    // the halo: rows [hy0, hy0 + hr), columns [cx, cx + NC) (na_geometry.h)
    const HaloGeom hg = halo_geometry<TY, NC, WM>(g.y0, g.x0, a.ks, a.H, a.W);
    g.hy0 = hg.hy0;
    g.hr = hg.hr;
    g.cx = hg.cx;
    return g;
}

// This head's bias tables, for keys inside a query's window and -inf
// outside it, unscaled or times the logit scale c = log2(e)/sqrt(d) as
// bias_in_acc says.  Two layouts:
//  - class (one 16-column block, k <= 9): a query's window columns depend on
//    e_x = x - sx only (its offset inside the clamped window), so there is one
//    table per e_x in [0, k): T_e[a][b'] = bias(a, b) for the relative offset
//    (a, b) = (ky - y + k - 1, kx - x + k - 1), b = b' - (NC - k), when b lies
//    in [k-1-e_x, 2k-2-e_x], else -inf.  A lane reads element (row i, col c)
//    of its candidate keys at lane_base + i * PC + c; rows outside its window
//    read from the -inf strip instead.
//  - split: the general table [2k + 1][pitch >= 2k]: a -inf row, the
//    (2k-1)^2 table, then a -inf row, with -inf in columns 2k-1 on (see
//    bias_pitch). Row a + 1 holds row offset a, so that a candidate row one
//    above a window (relative offset -k) still reads inside the table. Then the
//    interior table [NR + QY - 1][P]: for
//    a subtile none of whose queries is clamped, lane (qy, qx, g) reads
//    element (row i, col c) at (QY-1-qy+i) * P + (QX-1-qx+c), which holds the
//    bias of that offset or -inf where |dy| or |dx| exceeds k/2.
// Staging runs in two phases so that HBM is visited once, by every thread at
// the same time: load_raw_bias issues the loads of the head's (2k-1)^2 table
// (indices clamped rather than branched around, so no load waits for
// another), and stage_bias writes them, scaled, into `raw` -- an LDS scratch
// area that is free at every call -- then expands the tables from that copy.
// stage_bias ends with a barrier (`raw` may be overwritten afterwards, `bt`
// may be read).
// raw values per thread for a compile-time kernel size (0: any size)
__host__ __device__ constexpr int raw_per_thread(int ks, int nt)
{
    const int k = ks ? ks : NA2D_MFMA_MAX_KSIZE;
    return (2 * k - 1) * (2 * k - 1) / nt + 1;
}

template <int NT, int NV>
__device__ inline void load_raw_bias(const Args &a, int ks, int h, int tid, float (&val)[NV])
{
    if (!a.rpb) return;
    const int nb = 2 * ks - 1, nraw = nb * nb;
    const float *rb = a.rpb + (int64_t)h * nraw;
#pragma unroll
    for (int e = 0; e < NV; ++e) val[e] = rb[min(e * NT + tid, nraw - 1)];
}

template <int QY, int QX, int NC, int RPC, bool CLS, int NT, int NV>
__device__ inline void stage_bias(const Args &a, int ks, const float (&val)[NV], float *bt,
                                  float *raw, int nr, int tid)
{
    constexpr int P = bias_pitch(NC + QX - 1, QY), PC = 2 * NC - 1;
    const int nb = 2 * ks - 1, nraw = nb * nb, tw = bias_pitch(2 * ks, QY), r = ks >> 1;
    if (a.rpb) {
#pragma unroll
        for (int e = 0; e < NV; ++e)
            if (e * NT + tid < nraw) raw[e * NT + tid] = bias_in_acc(RPC) ? val[e] : val[e] * a.c;
    } else {
        for (int u = tid; u < nraw; u += NT) raw[u] = 0.f;
    }
    __syncthreads();
    int n1, n;
    if constexpr (CLS) {
        n1 = (int)class_floats(ks, PC);
        n = n1 + RPC * PC + NC;
    } else {
        n1 = (2 * ks + 1) * tw;
        n = n1 + (nr + QY - 1) * P;
    }
    for (int u = tid; u < n; u += NT) {
        int br = -1, bc = -1;
        if constexpr (CLS) {
            if (u < n1) {
                const int ex = u / (nb * PC), rem = u - ex * (nb * PC);
                br = rem / PC;
                bc = rem - br * PC - (NC - ks);
                if (bc < ks - 1 - ex || bc > 2 * ks - 2 - ex) br = -1;
            }
        } else {
            if (u < n1) {
                br = u / tw;
                bc = u - br * tw;
                --br;  // row 0 is the -inf row above the table
                if (br >= nb || bc >= nb) br = -1;
            } else {
                const int ui = u - n1, ai = ui / P, bi = ui - ai * P;
                br = ai + r - (QY - 1);
                bc = bi + r - (QX - 1);
                if (br < ks - 1 - r || br > ks - 1 + r || bc < ks - 1 - r || bc > ks - 1 + r)
                    br = -1;
            }
        }
        bt[u] = br < 0 ? -__builtin_inff() : raw[br * nb + bc];
    }
    __syncthreads();
}

template <int QY, int QX, int NC, int RPC, bool CLS, int NT = kThreads>
__device__ inline void stage_bias(const Args &a, int ks, int h, float *bt, float *raw, int nr,
                                  int tid)
{
    float val[raw_per_thread(0, NT)];
    load_raw_bias<NT>(a, ks, h, tid, val);
    stage_bias<QY, QX, NC, RPC, CLS, NT>(a, ks, val, bt, raw, nr, tid);
}

// Issue the copies of one tile's K/V halo into LDS (each wave its rows) and
// the load of this wave's queries into registers.
template <typename T, int QY, int QX, int NCB, int RPC>
__device__ inline void stage_tile(const Args &a, const Tile &t, unsigned char *smem, int lr,
                                  int wave, int lane, typename Frag<T>::type &qf)
{
    using S = Shape<QY, QX, NCB, RPC>;
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, t.map_base, kD * 2, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, t.map_base, kD * 2, map_bytes);
    const int c_lane = lane >> 2;  // pixel column within a 16-column block
    const int slot = lane & 3;
    for (int r = wave; r < lr; r += kWaves) {
        const int gy = t.hy0 + r;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int c = 16 * cb + c_lane;
            const int sl = halo_slot(slot, c);  // the d-slice this LDS slot holds
            const int gx = t.cx + c;
            const unsigned off = (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W
                                     ? (unsigned)(gy * a.W + gx) * 64u + 16u * sl
                                     : kOutOfRange;
            unsigned char *dk = smem + (unsigned)(r * S::NC + 16 * cb) * 64u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)dk, 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dk + halo_bytes(lr, S::NC)), 16,
                                                     off, 0, 0, 0);
        }
    }
    // queries: lane (g, qi) takes d-slice g of query qi (the B operand of S^T)
    const int g = lane >> 4, qi = lane & 15;
    const int y = min(t.y0 + QY * wave + qi / QX, a.H - 1);
    const int x = min(t.x0 + qi % QX, a.W - 1);
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, t.map_base, kD * 2, map_bytes);
    const u32x4 qv =
        __builtin_amdgcn_raw_buffer_load_b128(rq, (unsigned)(y * a.W + x) * 64u + 16u * g, 0, 0);
    qf = __builtin_bit_cast(typename Frag<T>::type, qv);
}

// Attention for one wave's 16 queries of tile t, reading the staged halo.
// Leaves the unnormalised output in o (lane: query lane % 16, d = 16 dh +
// 4 (lane / 16) + j) and the softmax sum of this lane's keys in lsum.
// `ry` is the wave's first candidate key row (map coordinates).  MODE picks
// how bias and window mask are read (see stage_bias):
//  kClass:    class tables; per-lane base plus fixed offsets, rows outside the
//             window redirected to the -inf strip;
//  kInterior: split layout, no query of the subtile clamped, candidate keys
//             start k/2 rows above / columns left of the first query;
//  kGeneral:  split layout, general table with per-row / per-column indices.
enum { kClass = 0, kInterior = 1, kGeneral = 2 };

// With LSE, also leaves the running max (log2 units, shared by a query's four
// lanes) in st.m and, in st.l, this lane's softmax sum over the unrounded
// weights (the fp16 path's lsum sums the weights as rounded to fp16).
struct SoftStats {
    float m, l;
};

// RING > 0: the halo is a ring of RING rows in which map row gy sits at slot
// gy & (RING - 1) (see na2d_mfma_ring_kernel); 0: halo row i at LDS row i.
template <typename T, int QY, int QX, int NCB, int RPC, int KS, int MODE, int WM, bool CT, bool LSE = false,
          int RING = 0>
__device__ inline void attend(const Args &a, const Tile &t, const unsigned char *smem,
                              const float *btab, int lr, int wave, int ry, int lane,
                              const typename Frag<T>::type &qf, floatx4 (&o)[2], float &lsum,
                              SoftStats &st)
{
    using S = Shape<QY, QX, NCB, RPC, kWaves, CT>;
    using FragT = typename Frag<T>::type;
    constexpr int P = S::P, PC = S::PC;
    constexpr bool kBiasAcc = bias_in_acc(RPC);
    const int ks = KS ? KS : a.ks;
    const int H = a.H, W = a.W;
    const int nr = wave_rows(QY, RPC, ks);
    const int tw = bias_pitch(2 * ks, QY);  // general table pitch
    const int g = lane >> 4, qi = lane & 15;
    const int qy = qi / QX, qx = qi % QX;
    const int y = min(t.y0 + QY * wave + qy, H - 1);
    const int x = min(t.x0 + qx, W - 1);
    const int rrel = RING ? 0 : ry - t.hy0;
    // LDS row of candidate row r of chunk c0 (a uniform value)
    auto slot = [&](int c0, int r) { return RING ? ((ry + c0 + r) & (RING - 1)) : r; };

    // K block row: 16 lanes read 16 columns' d-slice g (swizzled slot)
    lds_cu8 *kp = (lds_cu8 *)(smem + (unsigned)(rrel * S::NC) * 64u + (unsigned)qi * 64u +
                              16u * (unsigned)halo_slot(g, qi));
    // V^T fragment via the transposing read: lane (g, qi) supplies dims
    // 16 dh + 4 (qi & 3) .. + 3 of column 4 g + (qi >> 2) and receives dim
    // 16 dh + qi of columns 4 g .. 4 g + 3
    const unsigned char *vbase = smem + halo_bytes(lr, S::NC) + (unsigned)(rrel * S::NC) * 64u +
                                 (unsigned)(4 * g + (qi >> 2)) * 64u + 8u * (unsigned)(qi & 1);
    lds_cu8 *vp0 = (lds_cu8 *)(vbase + 16u * (unsigned)halo_slot(0 + ((qi >> 1) & 1), 4 * g + (qi >> 2)));
    lds_cu8 *vp1 = (lds_cu8 *)(vbase + 16u * (unsigned)halo_slot(2 + ((qi >> 1) & 1), 4 * g + (qi >> 2)));

    lds_cf32 *bp;          // per-lane bias base (advanced per chunk)
    lds_cf32 *bneg = nullptr;
    int sy = 0, lo = 0, coloff[NCB][4];
    // General path with a compile-time kernel size and one chunk: the table
    // pitch is a constant, so each of a lane's columns keeps one pointer and
    // a row is an instruction offset from it. Rows [nr - k, k) lie inside
    // every window; the others (the first and last for QY = 2) are masked by
    // a select on the value read.
    constexpr bool kFixedGeneral = MODE == kGeneral && KS && RPC == wave_rows(QY, RPC, KS);
    constexpr int kTW = KS ? bias_pitch(2 * KS, QY) : 0;
    lds_cf32 *gp[kFixedGeneral ? NCB : 1][4];
    if constexpr (MODE == kClass) {
        sy = window_start<WM>(y, ks, H);
        const int ex = x - window_start<WM>(x, ks, W);
        lo = sy - ry;  // first candidate row inside the window
        const int nb = 2 * ks - 1;
        bp = (lds_cf32 *)btab + ex * (nb * PC) + (ry - y + ks - 1) * PC + (t.cx - x + ks - 1) +
             (S::NC - ks) + 4 * g;
        bneg = (lds_cf32 *)btab + class_floats(ks, PC) + 4 * g;
    } else if constexpr (MODE == kInterior) {
        bp = (lds_cf32 *)btab + (2 * ks + 1) * tw + (QY - 1 - qy) * P + (QX - 1 - qx + 4 * g);
    } else {
        bp = (lds_cf32 *)btab + tw;  // row offset 0 (past the -inf row)
        sy = window_start<WM>(y, ks, H);
        const int sx = window_start<WM>(x, ks, W);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = t.cx + 16 * cb + 4 * g + j;
                coloff[cb][j] = (unsigned)(col - sx) < (unsigned)ks ? col - x + ks - 1 : 2 * ks - 1;
            }
        if constexpr (kFixedGeneral) {
            // candidate row r reads table row (ry + r - y + k - 1) + 1, which
            // lies in [0, 2k] for every NA map, so one pointer per column
            // serves all rows
            lo = sy - ry;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gp[cb][j] = (lds_cf32 *)btab + (ry - y + ks) * kTW + coloff[cb][j];
                    opaque(gp[cb][j]);
                }
        }
    }
    // keep each per-lane LDS pointer in one register, so that every access
    // below is that register plus an instruction offset
    opaque(kp);
    opaque(vp0);
    opaque(vp1);
    if constexpr (MODE != kGeneral) opaque(bp);
    if constexpr (MODE == kClass) opaque(bneg);

    float m = -__builtin_inff();
    lsum = 0.f;
    float lex = 0.f;
    o[0] = floatx4{0.f, 0.f, 0.f, 0.f};
    o[1] = floatx4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < nr; c0 += RPC) {
        float sc[RPC][NCB][4];
        // with a ring the row addresses are computed, and the chunk's K rows
        // are read up front so that the reads overlap
        FragT kring[RING ? RPC : 1][NCB];
        if constexpr (RING) {
#pragma unroll
            for (int rr = 0; rr < RPC; ++rr)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    kring[rr][cb] = __builtin_bit_cast(
                        FragT, *(lds_cu4 *)(kp + (slot(c0, rr) * S::NC + 16 * cb) * 64));
        }
#pragma unroll
        for (int rr = 0; rr < RPC; ++rr) {
            lds_cf32 *brow = bp;
            if constexpr (MODE == kClass) {
                // rows k .. nr-1-(nr-k) are inside every window when nr is fixed
                const bool always = KS && RPC == wave_rows(QY, RPC, KS) &&
                                    rr >= wave_rows(QY, RPC, KS) - KS && rr < KS;
                brow = (always || (unsigned)(c0 + rr - lo) < (unsigned)ks ? bp : bneg) + rr * PC;
            } else if constexpr (MODE == kInterior) {
                brow = bp + rr * P;
            } else if constexpr (!kFixedGeneral) {
                const int krow = ry + c0 + rr;
                brow = bp + ((unsigned)(krow - sy) < (unsigned)ks ? (krow - y + ks - 1) * tw
                                                                   : (2 * ks - 1) * tw);
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const FragT kf =
                    RING ? kring[RING ? rr : 0][cb]
                         : __builtin_bit_cast(FragT, *(lds_cu4 *)(kp + (rr * S::NC + 16 * cb) * 64));
                // the bias, -inf outside the window (see bias_in_acc)
                floatx4 bias;
                if constexpr (kFixedGeneral) {
                    constexpr int nr1 = wave_rows(QY, RPC, KS);
                    const bool always = rr >= nr1 - KS && rr < KS;
                    const bool rowin = always || (unsigned)(rr - lo) < (unsigned)KS;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bias[j] = gp[cb][j][rr * kTW];
                        if (!always) bias[j] = rowin ? bias[j] : -__builtin_inff();
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        bias[j] = MODE == kGeneral ? brow[coloff[cb][j]] : brow[16 * cb + j];
                }
                if constexpr (kBiasAcc) {
                    const floatx4 acc = mfma16x16x32(kf, qf, bias);  // q.k + B
#pragma unroll
                    for (int j = 0; j < 4; ++j) sc[rr][cb][j] = acc[j];
                } else {
                    const floatx4 acc = mfma16x16x32(kf, qf, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int j = 0; j < 4; ++j) sc[rr][cb][j] = fmaf(acc[j], a.c, bias[j]);  // log2 units
                }
            }
        }
        float mc = -__builtin_inff();
#pragma unroll
        for (int rr = 0; rr < RPC; ++rr)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) mc = fmaxf(mc, sc[rr][cb][j]);
        // in log2 units; with the bias in the accumulator the scores are not
        // yet scaled, and c > 0 makes this the max of the scaled ones, bit for bit
        mc = kBiasAcc ? quad_max(mc) * a.c : quad_max(mc);
        const float mnew = fmaxf(m, mc);
        const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
        if (c0 > 0) {  // rescale what earlier chunks accumulated
            const float corr = __builtin_amdgcn_exp2f(m - muse);
            lsum *= corr;
            if constexpr (LSE) lex *= corr;
#pragma unroll
            for (int dh = 0; dh < 2; ++dh)
#pragma unroll
                for (int j = 0; j < 4; ++j) o[dh][j] *= corr;
        }
        m = mnew;

#pragma unroll
        for (int bq = 0; bq < S::BPC; bq += 2) {
            const int rA = bq / NCB, cbA = bq % NCB;
            const int rB = (bq + 1) / NCB, cbB = (bq + 1) % NCB;
            const int offA = (slot(c0, rA) * S::NC + 16 * cbA) * 64;
            const int offB = (slot(c0, rB) * S::NC + 16 * cbB) * 64;
            FragT vf[2];
#pragma unroll
            for (int dh = 0; dh < 2; ++dh) {
                lds_cu8 *vp = dh ? vp1 : vp0;
                const v4i16 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vp + offA));
                const v4i16 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vp + offB));
                const v8i16 vv = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                vf[dh] = __builtin_bit_cast(FragT, vv);
            }
            float p[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // exp2(c (q.k + B) - m)
                p[j] = __builtin_amdgcn_exp2f(kBiasAcc ? fmaf(sc[rA][cbA][j], a.c, -muse) : sc[rA][cbA][j] - muse);
                p[4 + j] =
                    __builtin_amdgcn_exp2f(kBiasAcc ? fmaf(sc[rB][cbB][j], a.c, -muse) : sc[rB][cbB][j] - muse);
            }
            if constexpr (__is_same(T, _Float16)) {
                half8 pf;
#pragma unroll
                for (int j = 0; j < 8; ++j) pf[j] = static_cast<_Float16>(p[j]);
                // the sum takes the rounded weights, so they sum to exactly what multiplies V
#pragma unroll
                for (int j = 0; j < 8; j += 2)
                    lsum = __builtin_amdgcn_fdot2(half2{pf[j], pf[j + 1]}, half2{1, 1}, lsum, false);
                if constexpr (LSE) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) lex += p[j];
                }
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
        if constexpr (!RING) {
            kp += RPC * S::NC * 64;
            vp0 += RPC * S::NC * 64;
            vp1 += RPC * S::NC * 64;
        }
        if constexpr (MODE == kClass) {
            bp += RPC * PC;  // the -inf strip is long enough for any chunk
        } else if constexpr (MODE == kInterior) {
            bp += RPC * P;
        }
    }
    if constexpr (LSE) {
        st.m = m;
        st.l = __is_same(T, _Float16) ? lex : lsum;
    }
}

// One wave's share of a tile: choose its candidate key rows and the bias
// path, leave o / lsum for stage_out (or scale_out).
template <typename T, int QY, int QX, int NCB, int RPC, int KS, int WM, bool CT = true, bool LSE = false,
          int RING = 0>
__device__ inline void attend_wave(const Args &a, const Tile &t, const unsigned char *smem,
                                   const float *btab, int lr, int wave, int lane,
                                   const typename Frag<T>::type &qf, floatx4 (&o)[2], float &lsum,
                                   SoftStats &st)
{
    using S = Shape<QY, QX, NCB, RPC, kWaves, CT>;
    const int ks = KS ? KS : a.ks, H = a.H, W = a.W, r = ks >> 1;
    const int nr = wave_rows(QY, RPC, ks);
    const int y1 = t.y0 + QY * wave;
    const int ry = wave_first_row<WM>(y1, ks, H, t.hy0, t.hr, nr);
    if constexpr (S::CLS) {
        attend<T, QY, QX, NCB, RPC, KS, kClass, WM, CT, LSE, RING>(a, t, smem, btab, lr, wave, ry, lane,
                                                               qf, o, lsum, st);
    } else {
        // no query window clamped (SASA windows never are), and the candidate
        // rows / columns start k/2 above / left of the subtile's first query
        const bool unclamped = WM == NA_WINDOW_SASA ||
                               (y1 - r >= 0 && y1 + QY - 1 + r <= H - 1 && t.x0 - r >= 0 &&
                                t.x0 + QX - 1 + r <= W - 1);
        const bool interior = unclamped && ry == y1 - r && t.cx == t.x0 - r;
        if (interior)
            attend<T, QY, QX, NCB, RPC, KS, kInterior, WM, CT, LSE, RING>(a, t, smem, btab, lr, wave, ry,
                                                                  lane, qf, o, lsum, st);
        else
            attend<T, QY, QX, NCB, RPC, KS, kGeneral, WM, CT, LSE, RING>(a, t, smem, btab, lr, wave, ry,
                                                                 lane, qf, o, lsum, st);
    }
}

// Writing one wave's 16 outputs (fp32, 2 KB) takes two steps.
//
// stage_out normalises the o fragments and puts them in memory order. The
// fragments pass through a 1 KB LDS area of the wave's own, in two rounds
// of 8 queries, and each lane keeps 16 bytes per round. In the fragments a
// query's 128-byte row is split over four lanes. Staged, one store
// instruction writes 8 whole rows instead of half of each of 16 rows, which
// takes the write path far fewer partial lines.
//
// Layout: chunk k (16 bytes) of a round's query j (0 .. 7) sits at chunk
// 8 j + (k ^ j). Any 8 consecutive lanes then touch 8 different 16-byte bank
// groups, both when writing (fixed k, j = 0 .. 7) and when reading (fixed j,
// k = 0 .. 7). Lanes of one wave trade data here, so the writes and reads
// are fenced against code motion.
//
// issue_out then issues the stores, non-temporal since nothing reads the
// output again. Out-of-map queries are dropped by the range check. With LSE,
// lane g == 0 of each query also writes ln(sum of exp(logits)) =
// (m + log2 sum) ln 2.
struct OutRegs {
    floatx4 v[2];  // chunk `lane` of rounds 0 and 1
    float lse;
};

__device__ inline int out_chunk(int j, int k) { return 8 * j + (k ^ j); }

template <bool LSE = false>
__device__ inline void stage_out(int lane, const floatx4 (&o)[2], float lsum, const SoftStats &st,
                                 float *stage, OutRegs &r)
{
    const int g = lane >> 4, qi = lane & 15;
    const float inv = __builtin_amdgcn_rcpf(quad_sum(lsum));
    if constexpr (LSE) r.lse = (st.m + __builtin_amdgcn_logf(quad_sum(st.l))) * 0.6931471805599453f;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        __builtin_amdgcn_wave_barrier();
        if ((qi >> 3) == round) {
#pragma unroll
            for (int dh = 0; dh < 2; ++dh)
                *reinterpret_cast<floatx4 *>(stage + 4 * out_chunk(qi & 7, 4 * dh + g)) = o[dh] * inv;
        }
        __builtin_amdgcn_wave_barrier();
        r.v[round] = *reinterpret_cast<const floatx4 *>(stage + 4 * out_chunk(lane >> 3, lane & 7));
    }
    __builtin_amdgcn_wave_barrier();
}

// Without an LDS area to spare (the LDS-DMA kernel, whose occupancy its LDS
// sets), the normalised fragments are stored as they are, with the default
// cache policy (measured as fast there): v[dh] holds dims 16 dh + 4 g .. + 3
// of query `lane & 15`.
template <bool LSE = false>
__device__ inline void scale_out(const floatx4 (&o)[2], float lsum, const SoftStats &st, OutRegs &r)
{
    const float inv = __builtin_amdgcn_rcpf(quad_sum(lsum));
    if constexpr (LSE) r.lse = (st.m + __builtin_amdgcn_logf(quad_sum(st.l))) * 0.6931471805599453f;
    r.v[0] = o[0] * inv;
    r.v[1] = o[1] * inv;
}

template <int QY, int QX, bool LSE = false, bool STAGED = true>
__device__ inline void issue_out(const Args &a, const Tile &t, int wave, int lane, const OutRegs &r)
{
    const __amdgpu_buffer_rsrc_t ro =
        map_rsrc(a.out, t.map_base, kD * 4, (unsigned)a.H * a.W * (kD * 4));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // staged: round i, chunk `lane`; else: query lane & 15, dims 16 i + 4 g ..
        const int q = STAGED ? 8 * i + (lane >> 3) : lane & 15;
        const unsigned col = STAGED ? 16u * (unsigned)(lane & 7) : 64u * i + 16u * (unsigned)(lane >> 4);
        const int y = t.y0 + QY * wave + q / QX;
        const int x = t.x0 + q % QX;
        const unsigned off = y < a.H && x < a.W ? (unsigned)(y * a.W + x) * 128u + col : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r.v[i]), ro, off, 0,
                                               STAGED ? kNonTemporal : 0);
    }
    if constexpr (LSE) {
        const int g = lane >> 4, qi = lane & 15;
        const int y = t.y0 + QY * wave + qi / QX;
        const int x = t.x0 + qi % QX;
        if (g == 0 && y < a.H && x < a.W) a.lse[t.map_base + (int64_t)y * a.W + x] = r.lse;
    }
}

// Persistent workgroups.  Workgroup w takes every G-th tile of its range (the
// whole tile list, or with xcd_split its XCD's eighth of it, so the
// workgroups sharing an L2 work on neighbouring tiles).  Per tile: attend,
// barrier, issue the next tile's copies, store this tile's outputs, wait,
// barrier.
template <typename T, int QY, int QX, int NCB, int RPC, int KS, int WM, bool CT, bool LSE = false>
__global__ __launch_bounds__(kThreads) void na2d_mfma_kernel(Args a)
{
    using S = Shape<QY, QX, NCB, RPC, kWaves, CT>;
    using FragT = typename Frag<T>::type;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = a.lr;
    const int ks = KS ? KS : a.ks;
    const int nr = wave_rows(QY, RPC, ks);

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

    float *bt = reinterpret_cast<float *>(smem + b_offset(lr, S::NC));
    FragT qf;
    Tile t = tile_geometry<S::TY, S::TX, S::NC, WM>(a, tile);
    int bias_head = t.h;
    stage_bias<QY, QX, S::NC, RPC, S::CLS>(a, ks, t.h, bt, reinterpret_cast<float *>(smem), nr, tid);
    stage_tile<T, QY, QX, NCB, RPC>(a, t, smem, lr, wave, lane, qf);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    while (true) {
        work_priority(end, tile, step);
        floatx4 o[2];
        float lsum;
        SoftStats st{0.f, 1.f};
        attend_wave<T, QY, QX, NCB, RPC, KS, WM, CT, LSE>(a, t, smem, bt, lr, wave, lane, qf, o, lsum, st);
        const Tile done = t;
        const unsigned next = tile + step;
        __syncthreads();  // every wave is done reading the LDS copy
        if (next < end) {
            t = tile_geometry<S::TY, S::TX, S::NC, WM>(a, next);
            if (t.h != bias_head) {  // rare: the tile list is head-major
                stage_bias<QY, QX, S::NC, RPC, S::CLS>(a, ks, t.h, bt, reinterpret_cast<float *>(smem), nr, tid);
                bias_head = t.h;
            }
            stage_tile<T, QY, QX, NCB, RPC>(a, t, smem, lr, wave, lane, qf);
        }
        OutRegs orr;
        scale_out<LSE>(o, lsum, st, orr);
        issue_out<QY, QX, LSE, false>(a, done, wave, lane, orr);
        if (next >= end) break;
        // loads and stores may retire out of order against each other, so
        // only an empty counter proves the copies have landed
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        tile = next;
    }
}

// Pipelined variant for a compile-time kernel size: while tile i is computed
// from LDS, tile i+1's K/V halo rows and queries are already loading into
// registers (plain buffer loads; out-of-map pixels return zeros), and are
// written to LDS between two barriers once tile i is done.  The loads are
// ordinary register loads, so the compiler's wait counts follow them exactly.
template <int QY, int QX, int NCB, int LR, int NW>
struct TileRegs {
    static constexpr int ROWS = (LR + NW - 1) / NW;  // halo rows per wave (at most)
    u32x4 k[ROWS][NCB], v[ROWS][NCB];
    u32x4 q;  // this lane's query fragment
};

// With `live` false every offset is out of range: the loads still issue (so
// the wait counts do not depend on it) but return zeros without touching memory.
template <typename T, int QY, int QX, int NCB, int RPC, int LR, int NW>
__device__ inline void load_tile_regs(const Args &a, const Tile &t, int wave, int lane,
                                      TileRegs<QY, QX, NCB, LR, NW> &rg, bool live = true)
{
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, t.map_base, kD * 2, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, t.map_base, kD * 2, map_bytes);
    const int c_lane = lane >> 2, slot = lane & 3;
#pragma unroll
    for (int j = 0; j < TileRegs<QY, QX, NCB, LR, NW>::ROWS; ++j) {
        const int r = wave + NW * j;
        const int gy = t.hy0 + r;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int c = 16 * cb + c_lane;
            const int sl = halo_slot(slot, c);
            const int gx = t.cx + c;
            const unsigned off =
                live && r < LR && (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W
                    ? (unsigned)(gy * a.W + gx) * 64u + 16u * sl
                    : kOutOfRange;
            rg.k[j][cb] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
            rg.v[j][cb] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
        }
    }
    const int g = lane >> 4, qi = lane & 15;
    const int y = min(t.y0 + QY * wave + qi / QX, a.H - 1);
    const int x = min(t.x0 + qi % QX, a.W - 1);
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, t.map_base, kD * 2, map_bytes);
    rg.q = __builtin_amdgcn_raw_buffer_load_b128(
        rq, live ? (unsigned)(y * a.W + x) * 64u + 16u * g : kOutOfRange, 0, kNonTemporal);
}

// the queries sit after the K and V halos: [wave][lane] 16-byte fragments
__host__ __device__ constexpr unsigned q_frag_offset(int lr, int nc) { return 2u * lr * nc * 64u; }

template <int QY, int QX, int NCB, int RPC, int LR, int NW>
__device__ inline void write_tile_regs(unsigned char *smem, int wave, int lane,
                                       const TileRegs<QY, QX, NCB, LR, NW> &rg)
{
    using S = Shape<QY, QX, NCB, RPC, NW>;
    *reinterpret_cast<u32x4 *>(smem + q_frag_offset(LR, S::NC) + (unsigned)(wave * 64 + lane) * 16u) = rg.q;
#pragma unroll
    for (int j = 0; j < TileRegs<QY, QX, NCB, LR, NW>::ROWS; ++j) {
        const int r = wave + NW * j;
        if (r < LR) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                unsigned char *dk = smem + (unsigned)(r * S::NC + 16 * cb) * 64u + 16u * lane;
                *reinterpret_cast<u32x4 *>(dk) = rg.k[j][cb];
                *reinterpret_cast<u32x4 *>(dk + halo_bytes(LR, S::NC)) = rg.v[j][cb];
            }
        }
    }
}

// The SASA variants compile to 128 VGPRs when held there, which fits four
// workgroups per CU instead of three: 1.5 us faster at stage 1. The NA
// variants would spill at that bound.
template <typename T, int QY, int QX, int NCB, int RPC, int KS, int NW, int WM, bool CT, bool LSE = false>
__global__ __launch_bounds__(64 * NW, WM == NA_WINDOW_SASA ? 4 : 1) void na2d_mfma_pipe_kernel(Args a)
{
    using S = Shape<QY, QX, NCB, RPC, NW, CT>;
    using FragT = typename Frag<T>::type;
    constexpr int NR = wave_rows(QY, RPC, KS);
    constexpr int LR = S::TY + KS - 1 > NR ? S::TY + KS - 1 : NR;
    constexpr unsigned HB = 2u * LR * S::NC * 64u + S::NT * 16u;  // K, V halos and queries
    constexpr unsigned BF = bias_floats(S::CLS, KS, NR, QY, QX, S::NC, RPC);
    __shared__ __align__(16) unsigned char halo[HB];
    __shared__ __align__(16) float btab[BF];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar code and branches

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

    // Prologue: the bias table and the first tile are in flight together.
    // The second tile's loads are issued only once the first tile is in LDS:
    // every workgroup starts at once, and a CU serves its workgroups' loads
    // in the order they were issued, so the second tile of the first
    // workgroups on a CU would otherwise arrive before the first tile of the
    // last one (measured -0.2 to -0.4 us at NAT-Tiny stage 1).
    constexpr int NV = raw_per_thread(KS, S::NT);
    TileRegs<QY, QX, NCB, LR, NW> rg0, rg;
    Tile t = tile_geometry<S::TY, S::TX, S::NC, WM>(a, tile);
    int bias_head = t.h;
    float raw_bias[NV];
    load_raw_bias<S::NT>(a, KS, t.h, tid, raw_bias);
    load_tile_regs<T, QY, QX, NCB, RPC, LR>(a, t, wave, lane, rg0);
    unsigned next = tile + step;
    Tile tn = tile_geometry<S::TY, S::TX, S::NC, WM>(a, next < end ? next : tile);
    // the halo area is free until the first tile is written into it
    stage_bias<QY, QX, S::NC, RPC, S::CLS, S::NT>(a, KS, raw_bias, btab,
                                                  reinterpret_cast<float *>(halo), NR, tid);
    write_tile_regs<QY, QX, NCB, RPC, LR>(halo, wave, lane, rg0);
    __syncthreads();
    load_tile_regs<T, QY, QX, NCB, RPC, LR>(a, tn, wave, lane, rg, next < end);
    const auto *qfrag = reinterpret_cast<const u32x4 *>(halo + q_frag_offset(LR, S::NC)) + tid;
    // a wave's query fragments (1 KB) are read by that wave alone, at the top
    // of attend, so the area doubles as the wave's output staging area
    float *ostage = reinterpret_cast<float *>(halo + q_frag_offset(LR, S::NC)) + 256 * wave;
    while (true) {
        work_priority(end, tile, step);
        // attend from LDS; the next tile is loading into `rg` meanwhile
        floatx4 o[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
        float lsum = 1.f;
        SoftStats st{0.f, 1.f};
        if (t.y0 + QY * wave < a.H) {  // the bottom tile row may leave whole waves idle
            const FragT qf = __builtin_bit_cast(FragT, *qfrag);
            attend_wave<T, QY, QX, NCB, RPC, KS, WM, CT, LSE>(a, t, halo, btab, LR, wave, lane, qf, o,
                                                              lsum, st);
        }
        const Tile done = t;
        const bool more = next < end;
        OutRegs orr;
        stage_out<LSE>(lane, o, lsum, st, ostage, orr);
        __syncthreads();  // every wave is done reading the halo (and the bias table)
        if (more) {
            if (tn.h != bias_head) {  // rare: the tile list is head-major
                stage_bias<QY, QX, S::NC, RPC, S::CLS, S::NT>(a, KS, tn.h, btab,
                                                              reinterpret_cast<float *>(halo), NR,
                                                              tid);
                bias_head = tn.h;
            }
            // everything outstanding -- `rg` and the previous tile's stores --
            // was issued a whole tile earlier, so an empty counter costs little
            // (loads and stores may retire out of order, so nothing less will do)
            __builtin_amdgcn_s_waitcnt(0);
            write_tile_regs<QY, QX, NCB, RPC, LR>(halo, wave, lane, rg);
        }
        issue_out<QY, QX, LSE>(a, done, wave, lane, orr);
        if (!more) break;
        t = tn;
        tile = next;
        next = tile + step;
        if (next < end) {
            tn = tile_geometry<S::TY, S::TX, S::NC, WM>(a, next);
            load_tile_regs<T, QY, QX, NCB, RPC, LR>(a, tn, wave, lane, rg);
        }
        __syncthreads();  // the new halo is visible
    }
}

// Column-run variant for a compile-time kernel size (8 x 8 tiles of 2 x 8
// subtiles, one 16-column block).  A workgroup walks a run of tiles down one
// tile column of one map.  Consecutive tiles' halos overlap by all but at
// most TY rows, so the halo lives in a ring of kRing LDS rows -- map row gy
// at slot gy & (kRing - 1) -- and each step loads only the rows that enter
// it (8 of 14 in the interior), into registers while the previous tile is
// computed.  The first tile of the run is copied HBM -> LDS directly.
// One run per workgroup; the launch makes the runs as long as it must for
// all of them to be resident at once.
constexpr int kRing = 16;

template <int QY, int QX, int NW>
struct RingRegs {
    u32x4 k[QY], v[QY];  // QY = TY / NW rows per wave
    u32x4 q;             // this lane's query fragment
};

// Issue the loads of the rows [lo, hi) that enter tile t's halo (hi - lo <=
// TY), wave w taking rows lo + w, lo + w + NW, ...; rows past the range, the
// map or the tile's columns load as zeros.  Also the tile's query fragment.
template <int QY, int QX, int NW>
__device__ inline void load_ring_rows(const Args &a, const Tile &t, int lo, int hi, int wave, int lane,
                                      RingRegs<QY, QX, NW> &rg)
{
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, t.map_base, kD * 2, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, t.map_base, kD * 2, map_bytes);
    const int c_lane = lane >> 2, slot = lane & 3;
    const int sl = halo_slot(slot, c_lane);
    const int gx = t.cx + c_lane;
#pragma unroll
    for (int j = 0; j < QY; ++j) {
        const int gy = lo + wave + NW * j;
        const unsigned off = gy < hi && (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W
                                 ? (unsigned)(gy * a.W + gx) * 64u + 16u * sl
                                 : kOutOfRange;
        rg.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        rg.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
    const int g = lane >> 4, qi = lane & 15;
    const int y = min(t.y0 + QY * wave + qi / QX, a.H - 1);
    const int x = min(t.x0 + qi % QX, a.W - 1);
    const __amdgpu_buffer_rsrc_t rq = map_rsrc(a.q, t.map_base, kD * 2, map_bytes);
    rg.q = __builtin_amdgcn_raw_buffer_load_b128(rq, (unsigned)(y * a.W + x) * 64u + 16u * g, 0, kNonTemporal);
}

// Write the rows [lo, hi) loaded by load_ring_rows into their ring slots.
template <int QY, int QX, int NW>
__device__ inline void write_ring_rows(unsigned char *halo, int lo, int hi, int wave, int lane,
                                       const RingRegs<QY, QX, NW> &rg)
{
#pragma unroll
    for (int j = 0; j < QY; ++j) {
        const int gy = lo + wave + NW * j;
        if (gy < hi) {
            unsigned char *dk = halo + (unsigned)((gy & (kRing - 1)) * 16) * 64u + 16u * lane;
            *reinterpret_cast<u32x4 *>(dk) = rg.k[j];
            *reinterpret_cast<u32x4 *>(dk + halo_bytes(kRing, 16)) = rg.v[j];
        }
    }
}

// Copy tile t's whole halo (rows hy0 .. hy0 + lr - 1, past the map zeros)
// HBM -> LDS into the ring.
template <int NW>
__device__ inline void stage_ring_full(const Args &a, const Tile &t, unsigned char *halo, int lr,
                                       int wave, int lane)
{
    const unsigned map_bytes = (unsigned)a.H * a.W * (kD * 2);
    const __amdgpu_buffer_rsrc_t rk = map_rsrc(a.k, t.map_base, kD * 2, map_bytes);
    const __amdgpu_buffer_rsrc_t rv = map_rsrc(a.v, t.map_base, kD * 2, map_bytes);
    const int c_lane = lane >> 2, slot = lane & 3;
    const int sl = halo_slot(slot, c_lane);
    const int gx = t.cx + c_lane;
    for (int r = wave; r < lr; r += NW) {
        const int gy = t.hy0 + r;
        const unsigned off = (unsigned)gy < (unsigned)a.H && (unsigned)gx < (unsigned)a.W
                                 ? (unsigned)(gy * a.W + gx) * 64u + 16u * sl
                                 : kOutOfRange;
        unsigned char *dk = halo + (unsigned)((gy & (kRing - 1)) * 16) * 64u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)dk, 16, off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(dk + halo_bytes(kRing, 16)), 16, off,
                                                 0, 0, 0);
    }
}

template <typename T, int KS, int WM, bool LSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void
na2d_mfma_ring_kernel(Args a)
{
    constexpr int QY = 2, QX = 8, NCB = 1, RPC = 8, NW = kWaves;
    using S = Shape<QY, QX, NCB, RPC, NW, false>;
    using FragT = typename Frag<T>::type;
    constexpr int NR = wave_rows(QY, RPC, KS);
    constexpr int LR = halo_lds_rows(S::TY, QY, RPC, KS);  // rows a tile's halo needs
    static_assert(LR < kRing && S::NC == 16, "ring shape");
    constexpr unsigned BF = bias_floats(false, KS, NR, QY, QX, S::NC, RPC);
    __shared__ __align__(16) unsigned char halo[2 * kRing * 16 * 64];  // K ring, then V ring
    __shared__ __align__(16) float btab[BF];
    __shared__ __align__(16) float ostage_all[NW * 256];  // 1 KB of output staging per wave
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float *ostage = ostage_all + 256 * wave;

    const unsigned run = xcd_tile(blockIdx.x, gridDim.x);
    if (run >= a.nruns) return;
    const int col = (int)(run / (unsigned)a.runs_per_col);
    const int part = (int)run - col * a.runs_per_col;
    const int ty0 = part * a.run_len, ty1 = min(a.tiles_y, ty0 + a.run_len);
    if (ty0 >= ty1) return;
    const int mapi = col / a.tiles_x, tx = col - mapi * a.tiles_x;  // mapi = h * B + b
    auto tile_at = [&](int ty) {
        return tile_geometry<S::TY, S::TX, S::NC, WM>(a, (unsigned)((mapi * a.tiles_y + ty) * a.tiles_x + tx));
    };

    Tile t = tile_at(ty0);
    {
        constexpr int NV = raw_per_thread(KS, S::NT);
        float raw_bias[NV];
        load_raw_bias<S::NT>(a, KS, t.h, tid, raw_bias);
        stage_bias<QY, QX, S::NC, RPC, false, S::NT>(a, KS, raw_bias, btab,
                                                     reinterpret_cast<float *>(halo), NR, tid);
    }
    stage_ring_full<NW>(a, t, halo, LR, wave, lane);
    RingRegs<QY, QX, NW> rg;
    Tile tn = t;
    int nlo = 0, nhi = 0;  // rows entering the next tile's halo
    FragT qf;
    {
        const int g = lane >> 4, qi = lane & 15;
        const int y = min(t.y0 + QY * wave + qi / QX, a.H - 1);
        const int x = min(t.x0 + qi % QX, a.W - 1);
        const __amdgpu_buffer_rsrc_t rq =
            map_rsrc(a.q, t.map_base, kD * 2, (unsigned)a.H * a.W * (kD * 2));
        qf = __builtin_bit_cast(
            FragT, __builtin_amdgcn_raw_buffer_load_b128(rq, (unsigned)(y * a.W + x) * 64u + 16u * g, 0, kNonTemporal));
    }
    // loads and stores may retire out of order against each other, so only an
    // empty counter proves the copies have landed; the next tile's rows are
    // asked for only then, so that the first halo arrives alone
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ty0 + 1 < ty1) {
        tn = tile_at(ty0 + 1);
        const RowRange e = ring_entering(t.hy0, tn.hy0, LR);
        nlo = e.lo;
        nhi = e.hi;
        load_ring_rows<QY, QX, NW>(a, tn, nlo, nhi, wave, lane, rg);
    }
    for (int ty = ty0;;) {
        work_priority((unsigned)ty1, (unsigned)ty, 1u);
        floatx4 o[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
        float lsum = 1.f;
        SoftStats st{0.f, 1.f};
        if (t.y0 + QY * wave < a.H)  // the bottom tile row may leave whole waves idle
            attend_wave<T, QY, QX, NCB, RPC, KS, WM, false, LSE, kRing>(a, t, halo, btab, kRing, wave,
                                                                        lane, qf, o, lsum, st);
        const Tile done = t;
        const bool more = ty + 1 < ty1;
        OutRegs orr;
        stage_out<LSE>(lane, o, lsum, st, ostage, orr);
        __syncthreads();  // every wave is done reading the ring
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);
            write_ring_rows<QY, QX, NW>(halo, nlo, nhi, wave, lane, rg);
            qf = __builtin_bit_cast(FragT, rg.q);
        }
        issue_out<QY, QX, LSE>(a, done, wave, lane, orr);
        if (!more) break;
        t = tn;
        ++ty;
        if (ty + 1 < ty1) {
            tn = tile_at(ty + 1);
            const RowRange e = ring_entering(t.hy0, tn.hy0, LR);
            nlo = e.lo;
            nhi = e.hi;
            load_ring_rows<QY, QX, NW>(a, tn, nlo, nhi, wave, lane, rg);
        }
        __syncthreads();  // the entering rows are visible
    }
}

// Arguments and tile counts for a tile shape S; false if the tile list does
// not fit 32 bits.
template <typename S, int QY, int RPC>
bool make_args(const Problem &p, Args &a)
{
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
    a.tiles_x = (p.W + S::TX - 1) / S::TX;
    a.tiles_y = (p.H + S::TY - 1) / S::TY;
    const uint64_t ntiles = (uint64_t)p.B * p.heads * a.tiles_x * a.tiles_y;
    if (ntiles == 0 || ntiles > 0x7fffffffull) return false;
    a.ntiles = (unsigned)ntiles;
    a.lr = halo_lds_rows(S::TY, QY, RPC, p.ksize);
    a.c = 1.4426950408889634f / sqrtf((float)kD);
    return true;
}

// One workgroup per resident slot (measured faster than fewer, evenly loaded
// workgroups: the memory system wants every slot's loads in flight), each
// XCD given its own contiguous tile range when there are enough workgroups.
template <typename K>
hipError_t launch_persistent(K kern, Args &a, int threads, size_t lds, hipStream_t stream,
                             bool flat = false)
{
    int per_cu = 0;
    const hipError_t e = occupancy(reinterpret_cast<const void *>(kern), threads, lds, per_cu);
    if (e != hipSuccess) return e;
    const int cus = device_cus();
    if (per_cu <= 0 || cus <= 0) return hipErrorInvalidConfiguration;
    uint64_t grid = (uint64_t)cus * per_cu;
    if (flat || grid > a.ntiles) grid = a.ntiles;  // flat: one tile per workgroup
    a.xcd_split = 0;
    if (grid >= 64) {
        grid = flat ? (grid + 7) & ~7ull : grid & ~7ull;
        a.xcd_split = 1;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, stream, a);
    return hipGetLastError();
}

// General kernel sizes: the LDS-DMA kernel with 4 waves per workgroup.
template <typename T, int QY, int QX, int NCB, int RPC, int WM, bool LSE, bool CT = true, bool FLAT = false>
hipError_t launch_dma(const Problem &p, hipStream_t stream)
{
    using S = Shape<QY, QX, NCB, RPC, kWaves, CT>;
    Args a;
    if (!make_args<S, QY, RPC>(p, a)) return hipErrorInvalidConfiguration;
    const int nr = wave_rows(QY, RPC, p.ksize);
    const size_t lds =
        lds_bytes(a.lr, S::NC, bias_floats(S::CLS, p.ksize, nr, QY, QX, S::NC, RPC));
    return launch_persistent(na2d_mfma_kernel<T, QY, QX, NCB, RPC, 0, WM, CT, LSE>, a, S::NT, lds,
                             stream, FLAT);
}

// A compile-time kernel size: the register-prefetch kernel with NW waves.
template <typename T, int QY, int QX, int NCB, int RPC, int KS, int NW, int WM, bool LSE, bool CT = true>
hipError_t launch_pipe(const Problem &p, hipStream_t stream)
{
    using S = Shape<QY, QX, NCB, RPC, NW, CT>;
    Args a;
    if (!make_args<S, QY, RPC>(p, a)) return hipErrorInvalidConfiguration;
    return launch_persistent(na2d_mfma_pipe_kernel<T, QY, QX, NCB, RPC, KS, NW, WM, CT, LSE>, a, S::NT,
                             0, stream);
}

// The column-run kernel: runs as short as they can be while every run of the
// launch fits in the resident workgroup slots at once (one run per
// workgroup), each XCD taking a contiguous stretch of runs.
// Returns hipErrorNotReady, launching nothing, when the runs would be 2 to 7
// tiles long: there the persistent register-prefetch kernel measured faster
// (NAT-Tiny stage 1: 21.9 against 23.3 us; at 448^2, runs of 14 tiles, the
// ring kernel takes 68 against 73 us, and with one-tile runs 9.4 against
// 10.2 us at stage 3).
template <typename T, int KS, int WM, bool LSE>
hipError_t launch_ring(const Problem &p, hipStream_t stream)
{
    using S = Shape<2, 8, 1, 8, kWaves, false>;
    Args a;
    if (!make_args<S, 2, 8>(p, a)) return hipErrorInvalidConfiguration;
    const auto kern = na2d_mfma_ring_kernel<T, KS, WM, LSE>;
    int per_cu = 0;
    const hipError_t e = occupancy(reinterpret_cast<const void *>(kern), kThreads, 0, per_cu);
    if (e != hipSuccess) return e;
    const int cus = device_cus();
    if (per_cu <= 0 || cus <= 0) return hipErrorInvalidConfiguration;
    const uint64_t slots = (uint64_t)cus * per_cu;
    const uint64_t cols = (uint64_t)p.B * p.heads * a.tiles_x;
    int len = 1;
    while (len < a.tiles_y && cols * ((a.tiles_y + len - 1) / len) > slots) ++len;
    if (len > 1 && len < 8) return hipErrorNotReady;
    a.run_len = len;
    a.runs_per_col = (a.tiles_y + len - 1) / len;
    const uint64_t runs = cols * a.runs_per_col;
    if (xcd_grid(runs) > 0x7fffffffull) return hipErrorInvalidConfiguration;
    a.nruns = (unsigned)runs;
    hipLaunchKernelGGL(kern, dim3((unsigned)xcd_grid(runs)), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int WM, bool LSE>
hipError_t launch_typed(const Problem &p, hipStream_t stream)
{
    const int ks = p.ksize;
    if (ks == 7) {
        const hipError_t e = launch_ring<T, 7, WM, LSE>(p, stream);
        return e == hipErrorNotReady ? launch_pipe<T, 2, 8, 1, 8, 7, 4, WM, LSE, false>(p, stream) : e;
    }
    if (ks <= 9) return launch_dma<T, 2, 8, 1, 2, WM, LSE>(p, stream);
    if (ks <= 13) return launch_dma<T, 4, 4, 1, 8, WM, LSE>(p, stream);
    return launch_dma<T, 2, 8, 2, 2, WM, LSE>(p, stream);
}

// The log-sum-exp output exists for NA windows only (it feeds the NA2D backward).
template <typename T>
hipError_t launch_mode(const Problem &p, hipStream_t stream)
{
    if (p.mode == NA_WINDOW_SASA)
        return p.lse ? hipErrorInvalidValue : launch_typed<T, NA_WINDOW_SASA, false>(p, stream);
    return p.lse ? launch_typed<T, NA_WINDOW_NA, true>(p, stream)
                 : launch_typed<T, NA_WINDOW_NA, false>(p, stream);
}

}  // namespace

long long occupancy_queries() { return g_occ_queries.load(); }

hipError_t launch_mfma(const Problem &p, hipStream_t stream)
{
    if (p.d != kD || p.ksize < 3 || p.ksize > NA2D_MFMA_MAX_KSIZE) return hipErrorInvalidValue;
    // byte offsets inside one map are 32-bit (buffer addressing)
    if ((uint64_t)p.H * p.W * (kD * 4) > 0x7fffffffull) return hipErrorInvalidValue;
    if (p.depth != 1 || p.kd != 1 || p.kh != p.kw) return hipErrorInvalidValue;
    if (p.dtype == NA2D_F16) return launch_mode<_Float16>(p, stream);
    if (p.dtype == NA2D_BF16) return launch_mode<__bf16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace na2d
