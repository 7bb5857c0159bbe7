// na_geometry.h -- where the matrix-core NA2D forward kernels put a query
// tile's keys: window starts, the LDS halo of a tile, each wave's candidate
// rows, the ring of the column-run kernel, and the block grid and bias-table
// indexing of the wide-window kernel.
//
// These are host/device functions so that the same arithmetic the kernels
// run can be enumerated on the CPU over window sizes, map sizes and tile
// origins (the geometry test checks that every window a tile needs lies in
// what the tile stages, and that every bias read lands on the right entry).
//
// The window is Neighborhood Attention's ("Neighborhood Attention
// Transformer", CSDN translation, section 3.1): the k nearest pixels of a
// query on each axis, start = clamp(i - k/2, 0, L - k); or, for SASA, the
// window centred on the query over the zero-padded map.
#pragma once

#include <hip/hip_runtime.h>

#include "na2d.h"

namespace na2d {

// Start of the window of ks pixels around i on an axis of length L: for NA
// (WM = NA_WINDOW_NA) the ks nearest pixels, pushed inward at the borders;
// for SASA (NA_WINDOW_SASA) the window centred on i, reaching into the zero
// padding past either end.
template <int WM>
__host__ __device__ inline int window_start(int i, int ks, int L)
{
    int s = i - (ks >> 1);
    if constexpr (WM == NA_WINDOW_NA) {
        s = s < 0 ? 0 : s;
        s = s > L - ks ? L - ks : s;
    }
    return s;
}

// ---- halo kernels (na2d_mfma.hip): tiles of TY x TX queries, waves of QY
// query rows, halos of NC columns

// Rows of candidate keys per wave: QY + ks - 1 rounded up to whole chunks
// of RPC rows.
__host__ __device__ constexpr int wave_rows(int QY, int RPC, int ks)
{
    const int n = QY + ks - 1;
    return (n + RPC - 1) / RPC * RPC;
}

// Halo rows held in LDS: the tile's TY + ks - 1 rows, or a wave's candidate
// rows if those are more.
__host__ __device__ constexpr int halo_lds_rows(int TY, int QY, int RPC, int ks)
{
    return TY + ks - 1 > wave_rows(QY, RPC, ks) ? TY + ks - 1 : wave_rows(QY, RPC, ks);
}

// The halo of the tile whose first query is (y0, x0): rows [hy0, hy0 + hr)
// hold every window of the tile's rows (LDS holds halo_lds_rows >= hr rows,
// the ones past the map zero-filled); columns [cx, cx + NC) hold the
// windows of columns x0 .. x0 + TX - 1. SASA windows are centred, so the
// halo is too; its rows and columns past the map are the zero padding.
struct HaloGeom {
    int hy0, hr, cx;
};

template <int TY, int NC, int WM>
__host__ __device__ inline HaloGeom halo_geometry(int y0, int x0, int ks, int H, int W)
{
    HaloGeom g;
    if constexpr (WM == NA_WINDOW_SASA) {
        g.hr = TY + ks - 1;
        g.hy0 = y0 - (ks >> 1);
        g.cx = x0 - (ks >> 1);
    } else {
        g.hr = TY + ks - 1 < H ? TY + ks - 1 : H;
        const int s = window_start<WM>(y0, ks, H);
        g.hy0 = s < H - g.hr ? s : H - g.hr;
        const int sx = window_start<WM>(x0, ks, W);
        g.cx = W >= NC ? (sx < W - NC ? sx : W - NC) : 0;
    }
    return g;
}

// First candidate key row of the wave whose first query row is y1: its
// first query's window start, kept inside the halo so that the nr candidate
// rows are halo rows.
template <int WM>
__host__ __device__ inline int wave_first_row(int y1, int ks, int H, int hy0, int hr, int nr)
{
    const int s = window_start<WM>(y1 < H - 1 ? y1 : H - 1, ks, H);
    const int top = hy0 + hr - nr;
    const int r = s < top ? s : top;
    return r > hy0 ? r : hy0;
}

// Column-run kernel: consecutive tiles of a run share all but the rows that
// enter; with a halo of lr rows starting at hy0 (this tile) and hy0n (the
// next), the rows [lo, hi) entering the next halo.
struct RowRange {
    int lo, hi;
};
__host__ __device__ inline RowRange ring_entering(int hy0, int hy0n, int lr)
{
    RowRange r;
    r.lo = hy0 + lr > hy0n ? hy0 + lr : hy0n;
    r.hi = hy0n + lr;
    return r;
}

// ---- wide-window kernel (na2d_large_mfma.hip): tiles of four waves of 4 x 4
// queries, WX waves across (8 x 8 tiles for WX = 2, 4 x 16 for WX = 4), keys
// in 4 x 4 blocks

constexpr int kLargeMaxBlocks = 8;  // block columns staged per block row (ksize <= 25)

// The bias tables (unscaled: the bias enters the QK product's accumulator).
//  - `col`: rows for key-minus-query row offsets dy in [-(k-1), k-1], then a
//    -inf row; columns for column offsets dx in [-X, X + 3], X = k/2 + 6:
//    the bias where |dx| <= k/2, else -inf. It serves every wave whose
//    queries' windows are not clamped on the column axis: a query's window
//    columns are then exactly |dx| <= k/2, and a key row outside its window
//    reads the -inf row. Such a wave's blocks reach k/2 + 6 columns past its
//    queries (the subtile spans 3, and the block grid, aligned to the
//    tile's union, may start up to 3 before the subtile's own), and the
//    blocks a row reads past the wave's last one 3 further.
//    Its pitch is 4 mod 8, so that the 28 entries a wave reads at once (7
//    row offsets x 4 column offsets) fall in 28 different banks.
//  - `raw`: the (2k-1)^2 table, then a -inf row long enough for any column a
//    row reads (the columns past a window reach 2k + 7), for waves clamped
//    on the column axis, which mask by each query's window (`cmask`).
__host__ __device__ constexpr int col_extent(int ks) { return (ks >> 1) + 6; }
__host__ __device__ constexpr int col_pitch(int ks)
{
    return (2 * col_extent(ks) + 4 + 3) / 8 * 8 + 4;  // >= the 2X + 4 columns, = 4 mod 8
}
__host__ __device__ constexpr int col_floats(int ks) { return 2 * ks * col_pitch(ks); }
__host__ __device__ constexpr int raw_floats(int ks) { return (2 * ks - 1) * (2 * ks - 1) + 2 * ks + 16; }
// the raw table starts kRawPad floats into its LDS area: a row's first
// columns may lie a few entries before a table row (they are masked, but read)
constexpr int kRawPad = 4;
// The column mask of a wave whose windows are clamped on the column axis:
// entry kMaskPad + i is 0 for window column i in [0, ksize), else -inf, for
// i from the first column of the wave's blocks (at most 6 before a window's
// first: 3 from aligning the blocks, 3 across the subtile) to its last
// (4 kLargeMaxBlocks - 1 past a window's first at most).
constexpr int kMaskPad = 8;
constexpr int kMaskFloats = kMaskPad + 4 * kLargeMaxBlocks;

// Source of `col` entry u: the index into the head's (2k-1)^2 table, or -1
// for -inf.
__host__ __device__ inline int col_entry_source(int u, int ks)
{
    const int nb = 2 * ks - 1, r = ks >> 1, P = col_pitch(ks), X = col_extent(ks);
    const int row = u / P, dx = u - row * P - X;
    return row >= nb || dx < -r || dx > r ? -1 : row * nb + dx + ks - 1;
}

// The union of the windows of the TY x TX tile whose first query is (y0,
// x0): key rows from uy0 and columns from ux0, nbr x nbc blocks of 4 x 4 keys.
struct LargeTileGeom {
    int uy0, ux0, nbr, nbc;
};
__host__ __device__ inline LargeTileGeom large_tile_geometry(int y0, int x0, int TY, int TX, int ks, int H, int W)
{
    LargeTileGeom g;
    g.uy0 = window_start<NA_WINDOW_NA>(y0, ks, H);
    g.ux0 = window_start<NA_WINDOW_NA>(x0, ks, W);
    const int yl = y0 + TY - 1 < H - 1 ? y0 + TY - 1 : H - 1;
    const int xl = x0 + TX - 1 < W - 1 ? x0 + TX - 1 : W - 1;
    const int uy1 = window_start<NA_WINDOW_NA>(yl, ks, H) + ks;
    const int ux1 = window_start<NA_WINDOW_NA>(xl, ks, W) + ks;
    g.nbr = (uy1 - g.uy0 + 3) >> 2;
    g.nbc = (ux1 - g.ux0 + 3) >> 2;
    return g;
}

// Query c (row-major in its 4 x 4 subtile) of wave `wave` of the tile whose
// first query is (y0, x0), before clamping to the map: the wave's loads, its
// stores and large_wave_geometry all use this placement.
struct QueryPos {
    int y, x;
};
__host__ __device__ inline QueryPos large_query(int y0, int x0, int wave, int WX, int c)
{
    QueryPos q;
    q.y = y0 + 4 * (wave / WX) + (c >> 2);
    q.x = x0 + 4 * (wave % WX) + (c & 3);
    return q;
}

// Wave w of the tile: the 4 x 4 subtile (w / WX, w % WX); its block rows
// [rb0, rb1] and columns [cb0, cb0 + ncb) of the tile's union; colclamp:
// some query's window is pushed in on the column axis.
struct LargeWaveGeom {
    bool active, colclamp;
    int ya, xa;  // first query of the subtile
    int rb0, rb1, cb0, ncb;
};
__host__ __device__ inline LargeWaveGeom large_wave_geometry(const LargeTileGeom &t, int y0, int x0, int wave,
                                                             int WX, int ks, int H, int W)
{
    const int r = ks >> 1;
    LargeWaveGeom w;
    const QueryPos first = large_query(y0, x0, wave, WX, 0);
    w.ya = first.y;
    w.xa = first.x;
    w.active = w.ya < H && w.xa < W;
    const int yf = w.ya < H - 1 ? w.ya : H - 1, xf = w.xa < W - 1 ? w.xa : W - 1;
    const int yl = w.ya + 3 < H - 1 ? w.ya + 3 : H - 1, xl = w.xa + 3 < W - 1 ? w.xa + 3 : W - 1;
    w.rb0 = (window_start<NA_WINDOW_NA>(yf, ks, H) - t.uy0) >> 2;
    w.rb1 = (window_start<NA_WINDOW_NA>(yl, ks, H) + ks - 1 - t.uy0) >> 2;
    w.cb0 = (window_start<NA_WINDOW_NA>(xf, ks, W) - t.ux0) >> 2;
    w.ncb = ((window_start<NA_WINDOW_NA>(xl, ks, W) + ks - 1 - t.ux0) >> 2) - w.cb0 + 1;
    w.colclamp = !(w.xa - r >= 0 && xl + r <= W - 1 && w.xa + 3 < W);
    return w;
}

// Lane c (query c of the subtile, row-major) of the wave: its query, its
// window's first row, the first column of the wave's blocks minus its
// window's first (cxw), and its bias column base in `col` or `raw`.
struct LargeLaneGeom {
    int qy, qx, sy, cxw, bcol;
};
__host__ __device__ inline LargeLaneGeom large_lane_geometry(const LargeTileGeom &t, const LargeWaveGeom &w, int c,
                                                             int ks, int H, int W)
{
    LargeLaneGeom l;
    l.qy = w.ya + (c >> 2) < H - 1 ? w.ya + (c >> 2) : H - 1;
    l.qx = w.xa + (c & 3) < W - 1 ? w.xa + (c & 3) : W - 1;
    l.sy = window_start<NA_WINDOW_NA>(l.qy, ks, H);
    const int kx0 = t.ux0 + 4 * w.cb0;  // first key column of the wave's blocks
    l.cxw = kx0 - window_start<NA_WINDOW_NA>(l.qx, ks, W);
    l.bcol = w.colclamp ? kx0 - l.qx + ks - 1 : kx0 - l.qx + col_extent(ks);
    return l;
}

// Row base (in floats) of the bias of key row ky for a query in row qy
// whose window starts at row sy: in
// `raw` (colclamp) or `col`; a key row outside the window reads a -inf row.
__host__ __device__ inline int large_bias_row(bool colclamp, int ky, int qy, int sy, int ks)
{
    const int nb = 2 * ks - 1;
    const bool rowin = (unsigned)(ky - sy) < (unsigned)ks;
    if (colclamp) return rowin ? (ky - qy + ks - 1) * nb : nb * nb;
    return (rowin ? ky - qy + ks - 1 : nb) * col_pitch(ks);
}

}  // namespace na2d
