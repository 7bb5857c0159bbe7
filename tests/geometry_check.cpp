// geometry_check.cpp -- enumerates the matrix-core forward kernels' tile
// geometry (vision_sliding_window_amd/csrc/na_geometry.h, the functions the
// kernels call) over window sizes, map sizes and tile origins, and checks:
//
//  halo kernels (each shape the launcher uses, NA and SASA windows):
//   - every window row of a tile lies in the tile's halo rows, which lie in
//     the map (NA) and in the LDS rows;
//   - every window column of a tile lies in its NC-column halo, which lies
//     in the map when the map is at least NC wide (else it starts at 0);
//   - each wave's candidate rows hold its queries' windows and lie in the
//     LDS halo;
//   - the column-run kernel's ring of 16 rows: a tile's halo fits, and after
//     each step (rows entering the next halo written to slot row & 15) every
//     row a wave reads sits in its slot;
//  wide-window kernel (8 x 8 tiles, and 4 x 16 tiles up to k = 17):
//   - the tile's block grid stages at most kLargeMaxBlocks block columns, and
//     each wave's block rows and columns hold its queries' windows;
//   - the row kind the kernel dispatches (blocks per row, clamped or not)
//     has room for the wave's blocks;
//   - every bias read lands on the bias of that key-minus-query offset when
//     the key is in the query's window, and on -inf (table or column mask)
//     when it is not, including the repeated blocks of a short row; every
//     table and mask index is inside its LDS area.
//
// Windows follow "Neighborhood Attention Transformer" (CSDN translation,
// section 3.1): start = clamp(i - k/2, 0, L - k); SASA windows are centred.
//
// Prints "ok <checks>" and exits 0, or prints the first failures and exits 1.
#include "na_geometry.h"

#include <cstdio>
#include <vector>

using namespace na2d;

static long g_checks = 0, g_fails = 0;

#define CHECK(cond, ...)                                                 \
    do {                                                                 \
        ++g_checks;                                                      \
        if (!(cond)) {                                                   \
            if (g_fails++ < 20) {                                        \
                std::printf("FAIL (line %d, %s): ", __LINE__, #cond);    \
                std::printf(__VA_ARGS__);                                \
                std::printf("\n");                                       \
            }                                                            \
        }                                                                \
    } while (0)

static std::vector<int> axis_lengths(int k, bool sasa)
{
    std::vector<int> v;
    for (int L = sasa ? 1 : k; L <= k + 40; ++L) v.push_back(L);
    for (int L : {56, 64, 100, 128, 224})
        if (L > k + 40) v.push_back(L);
    return v;
}

static int imin(int a, int b) { return a < b ? a : b; }

// ---- halo kernels

template <int QY, int QX, int NCB, int RPC, int NW, int WM>
static void check_halo_shape(const char *name, int kmin, int kmax)
{
    constexpr int TY = QY * NW, TX = QX, NC = 16 * NCB;
    constexpr bool sasa = WM == NA_WINDOW_SASA;
    for (int k = kmin; k <= kmax; k += 2) {
        const int nr = wave_rows(QY, RPC, k), lr = halo_lds_rows(TY, QY, RPC, k);
        for (int L : axis_lengths(k, sasa)) {
            // rows (the geometry of an axis depends on that axis only)
            for (int y0 = 0; y0 < L; y0 += TY) {
                const HaloGeom g = halo_geometry<TY, NC, WM>(y0, 0, k, L, L);
                CHECK(g.hr <= lr, "%s k=%d H=%d y0=%d hr=%d lr=%d", name, k, L, y0, g.hr, lr);
                if (!sasa) CHECK(g.hy0 >= 0 && g.hy0 + g.hr <= L, "%s k=%d H=%d y0=%d hy0=%d", name, k, L, y0, g.hy0);
                for (int y = y0; y < imin(y0 + TY, L); ++y) {
                    const int s = window_start<WM>(y, k, L);
                    CHECK(s >= g.hy0 && s + k <= g.hy0 + g.hr, "%s k=%d H=%d y=%d window rows", name, k, L, y);
                }
                for (int w = 0; w < NW; ++w) {
                    const int y1 = y0 + QY * w;
                    if (y1 >= L) continue;  // the wave has no queries
                    const int ry = wave_first_row<WM>(y1, k, L, g.hy0, g.hr, nr);
                    CHECK(ry >= g.hy0 && ry + nr <= g.hy0 + lr, "%s k=%d H=%d y0=%d wave %d ry=%d", name, k, L, y0,
                          w, ry);
                    for (int q = 0; q < QY; ++q) {
                        const int y = imin(y1 + q, L - 1);
                        const int s = window_start<WM>(y, k, L);
                        CHECK(s >= ry && s + k <= ry + nr, "%s k=%d H=%d y=%d candidate rows", name, k, L, y);
                    }
                }
            }
            // columns
            for (int x0 = 0; x0 < L; x0 += TX) {
                const HaloGeom g = halo_geometry<TY, NC, WM>(0, x0, k, L, L);
                if (!sasa) {
                    if (L >= NC)
                        CHECK(g.cx >= 0 && g.cx + NC <= L, "%s k=%d W=%d x0=%d cx=%d", name, k, L, x0, g.cx);
                    else
                        CHECK(g.cx == 0, "%s k=%d W=%d cx=%d", name, k, L, g.cx);
                }
                for (int x = x0; x < imin(x0 + TX, L); ++x) {
                    const int s = window_start<WM>(x, k, L);
                    CHECK(s >= g.cx && s + k <= g.cx + NC, "%s k=%d W=%d x=%d window cols", name, k, L, x);
                }
            }
        }
    }
}

// The column-run kernel (2 x 8 subtiles, 4 waves, chunks of 8 rows, NA):
// simulate the ring over every run start.
static void check_ring(int k)
{
    constexpr int QY = 2, RPC = 8, NW = 4, TY = QY * NW, NC = 16, kRing = 16;
    const int nr = wave_rows(QY, RPC, k), lr = halo_lds_rows(TY, QY, RPC, k);
    CHECK(lr < kRing, "ring k=%d lr=%d", k, lr);
    for (int H : axis_lengths(k, false)) {
        const int tiles = (H + TY - 1) / TY;
        for (int ty0 = 0; ty0 < tiles; ++ty0) {
            int slot[kRing];
            for (int i = 0; i < kRing; ++i) slot[i] = -1000000;
            HaloGeom g = halo_geometry<TY, NC, NA_WINDOW_NA>(ty0 * TY, 0, k, H, H);
            for (int r = g.hy0; r < g.hy0 + lr; ++r) slot[r & (kRing - 1)] = r;  // the full first halo
            for (int ty = ty0; ty < tiles; ++ty) {
                if (ty > ty0) {
                    const HaloGeom gn = halo_geometry<TY, NC, NA_WINDOW_NA>(ty * TY, 0, k, H, H);
                    CHECK(gn.hy0 >= g.hy0, "ring k=%d H=%d ty=%d halo moves up", k, H, ty);
                    const RowRange e = ring_entering(g.hy0, gn.hy0, lr);
                    for (int r = e.lo; r < e.hi; ++r) slot[r & (kRing - 1)] = r;
                    g = gn;
                }
                for (int w = 0; w < NW; ++w) {
                    const int y1 = ty * TY + QY * w;
                    if (y1 >= H) continue;
                    const int ry = wave_first_row<NA_WINDOW_NA>(y1, k, H, g.hy0, g.hr, nr);
                    for (int r = ry; r < ry + nr; ++r)
                        CHECK(slot[r & (kRing - 1)] == r, "ring k=%d H=%d run from %d tile %d wave %d row %d", k, H,
                              ty0, ty, w, r);
                }
            }
        }
    }
}

// ---- wide-window kernel

// WX waves across a tile of four waves: TY x TX = (16 / WX) x (4 WX) queries
static void check_large(int k, int WX)
{
    const int nb = 2 * k - 1, r = k >> 1, P = col_pitch(k), X = col_extent(k);
    const int NBW = (k + 9) / 4;  // blocks per row of the widest kind (the launcher's choice)
    const int TY = 16 / WX, TX = 4 * WX;
    // the four waves' 16 lanes place the tile's TY x TX queries once each
    {
        std::vector<int> seen(TY * TX, 0);
        for (int wave = 0; wave < 4; ++wave)
            for (int c = 0; c < 16; ++c) {
                const QueryPos q = large_query(0, 0, wave, WX, c);
                CHECK(q.y >= 0 && q.y < TY && q.x >= 0 && q.x < TX, "large WX=%d wave %d lane %d outside the tile",
                      WX, wave, c);
                if (q.y >= 0 && q.y < TY && q.x >= 0 && q.x < TX) ++seen[q.y * TX + q.x];
            }
        for (int i = 0; i < TY * TX; ++i) CHECK(seen[i] == 1, "large WX=%d query %d placed %d times", WX, i, seen[i]);
    }
    for (int L : axis_lengths(k, false)) {
        // rows: block rows of each wave and the bias row of every key row
        for (int y0 = 0; y0 < L; y0 += TY) {
            const LargeTileGeom t = large_tile_geometry(y0, 0, TY, TX, k, L, L);
            CHECK(t.nbr >= 1, "large k=%d H=%d y0=%d nbr=%d", k, L, y0, t.nbr);
            for (int wr = 0; wr < 4 / WX; ++wr) {
                const LargeWaveGeom w = large_wave_geometry(t, y0, 0, WX * wr, WX, k, L, L);
                if (!w.active) continue;
                CHECK(0 <= w.rb0 && w.rb0 <= w.rb1 && w.rb1 < t.nbr, "large k=%d H=%d y0=%d rows %d..%d of %d", k, L,
                      y0, w.rb0, w.rb1, t.nbr);
                for (int cy = 0; cy < 4; ++cy) {
                    const LargeLaneGeom l = large_lane_geometry(t, w, 4 * cy, k, L, L);
                    CHECK(l.sy == window_start<NA_WINDOW_NA>(l.qy, k, L), "large k=%d H=%d qy=%d sy", k, L, l.qy);
                    CHECK(l.sy >= t.uy0 + 4 * w.rb0 && l.sy + k <= t.uy0 + 4 * (w.rb1 + 1),
                          "large k=%d H=%d qy=%d window rows outside the wave's block rows", k, L, l.qy);
                    for (int rb = w.rb0; rb <= w.rb1; ++rb)
                        for (int g = 0; g < 4; ++g) {
                            const int ky = t.uy0 + 4 * rb + g;
                            const bool in = ky >= l.sy && ky < l.sy + k;
                            const int bc = large_bias_row(false, ky, l.qy, l.sy, k);
                            const int br = large_bias_row(true, ky, l.qy, l.sy, k);
                            // `col` rows: offset ky - qy (+ k - 1), or the -inf row nb
                            CHECK(bc % P == 0 && bc / P == (in ? ky - l.qy + k - 1 : nb), "large k=%d qy=%d ky=%d col row",
                                  k, l.qy, ky);
                            CHECK(in ? br == (ky - l.qy + k - 1) * nb : br == nb * nb, "large k=%d qy=%d ky=%d raw row", k,
                                  l.qy, ky);
                            if (in) CHECK(ky - l.qy + k - 1 >= 0 && ky - l.qy + k - 1 < nb, "large k=%d offset", k);
                        }
                }
            }
        }
        // columns: block columns, row kinds, and the column part of every bias read
        for (int x0 = 0; x0 < L; x0 += TX) {
            const LargeTileGeom t = large_tile_geometry(0, x0, TY, TX, k, L, L);
            CHECK(t.nbc >= 1 && t.nbc <= kLargeMaxBlocks, "large k=%d WX=%d W=%d x0=%d nbc=%d", k, WX, L, x0, t.nbc);
            for (int wc = 0; wc < WX; ++wc) {
                const LargeWaveGeom w = large_wave_geometry(t, 0, x0, wc, WX, k, L, L);
                if (!w.active) continue;
                CHECK(w.cb0 >= 0 && w.ncb >= 1 && w.cb0 + w.ncb <= t.nbc && w.ncb <= NBW,
                      "large k=%d W=%d x0=%d wave %d blocks %d+%d of %d", k, L, x0, wc, w.cb0, w.ncb, t.nbc);
                // the kernel's row kinds: NBW blocks, NBW - 1, or NBW - 1 with the last masked
                const int NB = w.ncb == NBW ? NBW : NBW - 1;
                const bool clamp = w.ncb < NB;
                const int kx0 = t.ux0 + 4 * w.cb0;
                for (int cx = 0; cx < 4; ++cx) {
                    const LargeLaneGeom l = large_lane_geometry(t, w, cx, k, L, L);
                    const int sx = window_start<NA_WINDOW_NA>(l.qx, k, L);
                    CHECK(l.cxw == kx0 - sx, "large k=%d W=%d qx=%d cxw", k, L, l.qx);
                    CHECK(sx >= kx0 && sx + k <= kx0 + 4 * w.ncb, "large k=%d W=%d qx=%d window cols outside the blocks",
                          k, L, l.qx);
                    if (!w.colclamp)
                        CHECK(sx == l.qx - r, "large k=%d W=%d qx=%d: a clamped window in an unclamped wave", k, L, l.qx);
                    for (int j = 0; j < NB; ++j)
                        for (int e = 0; e < 4; ++e) {
                            const int jj = clamp && j > w.ncb - 1 ? w.ncb - 1 : j;
                            const int kx = kx0 + 4 * jj + e;  // the key whose K and V this slot uses
                            // a repeated block (j past the wave's last) must be masked
                            const bool in = j < w.ncb && kx >= sx && kx < sx + k;
                            const int ci = l.bcol + 4 * j + e;
                            if (!w.colclamp) {
                                CHECK(ci >= 0 && ci < P, "large k=%d W=%d qx=%d j=%d e=%d col column %d", k, L, l.qx, j,
                                      e, ci);
                                const int dx = ci - X;
                                const bool valid = dx >= -r && dx <= r;
                                CHECK(valid == in, "large k=%d W=%d qx=%d j=%d e=%d: col entry %s", k, L, l.qx, j, e,
                                      in ? "masked for a key in the window" : "unmasked for a key outside");
                                if (in) CHECK(dx == kx - l.qx, "large k=%d qx=%d kx=%d col offset", k, l.qx, kx);
                                // and the table holds the bias of that offset there
                                for (int dy = 0; dy < nb && in; dy += nb - 1)
                                    CHECK(col_entry_source(dy * P + ci, k) == dy * nb + dx + k - 1,
                                          "large k=%d col entry source", k);
                            } else {
                                const int mi = kMaskPad + l.cxw + 4 * j + e;
                                CHECK(mi >= 0 && mi < kMaskFloats, "large k=%d W=%d qx=%d mask index %d", k, L, l.qx, mi);
                                const bool open = l.cxw + 4 * j + e >= 0 && l.cxw + 4 * j + e < k;
                                CHECK(open == in, "large k=%d W=%d qx=%d j=%d e=%d: mask %s", k, L, l.qx, j, e,
                                      in ? "closed on a key in the window" : "open on a key outside");
                                // raw index = row base (>= 0, <= nb * nb) + ci: inside the area
                                CHECK(ci >= -kRawPad && nb * nb + ci < raw_floats(k),
                                      "large k=%d W=%d qx=%d raw column %d", k, L, l.qx, ci);
                                if (in) CHECK(ci == kx - l.qx + k - 1, "large k=%d qx=%d kx=%d raw column", k, l.qx, kx);
                            }
                        }
                }
            }
        }
    }
}

int main()
{
    // the launcher's shapes: k = 7 (column runs or the 2 x 8 register-prefetch
    // kernel), k <= 9 (2 x 8), k <= 13 (4 x 4), wider SASA (2 x 8, two
    // 16-column blocks)
    check_halo_shape<2, 8, 1, 8, 4, NA_WINDOW_NA>("2x8 rpc8 NA", 7, 7);
    check_halo_shape<2, 8, 1, 8, 4, NA_WINDOW_SASA>("2x8 rpc8 SASA", 7, 7);
    check_halo_shape<2, 8, 1, 2, 4, NA_WINDOW_NA>("2x8 rpc2 NA", 3, 9);
    check_halo_shape<2, 8, 1, 2, 4, NA_WINDOW_SASA>("2x8 rpc2 SASA", 3, 9);
    check_halo_shape<4, 4, 1, 8, 4, NA_WINDOW_NA>("4x4 NA", 11, 13);
    check_halo_shape<4, 4, 1, 8, 4, NA_WINDOW_SASA>("4x4 SASA", 11, 13);
    check_halo_shape<2, 8, 2, 2, 4, NA_WINDOW_NA>("2x8 ncb2 NA", 15, 25);
    check_halo_shape<2, 8, 2, 2, 4, NA_WINDOW_SASA>("2x8 ncb2 SASA", 15, 25);
    check_ring(7);
    // the launcher's tile shapes: 4 x 16 while 16 + k - 1 <= 32 columns, else 8 x 8
    for (int k = 7; k <= NA2D_MFMA_MAX_KSIZE; k += 2) {
        check_large(k, 2);
        if (k <= 17) check_large(k, 4);
    }
    if (g_fails) {
        std::printf("%ld of %ld checks failed\n", g_fails, g_checks);
        return 1;
    }
    std::printf("ok %ld\n", g_checks);
    return 0;
}
