"""LDS table bounds that the matrix-core kernels rely on, checked by enumeration.

The kernels read their relative-position bias tables without clamping the
index: the tables are padded so that every index a wave can form lies inside
them. These tests restate the kernels' tile geometry (window starts, halo
rows, each wave's candidate rows and the streamed blocks) and enumerate every
index over window sizes and map sizes, so a change to the geometry that would
read outside a table fails here, on the CPU.

Window starts follow the clamped NA window of "Neighborhood Attention
Transformer" (CSDN translation, section 3.1): start = clamp(i - k/2, 0, L - k).
"""


def wstart(i, k, L):
    return min(max(i - k // 2, 0), L - k)


def test_forward_general_table_rows():
    """na2d_mfma.hip, attend (general path, compile-time kernel size, one chunk).

    A wave of QY = 2 query rows in a tile of four waves reads candidate rows
    ry .. ry + QY + k - 2 and, for its query row y, table row
    ry + r - y + k - 1 of the general bias table, which has one -inf row
    above the (2k - 1) rows of offsets and one below. So that index must lie
    in [-1, 2k - 1]; rows outside the query's window may only be the first
    and the last candidate rows (the kernel masks just those two).
    """
    QY, NW = 2, 4
    TY = QY * NW
    for k in range(3, 15, 2):
        nr = QY + k - 1
        lo, hi = 10 ** 9, -10 ** 9
        for H in range(k, 90):
            for y0 in range(0, H, TY):
                hr = min(TY + k - 1, H)
                hy0 = min(wstart(y0, k, H), H - hr)
                for wave in range(NW):
                    y1 = y0 + QY * wave
                    if y1 >= H:
                        continue
                    ry = max(hy0, min(wstart(min(y1, H - 1), k, H), hy0 + hr - nr))
                    # the wave's candidate rows lie in the LDS halo of max(TY + k - 1, nr) rows
                    assert hy0 <= ry and ry - hy0 + nr <= max(TY + k - 1, nr), (k, H, y0, wave)
                    for qy in range(QY):
                        y = min(y1 + qy, H - 1)
                        sy = wstart(y, k, H)
                        for r in range(nr):
                            idx = ry + r - y + k - 1
                            lo, hi = min(lo, idx), max(hi, idx)
                            inside = 0 <= ry + r - sy < k
                            if inside:
                                assert 0 <= idx <= 2 * k - 2, (k, H, y0, wave, qy, r)
                            else:
                                assert r in (0, nr - 1), (k, H, y0, wave, qy, r)
                            # rows [nr - k, k) are inside every window of the wave
                            if nr - k <= r < k:
                                assert inside, (k, H, y0, wave, qy, r)
        assert lo >= -1 and hi <= 2 * k - 1, (k, lo, hi)


def holders(j, k, L):
    """First and last query whose clamped window holds key j (na2d_bwd_mfma.hip)."""
    r = k // 2
    return (0 if j < k else j - r), (L - 1 if j >= L - k else j + r)


def test_backward_bias_table_bounds():
    """na2d_bwd_mfma.hip: the padded bias tables of both passes.

    Each wave owns a 2 x 8 patch of a tile of four waves and streams 16-wide
    blocks of the other side: its queries' keys (query pass) or the queries
    holding its keys (key pass). The tables hold one padding row above and
    below the 2k - 1 offset rows, and 8 | 24 padding columns (query pass) or
    24 | 8 (key pass) beside the 2k - 1 offset columns.
    """
    QL, QR, KL, KR = 8, 24, 24, 8
    for k in range(3, 27, 2):
        nb = 2 * k - 1
        for L in list(range(k, k + 40)) + [56, 100, 128]:
            for t0 in range(0, L, 8):
                for w in range(4):
                    r1 = t0 + 2 * w
                    if r1 >= L:
                        continue
                    own = {min(r1, L - 1), min(r1 + 1, L - 1)}
                    kylo = wstart(r1, k, L)
                    kyhi = wstart(min(r1 + 1, L - 1), k, L) + k - 1
                    for qy in own:  # query pass rows
                        for ky in range(kylo, kyhi + 1):
                            assert -1 <= ky - qy + k - 1 <= nb, (k, L, t0, w)
                    ylo = holders(r1, k, L)[0]
                    yhi = holders(min(r1 + 1, L - 1), k, L)[1]
                    for ky in own:  # key pass rows
                        for y in range(ylo, yhi + 1):
                            assert -1 <= ky - y + k - 1 <= nb, (k, L, t0, w)
                x0 = t0
                kxlo = wstart(x0, k, L)
                kxhi = wstart(min(x0 + 7, L - 1), k, L) + k - 1
                nblk = (kxhi - kxlo + 16) >> 4
                for c in range(8):  # query pass columns
                    qx = min(x0 + c, L - 1)
                    for kx in range(kxlo, kxlo + 16 * nblk):
                        assert -QL <= kx - qx + k - 1 < nb + QR, (k, L, t0, c)
                xlo = holders(x0, k, L)[0]
                xhi = holders(min(x0 + 7, L - 1), k, L)[1]
                nblk = (xhi - xlo + 16) >> 4
                for c in range(8):  # key pass columns
                    kx = min(x0 + c, L - 1)
                    for x in range(xlo, xlo + 16 * nblk):
                        assert -KL <= kx - x + k - 1 < nb + KR, (k, L, t0, c)
