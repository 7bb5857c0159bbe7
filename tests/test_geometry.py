"""The forward kernels' tile geometry, enumerated on the CPU.

tests/geometry_check.cpp includes vision_sliding_window_amd/csrc/na_geometry.h
-- the window starts, halos, candidate rows, ring steps, block grids and
bias-table indexing that the matrix-core kernels call -- and checks over
window sizes, map sizes and tile origins that every window a tile needs is
staged where the kernel reads it, and that every bias read lands on the bias
of that key-minus-query offset inside the window and on -inf outside it
(NA windows per "Neighborhood Attention Transformer", CSDN translation,
section 3.1; SASA windows centred on the zero-padded map).

The program is built with hipcc for the host only. Planted mistakes in a
copy of the header (one arithmetic change each) must make it fail.
"""
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "vision_sliding_window_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def build_and_run(tmp, header_dir):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = os.path.join(tmp, "geometry_check")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                    "-I", os.path.join(REPO, "include"), "-I", header_dir,
                    os.path.join(REPO, "tests", "geometry_check.cpp"), "-o", exe],
                   check=True, capture_output=True, timeout=300)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300)


def test_geometry():
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        r = build_and_run(tmp, CSRC)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-2000:]
    assert r.stdout.startswith("ok ")


# (name, text in na_geometry.h, replacement): each breaks one property
MUTANTS = [
    ("halo_columns_shifted", "g.cx = W >= NC ? (sx < W - NC ? sx : W - NC) : 0;",
     "g.cx = W >= NC ? (sx + 1 < W - NC ? sx + 1 : W - NC) : 0;"),
    ("halo_rows_short", "g.hr = TY + ks - 1 < H ? TY + ks - 1 : H;",
     "g.hr = TY + ks - 2 < H ? TY + ks - 2 : H;"),
    ("wave_rows_past_halo", "const int top = hy0 + hr - nr;", "const int top = hy0 + hr - nr + 1;"),
    ("ring_row_skipped", "r.lo = hy0 + lr > hy0n ? hy0 + lr : hy0n;",
     "r.lo = hy0 + lr + 1 > hy0n ? hy0 + lr + 1 : hy0n;"),
    ("large_block_columns_short", "g.nbc = (ux1 - g.ux0 + 3) >> 2;", "g.nbc = (ux1 - g.ux0) >> 2;"),
    ("large_wave_column_order", "q.x = x0 + 4 * (wave % WX) + (c & 3);", "q.x = x0 + 4 * (wave % 2) + (c & 3);"),
    ("large_clamp_test_off_by_one", "w.colclamp = !(w.xa - r >= 0 && xl + r <= W - 1 && w.xa + 3 < W);",
     "w.colclamp = !(w.xa - r >= 0 && xl + r <= W && w.xa + 3 < W);"),
    ("col_table_narrow", "return (ks >> 1) + 6;", "return (ks >> 1) + 5;"),
    ("mask_pad_short", "constexpr int kMaskPad = 8;", "constexpr int kMaskPad = 3;"),
    ("raw_pad_short", "constexpr int kRawPad = 4;", "constexpr int kRawPad = 2;"),
    ("col_row_offset", "return (rowin ? ky - qy + ks - 1 : nb) * col_pitch(ks);",
     "return (rowin ? ky - qy + ks : nb) * col_pitch(ks);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_geometry_mutant_fails(name, old, new, tmp_path):
    src = open(os.path.join(CSRC, "na_geometry.h")).read()
    assert src.count(old) == 1, name
    hdr = tmp_path / "hdr"
    hdr.mkdir()
    (hdr / "na_geometry.h").write_text(src.replace(old, new))
    r = build_and_run(str(tmp_path), str(hdr))
    assert r.returncode != 0, "%s: the check passed a planted mistake" % name
