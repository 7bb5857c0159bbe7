// na_xcd.h -- XCD-aware workgroup numbering for flat (one tile per workgroup)
// launches on MI355X.
//
// The dispatcher hands workgroups to the 8 XCDs in turn (workgroup b runs on
// XCD b mod 8), and each XCD has its own L2.  Neighbouring tiles share most
// of their halo data, so a launch should let each XCD walk one contiguous
// stretch of tiles: tile = (b mod 8) * (grid / 8) + b / 8.  The grid is
// launched as a multiple of 8 (xcd_grid); workgroups whose tile is past the
// end return at once.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {

constexpr unsigned kXcds = 8;

inline uint64_t xcd_grid(uint64_t blocks) { return (blocks + kXcds - 1) / kXcds * kXcds; }

__device__ inline unsigned xcd_tile(unsigned b, unsigned grid)
{
    return (b % kXcds) * (grid / kXcds) + b / kXcds;
}

}  // namespace na2d
