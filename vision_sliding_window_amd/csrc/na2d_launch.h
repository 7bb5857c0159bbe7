// na2d_launch.h -- internal interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace na2d {

// One validated forward problem (see include/na2d.h for the meaning of each
// field).  The grid is [B, heads, depth, H, W] with a kd x kh x kw window;
// `ksize` is the square window of the 2D case (kh = kw) that the MFMA kernel
// serves.
struct Problem {
    const void *q, *k, *v;
    const float *rpb;  // may be null: no positional bias
    float *out;
    int B, heads, H, W, d, ksize, dtype;
    int depth, kd, kh, kw, mode;
    float *lse = nullptr;  // per-query log-sum-exp of the logits (NA 2D only), or null
};

// One validated backward problem (include/na2d.h, na2d_backward).
struct BwdProblem {
    const void *q, *k, *v;
    const float *rpb, *out, *lse, *dout;  // lse: the forward's, or null (recomputed)
    float *dq, *dk, *dv, *drpb;
    void *workspace;
    int B, heads, H, W, d, ksize, dtype;
    int algo;  // NA2D_ALGO_MFMA: both passes on the matrix cores; NA2D_ALGO_VALU
};

// The backward workspace: per query its softmax statistics (a float2), then,
// from a 256-byte boundary, one (2k-1)^2 float table per 8 x 8 query tile
// (the tile's share of the bias gradient, summed by a second kernel).
inline unsigned long long bwd_stats_bytes(int B, int heads, int H, int W)
{
    return ((unsigned long long)B * heads * H * W * 8ull + 255ull) & ~255ull;
}
inline unsigned long long bwd_tiles(int B, int heads, int H, int W)
{
    return (unsigned long long)B * heads * ((H + 7) / 8) * ((W + 7) / 8);
}
inline unsigned long long bwd_workspace_bytes(int B, int heads, int H, int W, int ksize)
{
    const unsigned long long nb = 2ull * ksize - 1;
    return bwd_stats_bytes(B, heads, H, W) + bwd_tiles(B, heads, H, W) * nb * nb * 4ull;
}

// Launchers; each returns the HIP status of its launch.  The arguments have
// been checked by the caller.
hipError_t launch_valu(const Problem &p, hipStream_t stream);
hipError_t launch_mfma(const Problem &p, hipStream_t stream);     // square 2D windows
hipError_t launch_mfma_1d(const Problem &p, hipStream_t stream);  // NA1D
hipError_t launch_mfma_3d(const Problem &p, hipStream_t stream);  // other NA windows (3D, rectangular 2D)
hipError_t launch_mfma_large(const Problem &p, hipStream_t stream);  // wide square 2D NA windows
hipError_t launch_backward(const BwdProblem &p, hipStream_t stream);
hipError_t launch_backward_mfma(const BwdProblem &p, hipStream_t stream);  // both passes on MFMA

// Device address of this device's fixed scratch array (na2d_noalloc.hip),
// looked up on the first call per device and kept.
hipError_t noalloc_scratch(void **ptr);

// Compute units of the current device (cached per thread).
int device_cus();
// Resident workgroups per CU of kernel `f` with `threads` threads and `lds`
// bytes of dynamic LDS on the current device, queried once per kernel,
// device and LDS size and then read from a process-wide cache.
hipError_t occupancy(const void *f, int threads, size_t lds, int &per_cu);

// Occupancy queries made so far in this process (each kernel, device and LDS
// size is queried once, then cached).
long long occupancy_queries();

}  // namespace na2d
