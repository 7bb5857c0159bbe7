// na_stream.hip -- a memory-rate reference for the forward kernels: a plain
// streaming kernel that moves the bytes a fused forward must move (three
// 16-bit input tensors read once, one fp32 tensor of the same element count
// written once) and does no attention.  Each lane reads one 16-byte chunk of
// each input and writes the 32 bytes of their elementwise fp32 sum, with
// non-temporal loads and stores, one chunk per lane over a flat grid.  Timed
// beside a forward on the same buffers, it shows what the memory system gives
// a launch of that size with perfectly coalesced, single-pass traffic.
#include "na2d.h"

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ a,
                                                     const u32x4 *__restrict__ b,
                                                     const u32x4 *__restrict__ c,
                                                     floatx4 *__restrict__ out, uint64_t chunks)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i >= chunks) return;
    const half8 x = __builtin_bit_cast(half8, __builtin_nontemporal_load(a + i));
    const half8 y = __builtin_bit_cast(half8, __builtin_nontemporal_load(b + i));
    const half8 z = __builtin_bit_cast(half8, __builtin_nontemporal_load(c + i));
    floatx4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lo[j] = (float)x[j] + (float)y[j] + (float)z[j];
        hi[j] = (float)x[4 + j] + (float)y[4 + j] + (float)z[4 + j];
    }
    __builtin_nontemporal_store(lo, out + 2 * i);
    __builtin_nontemporal_store(hi, out + 2 * i + 1);
}

}  // namespace

extern "C" int na_stream_reference(const void *a, const void *b, const void *c, float *out,
                                   long long elems, void *stream)
{
    if (!a || !b || !c || !out) return NA2D_ERR_NULL;
    if (elems <= 0 || (elems & 7) || (unsigned long long)elems > (1ull << 40)) return NA2D_ERR_SHAPE;
    const void *ptrs[4] = {a, b, c, out};
    for (const void *p : ptrs)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return NA2D_ERR_ALIGN;
    const uint64_t chunks = (uint64_t)elems / 8;
    const uint64_t blocks = (chunks + 255) / 256;
    if (blocks > 0x7fffffffull) return NA2D_ERR_SHAPE;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(a),
                       static_cast<const u32x4 *>(b), static_cast<const u32x4 *>(c),
                       reinterpret_cast<floatx4 *>(out), chunks);
    return hipGetLastError() == hipSuccess ? NA2D_OK : NA2D_ERR_HIP;
}
