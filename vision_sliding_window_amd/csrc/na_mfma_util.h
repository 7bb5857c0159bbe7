// na_mfma_util.h -- device helpers shared by the matrix-core kernels (gfx950):
// fragment types, the 16x16x32 MFMA wrappers, the cross-lane reductions of
// the S^T = K Q^T layout, and raw buffer descriptors.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace na2d {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const unsigned char lds_cu8;
typedef __attribute__((address_space(3))) const u32x4 lds_cu4;
typedef __attribute__((address_space(3))) const float lds_cf32;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kD = 32;        // head dim handled here
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr unsigned kOutOfRange = 0x7ffffff0u;  // byte offset past any map: loads 0, stores dropped
// Buffer cache policy (gfx950 encoding): bit 1 marks an access non-temporal,
// for data that is not touched again -- outputs and inputs read exactly once.
constexpr int kNonTemporal = 2;

template <typename T> struct Frag;
template <> struct Frag<_Float16> { typedef half8 type; };
template <> struct Frag<__bf16> { typedef bf16x8 type; };

__device__ inline floatx4 mfma16x16x32(const half8 &a, const half8 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 x 16 x 16 products: one 16-key block against 16 queries (or 16 dims)
__device__ inline floatx4 mfma16x16x16(const half4 &a, const half4 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma16x16x16(const bf16x4 &a, const bf16x4 &b, const floatx4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, a),
                                                     __builtin_bit_cast(v4i16, b), c, 0, 0, 0);
}

// Max and sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 that hold one query.
// v_permlane16_swap(x, x) returns both members of each (l, l ^ 16) pair in its
// two results (and likewise permlane32 for l ^ 32), so op(r0, r1) is the
// pairwise reduction -- the same value, bit for bit, in both lanes.
// (v_max_f32 written out: fmaxf would first quiet both inputs, two more
// instructions per step, which a max over scores does not need)
__device__ inline float max_f32(float a, float b)
{
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(a), "v"(b));
    return m;
}
__device__ inline float quad_max(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = max_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_f32(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float quad_sum(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-wave LDS copy of a 16-position block [pos][32 dims] of 16-bit values
// that is read back with ds_read_b64_tr_b16: the 16-byte slice s of position
// p sits at byte p * 64 + 16 * (s ^ copy_swz(p)).
//
// 16-byte stores are served 8 lanes (128 bytes) at a time. Lane (g, c)
// writes slice g of position c, so positions 0, 2, 4, 6 (and 1, 3, 5, 7)
// need 4 different swizzles. In a transposed read, each group of 16 lanes
// reads four positions 4 g' .. 4 g' + 3, two slices each. Positions 4 g' and
// 4 g' + 2 (and likewise + 1 and + 3) need swizzles that differ in bit 1.
// (p & 2) | ((p >> 2) & 1) meets both conditions. p & 3 met only the second,
// and conflicted 2-way on the stores.
__device__ inline unsigned copy_swz(unsigned p) { return (p & 2u) | ((p >> 2) & 1u); }

__device__ inline unsigned stage_off(int g, int c)
{
    return (unsigned)c * 64u + 16u * ((unsigned)g ^ copy_swz((unsigned)c));
}
// Where lane (g, i) reads for the transposed load of dims 16 dh .. 16 dh + 15:
// dims 16 dh + 4 (i & 3) .. + 3 of position 4 g + (i >> 2); the lane then holds
// dim 16 dh + i of positions 4 g .. 4 g + 3.
__device__ inline unsigned tr_read_off(int g, int i, int dh)
{
    const unsigned p = 4u * g + ((unsigned)i >> 2);
    const unsigned s = 2u * dh + ((unsigned)(i & 3) >> 1);
    return p * 64u + 16u * (s ^ copy_swz(p)) + 8u * (unsigned)(i & 1);
}

// Hide a pointer's provenance from the optimiser (an empty asm that "may
// change" the register), so it is not re-derived from a shared base plus a
// large per-access constant.
template <typename P>
__device__ inline void opaque(P *&p)
{
    asm volatile("" : "+v"(p));
}

// Issue priority of a persistent workgroup from the tiles it has left
// (this one included): 3 while more than three remain, then 2, 1, 0. The
// sequencer issues from the oldest wave among equals, so without this the
// youngest workgroup on a CU falls behind the others all the way and runs
// its last tiles nearly alone; with it a workgroup that is ahead yields.
// Measured at NAT-Tiny stage 1: -0.4 to -0.5 us (the opposite order: +0.5).
__device__ inline void work_priority(unsigned end, unsigned tile, unsigned step)
{
    const unsigned left = (end - tile + step - 1) / step;
    if (left > 3) __builtin_amdgcn_s_setprio(3);
    else if (left == 3) __builtin_amdgcn_s_setprio(2);
    else if (left == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// A raw buffer resource over one (b, h) map of a [B, heads, H, W, ...] tensor.
__device__ inline __amdgpu_buffer_rsrc_t map_rsrc(const void *base, int64_t map_base,
                                                  unsigned pixel_bytes, unsigned map_bytes)
{
    const char *p = static_cast<const char *>(base) + map_base * pixel_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, (int)map_bytes,
                                             (int)kRsrcWord3);
}

}  // namespace
}  // namespace na2d
