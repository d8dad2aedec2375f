// Device arithmetic shared by the decode GEMV kernels (one kernel per
// projection, and the persistent sweep kernel): the exact INT4 unpack and fp32
// dot product of one 8-input block, the W4A8 integer dot, and the lane
// reduction of a tile's four row sums.  Both kernels use these same functions
// in the same order, so their outputs agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4i {
namespace gemv_math {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// The fp16 pair (1024.0, 1024.0) held in a VGPR the compiler cannot fold:
// with the magic number opaque, (d & mask) | magic selects one v_and_or_b32
// (mask in an SGPR) instead of an AND and an OR with two literals.
__device__ __forceinline__ uint32_t opaque_magic()
{
    uint32_t r;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(r));
    return r;
}

// fp32 dot product of two fp16 pairs started from zero: one VOP3P
// v_dot2_f32_f16 with an inline-constant accumulator (the builtin with a 0.0
// accumulator compiles to a register move plus v_dot2c).
__device__ __forceinline__ float dot2_first(h2_t a, h2_t b)
{
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// sum over the 8 inputs of one block of (q - 8) * x, fp32
__device__ __forceinline__ float dot8(uint32_t d, const uint4& xv, uint32_t magic)
{
    const uint32_t a = (d & 0x000F000Fu) | magic;  // inputs 0,1: 1024 + q
    const uint32_t b = (d & 0x00F000F0u) | magic;  // inputs 2,3: 1024 + 16 q
    const uint32_t d8 = d >> 8;
    const uint32_t c = (d8 & 0x000F000Fu) | magic;  // inputs 4,5
    const uint32_t e = (d8 & 0x00F000F0u) | magic;  // inputs 6,7
    const h2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const h2_t va = as_h2(a) + bias;
    const h2_t vb = __builtin_elementwise_fma(as_h2(b), sixteenth, bias16);
    const h2_t vc = as_h2(c) + bias;
    const h2_t ve = __builtin_elementwise_fma(as_h2(e), sixteenth, bias16);
    float p = dot2_first(va, as_h2(xv.x));
    p = __builtin_amdgcn_fdot2(vb, as_h2(xv.y), p, false);
    p = __builtin_amdgcn_fdot2(vc, as_h2(xv.z), p, false);
    p = __builtin_amdgcn_fdot2(ve, as_h2(xv.w), p, false);
    return p;
}

// W4A8: sum over the 8 inputs of one block of (q - 8) * c as an exact
// integer.  The nibbles of (d & 0x0F0F0F0F) and ((d >> 4) & 0x0F0F0F0F) are
// bytes 0..15 (non-negative as int8), in the byte order the activation codes
// are stored in, so two v_dot4_i32_i8 give sum q c; neg8cs = -8 sum c of the
// block (shared by every row) removes the zero point.
__device__ __forceinline__ int idot8(uint32_t d, const uint2& c, int neg8cs)
{
    const int lo = (int)(d & 0x0F0F0F0Fu);
    const int hi = (int)((d >> 4) & 0x0F0F0F0Fu);
    const int t = __builtin_amdgcn_sdot4(lo, (int)c.x, neg8cs, false);
    return __builtin_amdgcn_sdot4(hi, (int)c.y, t, false);
}

__device__ __forceinline__ int neg8_code_sum(const uint2& c)
{
    const int t = __builtin_amdgcn_sdot4((int)c.x, 0x01010101, 0, false);
    return -8 * __builtin_amdgcn_sdot4((int)c.y, 0x01010101, t, false);
}

__device__ __forceinline__ float half_lo(uint32_t v) { return (float)as_h2(v)[0]; }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)as_h2(v)[1]; }

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Non-temporal 16- and 8-byte loads for the weight and scale streams: every
// byte is read once per sweep, and the streaming hint measured ~5-10% more
// HBM bandwidth on MI355X than default-cached loads for this access pattern.
__device__ __forceinline__ uint4 ld_stream(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 ld_stream(const uint2* p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ float as_f(unsigned v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ unsigned as_u(float v) { return __builtin_bit_cast(unsigned, v); }

// Reduce the 64-lane partials of a tile's 4 rows at once with gfx950's lane
// swaps: v_permlane32_swap pairs rows (0,1) and (2,3) across the two wave
// halves, v_permlane16_swap pairs the results across 16-lane rows, and four
// DPP steps finish each 16-lane row.  Afterwards every lane of 16-lane row
// 0 holds row 0's sum, row 1 holds row 2's, row 2 holds row 1's and row 3
// holds row 3's (10 instructions instead of 4 x 11 for per-row reductions).
__device__ __forceinline__ float reduce4(float a, float b, float c, float d)
{
    const auto ab = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
    const auto cd = __builtin_amdgcn_permlane32_swap(as_u(c), as_u(d), false, false);
    const float p = as_f(ab[0]) + as_f(ab[1]);
    const float q = as_f(cd[0]) + as_f(cd[1]);
    const auto pq = __builtin_amdgcn_permlane16_swap(as_u(p), as_u(q), false, false);
    float r = as_f(pq[0]) + as_f(pq[1]);
    r += dpp<0xB1>(r);
    r += dpp<0x4E>(r);
    r += dpp<0x141>(r);
    r += dpp<0x140>(r);
    return r;
}

// tile row whose sum reduce4 leaves in this lane's 16-lane row
__device__ __forceinline__ int reduced_row(int lane)
{
    const int g = lane >> 4;  // 0, 1, 2, 3 -> rows 0, 2, 1, 3
    return ((g & 1) << 1) | (g >> 1);
}

__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi)
{
    return v > bv || (v == bv && i < bi);
}

}  // namespace gemv_math
}  // namespace w4i
