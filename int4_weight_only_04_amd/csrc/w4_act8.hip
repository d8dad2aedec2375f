// Per-group symmetric int8 quantization of an fp16 activation vector, the
// input of the W4A8 GEMV variant (the INT8-activation path the pages' runtime
// built and removed: "Tutorial: como construir seu proprio runtime de LLM do
// zero", noticiai.com.br, "As tres licoes", lesson 3).  For each group g of G
// consecutive inputs, in binary32 with round-to-nearest-even:
//
//     amax = max |x|,  inv = 127 / amax,  c = clamp(rint(x * inv), -127, 127),
//     s_g = amax / 127            (amax == 0: c = 0, s_g = 0)
//
// The codes are stored in the packed nibble order of the W4T4 layout: the 8
// bytes of block j hold inputs 8j + (0, 4, 1, 5, 2, 6, 3, 7), the order in
// which (word & 0x0F0F0F0F) and ((word >> 4) & 0x0F0F0F0F) of a packed weight
// word present their nibbles, so the GEMV dots bytes with bytes directly.
//
// One wave per group: lane i takes blocks i, i + 64, ... of the group; the
// group maximum is reduced across the wave with butterfly shuffles.  For
// groups of at most 512 inputs (64 blocks) a lane holds at most one block,
// which stays in registers between the maximum and the codes: one load round.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"

namespace w4i {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ float half_to_float(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

__device__ __forceinline__ uint32_t code_byte(float v, float inv)
{
    float r = __builtin_rintf(__fmul_rn(v, inv));
    r = r > 127.0f ? 127.0f : (r < -127.0f ? -127.0f : r);
    return (uint32_t)((int32_t)r) & 0xFFu;
}

// The 8 codes of one block of inputs, in the packed nibble order.
__device__ __forceinline__ uint2 block_codes(const uint4& v, float inv)
{
    // inputs 0..7 of the block: v.x = (0, 1), v.y = (2, 3), v.z = (4, 5), v.w = (6, 7)
    const uint32_t c0 = code_byte(half_to_float(v.x & 0xFFFFu), inv);
    const uint32_t c1 = code_byte(half_to_float(v.x >> 16), inv);
    const uint32_t c2 = code_byte(half_to_float(v.y & 0xFFFFu), inv);
    const uint32_t c3 = code_byte(half_to_float(v.y >> 16), inv);
    const uint32_t c4 = code_byte(half_to_float(v.z & 0xFFFFu), inv);
    const uint32_t c5 = code_byte(half_to_float(v.z >> 16), inv);
    const uint32_t c6 = code_byte(half_to_float(v.w & 0xFFFFu), inv);
    const uint32_t c7 = code_byte(half_to_float(v.w >> 16), inv);
    return make_uint2(c0 | (c4 << 8) | (c1 << 16) | (c5 << 24), c2 | (c6 << 8) | (c3 << 16) | (c7 << 24));
}

__global__ void __launch_bounds__(kQuantThreads) act8_quantize_kernel(const uint4* __restrict__ x, int64_t ngroups,
                                                                      int32_t blocks_per_group,
                                                                      uint2* __restrict__ codes,
                                                                      float* __restrict__ scales)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
    if (g >= ngroups) return;  // whole waves only; no barrier in this kernel
    const int64_t b0 = g * blocks_per_group;
    if (blocks_per_group <= 64) {  // uniform per launch
        const bool has = lane < blocks_per_group;
        const uint4 v = has ? x[b0 + lane] : make_uint4(0u, 0u, 0u, 0u);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(half_to_float(w[i] & 0xFFFFu)));
            amax = fmaxf(amax, fabsf(half_to_float(w[i] >> 16)));
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const float inv = amax > 0.0f ? __fdiv_rn(127.0f, amax) : 0.0f;
        if (has) codes[b0 + lane] = block_codes(v, inv);
        if (lane == 0) scales[g] = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 0.0f;
        return;
    }
    float amax = 0.0f;
    for (int b = lane; b < blocks_per_group; b += 64) {
        const uint4 v = x[b0 + b];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(half_to_float(w[i] & 0xFFFFu)));
            amax = fmaxf(amax, fabsf(half_to_float(w[i] >> 16)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float inv = amax > 0.0f ? __fdiv_rn(127.0f, amax) : 0.0f;
    for (int b = lane; b < blocks_per_group; b += 64) {
        codes[b0 + b] = block_codes(x[b0 + b], inv);
    }
    if (lane == 0) scales[g] = amax > 0.0f ? __fdiv_rn(amax, 127.0f) : 0.0f;
}

}  // namespace

hipError_t launch_act8_quantize(const uint16_t* x, int64_t k, int32_t group, int8_t* codes, float* scales,
                                hipStream_t stream)
{
    const int64_t ngroups = k / group;
    const int64_t grid = (ngroups + kQuantThreads / 64 - 1) / (kQuantThreads / 64);
    hipLaunchKernelGGL(act8_quantize_kernel, dim3((unsigned)grid), dim3(kQuantThreads), 0, stream,
                       reinterpret_cast<const uint4*>(x), ngroups, (int32_t)(group / 8), reinterpret_cast<uint2*>(codes),
                       scales);
    return hipGetLastError();
}

}  // namespace w4i
