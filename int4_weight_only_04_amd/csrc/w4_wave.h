// Reductions inside one 64-lane wave without LDS traffic: DPP row shifts
// within each 16-lane row, then lane reads of the four row totals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4i {
namespace wave {


// Sum over each row of 16 lanes with DPP row shifts (lanes whose source lies
// outside the row add 0): lane 15 of the row ends with the total, summed as a
// balanced tree of depth 4.
__device__ __forceinline__ float row16_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
    return v;
}

// lane 15 + 16 q of v, for the four rows q (uniform values)
__device__ __forceinline__ void row_totals(float v, float (&r)[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r[q] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * q + 15));
}

// Whole-wave sum as a tree of depth 6 (4 row levels, then (r0 + r1) + (r2 + r3)),
// the same depth as a 6-level butterfly; uniform result.
__device__ __forceinline__ float wave_sum_tree(float v)
{
    float r[4];
    row_totals(row16_sum(v), r);
    return (r[0] + r[1]) + (r[2] + r[3]);
}

}  // namespace wave
}  // namespace w4i
