// Greedy sampling's second half: the lowest-index maximum over the
// per-workgroup (value, row) partials that the lm_head GEMV's argmax
// epilogue writes.  The pages' runtime samples with code of its own after
// the lm_head projection ("How To Build Your Own LLM Runtime From Scratch",
// aitrending.vip, "Industry Insight"), read here as greedy decoding: the
// token is the first index of the largest logit, and NaN logits never win.
//
// One workgroup of 1024 threads reads every partial in one memory round
// trip (16-byte loads of 4 values and 4 rows, the count % 4 tail as 4-byte
// loads issued first), keeps the running best in registers, and reduces
// the wave with DPP exchanges and lane swaps; the 16 wave results meet once
// in LDS.  The kernel boundary after the GEMV orders the partials, so no
// device-scope fence or atomic is involved.  The decode step also passes
// its position counter, which thread 0 advances after writing the token:
// the step then needs no kernel of its own for that.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_gemv_math.h"
#include "w4_internal.h"

namespace w4i {
namespace {

using gemv_math::as_f;
using gemv_math::as_u;
using gemv_math::better;

constexpr int kFinalThreads = 1024;
constexpr int kFinalVec = 6;  // 4-partial loads per thread per round: 24576 partials a round

// keep the (v, i) that `better` prefers among this lane's and the lane the
// DPP control CTRL names
template <int CTRL>
__device__ __forceinline__ void best_dpp(float& bv, int32_t& bi)
{
    const float ov = gemv_math::dpp<CTRL>(bv);
    const int32_t oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xF, 0xF, false);
    if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
    }
}

// the preferred of the two (v, i) pairs a lane swap leaves in a lane
__device__ __forceinline__ void best_pair(float& bv, int32_t& bi, unsigned v0, unsigned v1, unsigned i0, unsigned i1)
{
    const bool one = better(as_f(v1), (int32_t)i1, as_f(v0), (int32_t)i0);
    bv = as_f(one ? v1 : v0);
    bi = (int32_t)(one ? i1 : i0);
}

// Every lane ends with the wave's lowest-index maximum: exchanges within
// quads, half rows and rows (DPP), then across 16-lane rows and wave halves
// (v_permlane16_swap / v_permlane32_swap of a register with itself leave
// the lane's own value and its partner's).  `better` is a strict order on
// (value, row) pairs, so every lane reaches the same pair.
__device__ __forceinline__ void wave_best(float& bv, int32_t& bi)
{
    best_dpp<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
    best_dpp<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
    best_dpp<0x141>(bv, bi);  // row_half_mirror
    best_dpp<0x140>(bv, bi);  // row_mirror
    const auto v16 = __builtin_amdgcn_permlane16_swap(as_u(bv), as_u(bv), false, false);
    const auto i16 = __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    best_pair(bv, bi, v16[0], v16[1], i16[0], i16[1]);
    const auto v32 = __builtin_amdgcn_permlane32_swap(as_u(bv), as_u(bv), false, false);
    const auto i32 = __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false);
    best_pair(bv, bi, v32[0], v32[1], i32[0], i32[1]);
}

__device__ __forceinline__ void take(float v, int32_t i, float& bv, int32_t& bi)
{
    if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
    }
}

// One load round: groups b0, b0 + 1024, ... of 4 partials (those below n4),
// all loaded before any is compared.
__device__ __forceinline__ void load_round(const float4* pv4, const int4* pi4, int32_t n4, int32_t b0, float& bv,
                                           int32_t& bi)
{
    const float ninf = -__builtin_inff();
    float4 v[kFinalVec];
    int4 ix[kFinalVec];
#pragma unroll
    for (int u = 0; u < kFinalVec; ++u) {
        const int32_t b = b0 + u * kFinalThreads;
        v[u] = b < n4 ? pv4[b] : make_float4(ninf, ninf, ninf, ninf);
        ix[u] = b < n4 ? pi4[b] : make_int4(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX);
    }
#pragma unroll
    for (int u = 0; u < kFinalVec; ++u) {
        take(v[u].x, ix[u].x, bv, bi);
        take(v[u].y, ix[u].y, bv, bi);
        take(v[u].z, ix[u].z, bv, bi);
        take(v[u].w, ix[u].w, bv, bi);
    }
}

// part_v and part_i are 16-byte aligned (the workspace is, and the rows
// start at a 256-byte offset); out[0] = the winning row, or -1 if no
// partial holds a number.  pos, if not null, is incremented by one.
__global__ void __launch_bounds__(kFinalThreads)
argmax_finalize_kernel(const float* __restrict__ part_v, const int32_t* __restrict__ part_i, int32_t count,
                       int32_t* __restrict__ out, int32_t* __restrict__ pos)
{
    __shared__ float sv[kFinalThreads / 64];
    __shared__ int32_t si[kFinalThreads / 64];
    const int tid = threadIdx.x;
    float bv = -__builtin_inff();
    int32_t bi = INT32_MAX;
    const int32_t n4 = count >> 2;
    // First loads, all without branches (a load inside a branch is waited
    // for where the paths join): the position, through an opaque VGPR zero
    // so that it is a vector load counted in order with the rest (part_i[0]
    // stands in when there is none; count >= 1), and the count % 4 tail,
    // clamped so that every thread may load it.  Nothing else writes the
    // position meanwhile, so advancing it costs no round trip of its own.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int32_t p0 = (pos ? pos : part_i)[zero];
    const int32_t tb = min((n4 << 2) + (tid & 3), count - 1);
    const float tv = part_v[tb];
    const int32_t ti = part_i[tb];
    const float4* pv4 = reinterpret_cast<const float4*>(part_v);
    const int4* pi4 = reinterpret_cast<const int4*>(part_i);
    // the first round is straight-line code: a loop here would have the
    // compiler wait for the loads above before entering it
    load_round(pv4, pi4, n4, tid, bv, bi);
    for (int32_t b0 = tid + kFinalThreads * kFinalVec; b0 < n4; b0 += kFinalThreads * kFinalVec)
        load_round(pv4, pi4, n4, b0, bv, bi);
    if (tid < (count & 3)) take(tv, ti, bv, bi);
    wave_best(bv, bi);
    if ((tid & 63) == 0) {
        sv[tid >> 6] = bv;
        si[tid >> 6] = bi;
    }
    __syncthreads();
    if (tid < 64) {
        bv = sv[tid & (kFinalThreads / 64 - 1)];
        bi = si[tid & (kFinalThreads / 64 - 1)];
        wave_best(bv, bi);
        if (tid == 0) {
            out[0] = (bi == INT32_MAX) ? -1 : bi;
            if (pos) *pos = p0 + 1;
        }
    }
}

}  // namespace

hipError_t launch_argmax_finalize(const float* part_v, const int32_t* part_i, int32_t count, int32_t* out,
                                  hipStream_t stream, int32_t* advance_pos)
{
    if (count < 1) return hipErrorInvalidValue;
    void* fargs[] = {&part_v, &part_i, &count, &out, &advance_pos};
    return hipLaunchKernel(reinterpret_cast<const void*>(&argmax_finalize_kernel), dim3(1), dim3(kFinalThreads),
                           fargs, 0, stream);
}

}  // namespace w4i
