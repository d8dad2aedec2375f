// INT4 weight-only GEMV kernels for MI355X (gfx950, CDNA4, wave64).
//
// What is computed ("How To Build Your Own LLM Runtime From Scratch",
// aitrending.vip, "Technical Details" bullet 1: INT4 weights dequantized at
// run time; noticiai.com.br, "As tres licoes" lesson 3: activations stay
// floating point): y[n] = sum_k (q[n][k] - 8) * s[n][k/G] * x[k], with fp16
// x and s, exact dequantization and fp32 accumulation, plus fused epilogues
// (SiLU-gated gate/up, lm_head argmax, residual add) and an RMSNorm prologue.
//
// Design (one GEMV is a pure HBM stream: 0.52 bytes per weight against 2
// flops, far below the chip's ridge point, so the kernel is shaped for
// bandwidth, not for MFMA):
//   * A "unit" is one W4T4 tile of 4 rows (plain, argmax) or a gate tile and
//     the matching up tile (gate/up, 8 rows).  SPLIT waves of a workgroup
//     share a unit, each taking a contiguous range of its k iterations; a
//     k iteration is 64 lanes x one 8-input block, so every weight load is a
//     16-byte load and a wave instruction reads 1 KiB of contiguous packed
//     weights per tile.  The partial sums of the SPLIT waves meet in LDS and
//     are added in wave order, so results do not depend on scheduling.
//   * Each wave issues all its loads for a round (D iterations: weights,
//     group scales and the 16 bytes of x its lane needs) before any math, so
//     a unit's whole k range is in flight at once.  x is read through the
//     L1/L2 caches (it is shared by every workgroup and small).
//   * The 16 bytes a lane loads are the same 8 inputs of the tile's 4 rows,
//     so one 16-byte read of x serves 4 (or 8) rows.
//   * Unpacking costs 5 integer ops per 8 nibbles (masks 0x000F000F /
//     0x00F000F0 OR-ed into the fraction of fp16 1024.0, before and after a
//     shift by 8), 4 packed-fp16 ops to remove the bias exactly (1024+q-1032
//     and (1024+16q)/16-72 are both exactly q-8), and 4 v_dot2_f32_f16 whose
//     products are exact in fp32; one mixed-precision fma per row and block
//     applies the group scale.  This is the gfx950 counterpart of the pages'
//     lesson that a byte-permute unpack beat an integer dot product for these
//     shapes ("Technical Details" bullet 4): keep the per-weight instruction
//     count low and stay in floating point for the activations.
//   * Per-row sums are reduced across the wave with DPP row operations and
//     four lane reads.
//   * Every wave of a workgroup reaches each barrier; tail units and lanes
//     are masked, never returned early before one (the pages'
//     warp-specialisation bug, "Technical Details" bullet 4, was a barrier
//     inside a divergent branch).
//   * lm_head argmax: each workgroup writes its best (value, row) to the
//     workspace with plain stores and a one-workgroup second kernel
//     (w4_argmax.hip) reduces them.  The kernel boundary orders the two, so
//     there are no device-scope fences or atomics on the hot path.
//   * Decode-step forms: the residual epilogue adds y into the fp32 residual
//     stream and writes one sum of squares of the new rows per unit; the
//     RMSNorm prologue (x mode kXNorm) takes h, gamma and those sums instead
//     of x.  Every wave sums the partials in one fixed order, so every
//     workgroup forms the same x = fp16((h * r) * gamma); the partials are
//     loaded before the weights, and each iteration's x is made from its own
//     h and gamma loads, so the weight stream is not held up.  The kernel
//     boundary between producer and consumer orders the partial sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "w4_gemv_math.h"
#include "w4_internal.h"

namespace w4i {
namespace {

using namespace gemv_math;


struct KernelArgs {
    const uint4* pw;
    const uint2* ps;
    const uint4* x;      // fp16 x, or (W4A8) int8 codes as uint2 per 8-input block
    const float* xs;     // W4A8: activation scale per group
    void* out;
    float* part_v;       // argmax: per-workgroup best value
    int32_t* part_i;     // argmax: per-workgroup best row
    int64_t n;           // logical rows (gate/up: 2I)
    int64_t units;       // units (tiles, or gate/up tile pairs)
    int64_t tiles_half;  // gate/up: tiles per half
    int64_t tiles;       // tiles in the packed matrix
    int32_t kb;          // k / 8
    int32_t ng;          // k / G
    int32_t gshift;      // log2(G / 8)
    int32_t iters;       // ceil(kb / 64)
    // residual epilogue (plain; h_out non-null): h_out = h_in + y, ss_out[unit] = sum of h_out^2 of the unit's rows
    const float* h_in;
    float* h_out;
    float* ss_out;
    // RMSNorm prologue (x mode kXNorm): x = fp16(h * r * gamma), r from the partial sums of squares
    const float4* nh;    // h fp32 [k], two float4 per 8-input block
    const uint4* ngamma; // gamma fp16 [k], one uint4 per 8-input block
    const float4* nss;   // partial sums of squares, padded to whole float4
    int32_t nparts;      // number of partial sums
    float nk;            // k as fp32 (the mean's divisor)
    float neps;
    uint4* x_out;        // workgroup 0 writes the fp16 x it used (or null)
};

// Where a GEMV takes its input from: fp16 x, int8 codes with per-group scales
// (W4A8), or fp32 h normalized on the fly (RMSNorm prologue).
enum XMode : int { kXHalf = 0, kXCodes = 1, kXNorm = 2 };


// RMSNorm prologue, step 1: lane l loads float4 l, l + 64, ... of the partial
// sums of squares.  Indices past the last float4 are clamped to it (the buffer
// is padded to whole float4, so every load is in bounds and unconditional);
// reduce_parts masks what lies past nparts.
__device__ __forceinline__ void load_parts(float4 (&pv)[kNormPartLoads], const float4* __restrict__ nss, int nparts,
                                           int lane)
{
    const int last = ((nparts + 3) >> 2) - 1;
#pragma unroll
    for (int p = 0; p < kNormPartLoads; ++p) {
        const int i = p * 64 + lane;
        pv[p] = nss[i < last ? i : last];
    }
}

// Step 2: r = 1 / sqrt(S / k + eps), S summed in a fixed order (each lane's 16
// values in index order, then a butterfly across the wave, which leaves the
// same sum in every lane), so every wave of every workgroup gets the same r.
__device__ __forceinline__ float reduce_parts(const float4 (&pv)[kNormPartLoads], int nparts, int lane, float nk,
                                              float eps)
{
    float t = 0.0f;
#pragma unroll
    for (int p = 0; p < kNormPartLoads; ++p) {
        const int b = 4 * (p * 64 + lane);
        t += b + 0 < nparts ? pv[p].x : 0.0f;
        t += b + 1 < nparts ? pv[p].y : 0.0f;
        t += b + 2 < nparts ? pv[p].z : 0.0f;
        t += b + 3 < nparts ? pv[p].w : 0.0f;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
    return 1.0f / sqrtf(t / nk + eps);
}

__device__ __forceinline__ uint32_t half_pair(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Step 3: the 8 fp16 inputs of one block, x = fp16((h * r) * gamma).
__device__ __forceinline__ uint4 normed_block(const float4& h0, const float4& h1, const uint4& g, float r)
{
    return make_uint4(half_pair(h0.x * r * half_lo(g.x), h0.y * r * half_hi(g.x)),
                      half_pair(h0.z * r * half_lo(g.y), h0.w * r * half_hi(g.y)),
                      half_pair(h1.x * r * half_lo(g.z), h1.y * r * half_hi(g.z)),
                      half_pair(h1.z * r * half_lo(g.w), h1.w * r * half_hi(g.w)));
}

// Lane N of each 16-lane row, broadcast to every lane of that row (DPP
// row_newbcast:N).
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + N, 0xF, 0xF, false);
}

// the same for n = 0..7, a constant once the caller's loop is unrolled
__device__ __forceinline__ uint32_t row_bcast(uint32_t v, int n)
{
    switch (n) {
        case 0: return row_bcast<0>(v);
        case 1: return row_bcast<1>(v);
        case 2: return row_bcast<2>(v);
        case 3: return row_bcast<3>(v);
        case 4: return row_bcast<4>(v);
        case 5: return row_bcast<5>(v);
        case 6: return row_bcast<6>(v);
        default: return row_bcast<7>(v);
    }
}

// Straight-line body for exactly C k iterations of one wave: all loads first
// (weights and scales non-temporal, x through L1), then the math for each
// iteration in order.  With no branches between the loads the compiler's
// wait counters are exact, so iteration d waits only for its own loads and
// its math overlaps the loads still in flight (with branches it falls back to
// waiting for every load before any math).
// RS (groups of 128 inputs or more, C <= 8): a 16-lane row's 16 blocks of an
// iteration then share one scale word per tile, so one load per tile brings
// every iteration's words: lane 16 q + d loads row q's word of iteration d
// (lanes past C repeat iteration C - 1's), and the math broadcasts it to the
// row.  That is one scale load per tile instead of one per iteration.
template <int C, int U, int XM, bool RS>
__device__ __forceinline__ void accumulate_exact(float (&acc)[U][4], const uint4* const (&wp)[U],
                                                 const uint2* const (&sp)[U], const bool (&tile_ok)[U],
                                                 const KernelArgs& a, int i0, int lane, uint32_t magic, bool write_x)
{
    static_assert(!RS || C <= 8, "row_bcast covers 8 iterations");
    uint4 w[C][U];
    uint2 s[C][U];      // per iteration (without RS)
    uint2 srow[U];      // every iteration's, one word per lane (RS)
    uint4 xr[C];
    uint2 cr[C];
    float sx[C];
    float4 hv[C][2];
    uint4 gv[C];
    float4 pv[kNormPartLoads];
    // The callers branch between C = D and C = D - 1; the two bodies begin
    // with the same loads, and the compiler would hoist those above the branch
    // (keeping them live across it and reordering the waits).  An assembler
    // comment that differs per C makes the bodies differ from the first
    // instruction on.
    asm volatile("; accumulate_exact %0 iterations, row scales %1" ::"n"(C), "n"(RS ? 1 : 0));
    // the norm's partial sums go first, so waiting for them does not wait
    // for the weight stream issued after them
    if constexpr (XM == kXNorm) load_parts(pv, a.nss, a.nparts, lane);
    if constexpr (RS) {
        const int dl = (lane & 15) < C ? (lane & 15) : C - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) srow[u] = ld_stream(sp[u] + (((i0 + dl) * 64 + (lane & 48)) >> a.gshift));
    }
#pragma unroll
    for (int d = 0; d < C; ++d) {
        const int j = (i0 + d) * 64 + lane;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            w[d][u] = ld_stream(wp[u] + j);
            if constexpr (!RS) s[d][u] = ld_stream(sp[u] + (j >> a.gshift));
        }
        if constexpr (XM == kXCodes) {
            cr[d] = reinterpret_cast<const uint2*>(a.x)[j];
            sx[d] = a.xs[j >> a.gshift];
        } else if constexpr (XM == kXNorm) {
            hv[d][0] = a.nh[2 * j];
            hv[d][1] = a.nh[2 * j + 1];
            gv[d] = a.ngamma[j];
        } else {
            xr[d] = a.x[j];
        }
    }
    float r = 0.0f;
    if constexpr (XM == kXNorm) {
        // keep every load above the reduction: it waits only for the partial
        // sums, while the weight stream stays in flight
        __builtin_amdgcn_sched_barrier(0);
        r = reduce_parts(pv, a.nparts, lane, a.nk, a.neps);
    }
#pragma unroll
    for (int d = 0; d < C; ++d) {
        // iteration d's x from its own h and gamma loads only
        if constexpr (XM == kXNorm) xr[d] = normed_block(hv[d][0], hv[d][1], gv[d], r);
        int n8 = 0;
        if constexpr (XM == kXCodes) n8 = neg8_code_sum(cr[d]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // a unit's missing second tile reads tile 0 (in bounds) with its
            // scales masked to zero (a mask, not a select, so the scale load
            // stays unconditional and in issue order)
            const uint32_t keep = 0u - (uint32_t)tile_ok[u];
            const uint2 sr = RS ? make_uint2(row_bcast(srow[u].x, d), row_bcast(srow[u].y, d)) : s[d][u];
            const uint2 sc = make_uint2(sr.x & keep, sr.y & keep);
            if constexpr (XM == kXCodes) {
                acc[u][0] = __builtin_fmaf((float)idot8(w[d][u].x, cr[d], n8), half_lo(sc.x) * sx[d], acc[u][0]);
                acc[u][1] = __builtin_fmaf((float)idot8(w[d][u].y, cr[d], n8), half_hi(sc.x) * sx[d], acc[u][1]);
                acc[u][2] = __builtin_fmaf((float)idot8(w[d][u].z, cr[d], n8), half_lo(sc.y) * sx[d], acc[u][2]);
                acc[u][3] = __builtin_fmaf((float)idot8(w[d][u].w, cr[d], n8), half_hi(sc.y) * sx[d], acc[u][3]);
            } else {
                acc[u][0] = __builtin_fmaf(dot8(w[d][u].x, xr[d], magic), half_lo(sc.x), acc[u][0]);
                acc[u][1] = __builtin_fmaf(dot8(w[d][u].y, xr[d], magic), half_hi(sc.x), acc[u][1]);
                acc[u][2] = __builtin_fmaf(dot8(w[d][u].z, xr[d], magic), half_lo(sc.y), acc[u][2]);
                acc[u][3] = __builtin_fmaf(dot8(w[d][u].w, xr[d], magic), half_hi(sc.y), acc[u][3]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (XM == kXNorm) {
        // after the math, so the branch does not split the load/math block
        if (write_x) {
#pragma unroll
            for (int d = 0; d < C; ++d) a.x_out[(i0 + d) * 64 + lane] = xr[d];
        }
    }
}

constexpr int waves_for(int split) { return split < 4 ? 4 : split; }

// U tiles per unit, epilogue EPI, SPLIT waves per unit, D iterations per load
// round, FULL: k/8 is a multiple of 64 (no lane masking), XM: where the input
// comes from (fp16 x, int8 codes, or fp32 h through the RMSNorm prologue).
template <int U, int EPI, int SPLIT, int D, bool FULL, int XM>
__global__ void __launch_bounds__(waves_for(SPLIT) * 64) gemv_w4_kernel(KernelArgs a)
{
    constexpr int WAVES = waves_for(SPLIT);
    constexpr int SLOTS = WAVES / SPLIT;
    __shared__ float red[SLOTS][SPLIT][U][4];
    __shared__ float best_v_s[SLOTS];
    __shared__ int32_t best_i_s[SLOTS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = wave / SPLIT;
    const int sub = wave % SPLIT;
    const uint32_t magic = opaque_magic();
    const int64_t unit = (int64_t)blockIdx.x * SLOTS + slot;
    const bool live = unit < a.units;
    const int it0 = sub * a.iters / SPLIT;
    const int it1 = (sub + 1) * a.iters / SPLIT;
    const bool writer = (lane & 15) == 0;   // one lane per reduced row
    const int row_in_tile = reduced_row(lane);
    // workgroup 0's first slot covers every k iteration: it writes the normalized x
    const bool write_x = XM == kXNorm && a.x_out != nullptr && blockIdx.x == 0 && slot == 0;

    // tiles of this unit (plain U == 2: tiles 2u and 2u+1, the second may be
    // past the end; gate/up: tile u and its up partner)
    bool tile_ok[U];
    int64_t tile_of[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        tile_of[u] = (EPI == kEpiGateUp) ? unit + u * a.tiles_half : unit * U + u;
        tile_ok[u] = live && (EPI == kEpiGateUp || tile_of[u] < a.tiles);
    }

    // residual epilogue: the owner wave fetches h_in of its rows up front (a
    // clamped, in-bounds index; rows past n are masked at the end)
    float hin[U];
#pragma unroll
    for (int u = 0; u < U; ++u) hin[u] = 0.0f;
    if constexpr (EPI == kEpiPlain) {
        if (a.h_out != nullptr && sub == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t row = tile_of[u] * 4 + row_in_tile;
                hin[u] = a.h_in[row < a.n ? row : a.n - 1];
            }
        }
    }

    float acc[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = 0.0f;

    const int count = it1 - it0;  // this wave's k iterations (uniform)
    if (live && FULL && (count == D || count == D - 1)) {
        const uint4* wp[U];
        const uint2* sp[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = tile_ok[u] ? tile_of[u] : 0;
            wp[u] = a.pw + t * a.kb;
            sp[u] = a.ps + t * a.ng;
        }
        if (a.gshift >= 4) {  // G >= 128: a 16-lane row lies in one group
            if (count == D)
                accumulate_exact<D, U, XM, true>(acc, wp, sp, tile_ok, a, it0, lane, magic, write_x);
            else if constexpr (D > 1)
                accumulate_exact<D - 1, U, XM, true>(acc, wp, sp, tile_ok, a, it0, lane, magic, write_x);
        } else {
            if (count == D)
                accumulate_exact<D, U, XM, false>(acc, wp, sp, tile_ok, a, it0, lane, magic, write_x);
            else if constexpr (D > 1)
                accumulate_exact<D - 1, U, XM, false>(acc, wp, sp, tile_ok, a, it0, lane, magic, write_x);
        }
    } else if (live) {
        const uint4* wp[U];
        const uint2* sp[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wp[u] = a.pw + tile_of[u] * a.kb;
            sp[u] = a.ps + tile_of[u] * a.ng;
        }
        float r = 0.0f;
        if constexpr (XM == kXNorm) {
            if (it0 < it1) {
                float4 pv[kNormPartLoads];
                load_parts(pv, a.nss, a.nparts, lane);
                r = reduce_parts(pv, a.nparts, lane, a.nk, a.neps);
            }
        }
        for (int i0 = it0; i0 < it1; i0 += D) {
            uint4 w[D][U];
            uint2 s[D][U];
            uint4 xr[D];
            uint2 cr[D];
            float sx[D];
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = (i0 + d) * 64 + lane;
                if ((i0 + d < it1) && (FULL || j < a.kb)) {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (tile_ok[u]) {
                            w[d][u] = ld_stream(wp[u] + j);
                            s[d][u] = ld_stream(sp[u] + (j >> a.gshift));
                        } else {
                            w[d][u] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
                            s[d][u] = make_uint2(0, 0);
                        }
                    }
                    if constexpr (XM == kXCodes) {
                        cr[d] = reinterpret_cast<const uint2*>(a.x)[j];
                        sx[d] = a.xs[j >> a.gshift];
                    } else if constexpr (XM == kXNorm) {
                        xr[d] = normed_block(a.nh[2 * j], a.nh[2 * j + 1], a.ngamma[j], r);
                        if (write_x) a.x_out[j] = xr[d];
                    } else {
                        xr[d] = a.x[j];
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int j = (i0 + d) * 64 + lane;
                if ((i0 + d < it1) && (FULL || j < a.kb)) {
                    if constexpr (XM == kXCodes) {
                        const int n8 = neg8_code_sum(cr[d]);
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            acc[u][0] = __builtin_fmaf((float)idot8(w[d][u].x, cr[d], n8), half_lo(s[d][u].x) * sx[d],
                                                       acc[u][0]);
                            acc[u][1] = __builtin_fmaf((float)idot8(w[d][u].y, cr[d], n8), half_hi(s[d][u].x) * sx[d],
                                                       acc[u][1]);
                            acc[u][2] = __builtin_fmaf((float)idot8(w[d][u].z, cr[d], n8), half_lo(s[d][u].y) * sx[d],
                                                       acc[u][2]);
                            acc[u][3] = __builtin_fmaf((float)idot8(w[d][u].w, cr[d], n8), half_hi(s[d][u].y) * sx[d],
                                                       acc[u][3]);
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            acc[u][0] = __builtin_fmaf(dot8(w[d][u].x, xr[d], magic), half_lo(s[d][u].x), acc[u][0]);
                            acc[u][1] = __builtin_fmaf(dot8(w[d][u].y, xr[d], magic), half_hi(s[d][u].x), acc[u][1]);
                            acc[u][2] = __builtin_fmaf(dot8(w[d][u].z, xr[d], magic), half_lo(s[d][u].y), acc[u][2]);
                            acc[u][3] = __builtin_fmaf(dot8(w[d][u].w, xr[d], magic), half_hi(s[d][u].y), acc[u][3]);
                        }
                    }
                }
            }
        }
    }

    // per tile: the sum of row reduced_row(lane) in every lane of its 16-lane row
    float rv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) rv[u] = reduce4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);

    if constexpr (SPLIT > 1) {
        if (writer) {
#pragma unroll
            for (int u = 0; u < U; ++u) red[slot][sub][u][row_in_tile] = rv[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float t = red[slot][0][u][row_in_tile];
#pragma unroll
            for (int q = 1; q < SPLIT; ++q) t += red[slot][q][u][row_in_tile];
            rv[u] = t;
        }
    }
    const bool owner = live && sub == 0;  // the wave that writes this unit's outputs

    if constexpr (EPI == kEpiGateUp) {
        const int64_t j = unit * 4 + row_in_tile;
        if (owner && writer && j < (a.n >> 1)) {
            const float g = rv[0];
            const float silu = g / (1.0f + __expf(-g));
            const _Float16 hv = (_Float16)(silu * rv[1]);
            reinterpret_cast<uint16_t*>(a.out)[j] = __builtin_bit_cast(uint16_t, hv);
        }
    } else {
        float* y = reinterpret_cast<float*>(a.out);
        float bv = -__builtin_inff();
        int32_t bi = INT32_MAX;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = tile_of[u] * 4 + row_in_tile;
            if (owner && row < a.n) {
                if (writer) y[row] = rv[u];
                if (EPI == kEpiArgmax && better(rv[u], (int32_t)row, bv, bi)) {
                    bv = rv[u];
                    bi = (int32_t)row;
                }
            }
        }
        if constexpr (EPI == kEpiPlain) {
            if (a.h_out != nullptr && owner) {
                // h_out = h_in + y; the unit's sum of squares of h_out, its tile
                // rows added as (r0 + r2) + (r1 + r3) (every lane of a 16-lane
                // row holds that row's value), then its tiles in order
                float ss = 0.0f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t row = tile_of[u] * 4 + row_in_tile;
                    const bool ok = row < a.n;
                    const float hn = hin[u] + rv[u];
                    if (ok && writer) a.h_out[row] = hn;
                    float sq = ok ? hn * hn : 0.0f;
                    sq += __shfl_xor(sq, 16);
                    sq += __shfl_xor(sq, 32);
                    ss += sq;
                }
                if (lane == 0) a.ss_out[unit] = ss;
            }
        }
        if constexpr (EPI == kEpiArgmax) {
            // the 4 rows of each tile sit in the 4 16-lane rows: reduce across them
#pragma unroll
            for (int off = 16; off < 64; off <<= 1) {
                const float ov = __shfl_xor(bv, off);
                const int32_t oi = __shfl_xor(bi, off);
                if (better(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (sub == 0 && lane == 0) {
                best_v_s[slot] = bv;
                best_i_s[slot] = bi;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                float v = best_v_s[0];
                int32_t i = best_i_s[0];
#pragma unroll
                for (int q = 1; q < SLOTS; ++q)
                    if (better(best_v_s[q], best_i_s[q], v, i)) {
                        v = best_v_s[q];
                        i = best_i_s[q];
                    }
                a.part_v[blockIdx.x] = v;
                a.part_i[blockIdx.x] = i;
            }
        }
    }
}

// ----------------------------------------------------------------- launch table

// Instantiated (split, depth) pairs: depth is the number of k iterations a
// wave loads per round before computing.
template <int U, int EPI, int XM>
const void* pick(int split, int depth, bool full)
{
#define W4_CASE(S, D)                                                                         \
    if (split == S && depth == D)                                                             \
        return full ? reinterpret_cast<const void*>(&gemv_w4_kernel<U, EPI, S, D, true, XM>) \
                    : reinterpret_cast<const void*>(&gemv_w4_kernel<U, EPI, S, D, false, XM>);
    // split 1 happens only with a single k iteration (k <= 512), hence depth 2,
    // for every unit size (tall matrices with short rows included)
    W4_CASE(1, 2)
    if constexpr (U == 1 || EPI == kEpiGateUp) {
        W4_CASE(4, 2)
        W4_CASE(4, 4)
        W4_CASE(4, 8)
        W4_CASE(8, 2)
        W4_CASE(8, 5)
        W4_CASE(8, 8)
    }
    W4_CASE(2, 2)
    W4_CASE(2, 4)
    W4_CASE(2, 8)
#undef W4_CASE
    return nullptr;
}

template <int XM>
const void* pick_epi(int32_t epi, const LaunchConfig& cfg, bool full)
{
    if (epi == kEpiGateUp) return pick<2, kEpiGateUp, XM>(cfg.split, cfg.depth, full);
    if (epi == kEpiPlain)
        return cfg.tiles == 2 ? pick<2, kEpiPlain, XM>(cfg.split, cfg.depth, full)
                              : pick<1, kEpiPlain, XM>(cfg.split, cfg.depth, full);
    if (epi == kEpiArgmax)
        return cfg.tiles == 2 ? pick<2, kEpiArgmax, XM>(cfg.split, cfg.depth, full)
                              : pick<1, kEpiArgmax, XM>(cfg.split, cfg.depth, full);
    return nullptr;
}

struct Plan {
    const void* fn;
    int threads;
    int64_t grid;
    KernelArgs args;
};

Plan make_plan(const GemvCall& c)
{
    const bool gateup = c.epi == kEpiGateUp;
    Plan p{};
    KernelArgs& a = p.args;
    a.pw = static_cast<const uint4*>(c.pw);
    a.ps = static_cast<const uint2*>(c.ps);
    a.x = static_cast<const uint4*>(c.x);
    a.xs = c.xs;
    a.out = c.out;
    a.n = c.n;
    a.kb = (int32_t)(c.k / 8);
    a.ng = (int32_t)(c.k / c.group);
    int gshift = 0;
    while ((8 << gshift) < c.group) ++gshift;
    a.gshift = gshift;
    a.iters = (a.kb + 63) / 64;
    a.tiles = tiles_for(c.n, gateup);
    a.tiles_half = gateup ? a.tiles / 2 : 0;
    const LaunchConfig cfg = choose_config(c.epi, gateup ? a.tiles / 2 : a.tiles, a.iters);
    a.units = gateup ? a.tiles / 2 : (a.tiles + cfg.tiles - 1) / cfg.tiles;
    const bool full = (a.kb % 64) == 0;
    if (c.norm_h)
        p.fn = pick_epi<kXNorm>(c.epi, cfg, full);
    else if (c.xs)
        p.fn = pick_epi<kXCodes>(c.epi, cfg, full);
    else
        p.fn = pick_epi<kXHalf>(c.epi, cfg, full);
    a.h_in = c.h_in;
    a.h_out = c.h_out;
    a.ss_out = c.ss_out;
    a.nh = reinterpret_cast<const float4*>(c.norm_h);
    a.ngamma = reinterpret_cast<const uint4*>(c.norm_gamma);
    a.nss = reinterpret_cast<const float4*>(c.norm_ss);
    a.nparts = (int32_t)c.norm_parts;
    a.nk = (float)c.k;
    a.neps = c.norm_eps;
    a.x_out = reinterpret_cast<uint4*>(c.x_out);
    const int waves = waves_for(cfg.split);
    const int slots = waves / cfg.split;
    p.threads = waves * 64;
    p.grid = (a.units + slots - 1) / slots;
    if (c.epi == kEpiArgmax) {
        uint8_t* ws = static_cast<uint8_t*>(c.ws);
        a.part_v = reinterpret_cast<float*>(ws);
        a.part_i = reinterpret_cast<int32_t*>(ws + argmax_index_offset(p.grid));
    }
    return p;
}

}  // namespace

// Device memory of the allocation-free argmax entry point: the per-workgroup
// (value, row) partials live in this file-scope array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends.  In host code the name is only a stand-in for the symbol, so
// its device address is looked up once per device (hipGetSymbolAddress) and
// only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int64_t launch_grid(const GemvCall& c)
{
    return make_plan(c).grid;
}

int64_t residual_parts(int64_t n, int64_t k, int32_t group)
{
    GemvCall c{};
    c.n = n;
    c.k = k;
    c.group = group;
    c.epi = kEpiPlain;
    return make_plan(c).args.units;
}

hipError_t launch_gemv(const GemvCall& c, hipStream_t stream, int32_t* advance_pos)
{
    Plan p = make_plan(c);
    if (!p.fn) return hipErrorInvalidValue;
    if (p.grid < 1 || p.grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    void* args[] = {&p.args};
    hipError_t err = hipLaunchKernel(p.fn, dim3((unsigned)p.grid), dim3(p.threads), args, 0, stream);
    if (err != hipSuccess || c.epi != kEpiArgmax) return err;
    return launch_argmax_finalize(p.args.part_v, p.args.part_i, (int32_t)p.grid, c.argmax, stream, advance_pos);
}

}  // namespace w4i
