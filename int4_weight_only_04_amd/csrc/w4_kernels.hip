// INT4 weight-only GEMV kernels for MI355X (gfx950, CDNA4, wave64).
//
// What is computed ("How To Build Your Own LLM Runtime From Scratch",
// aitrending.vip, "Technical Details" bullet 1: INT4 weights dequantized at
// run time; noticiai.com.br, "As tres licoes" lesson 3: activations stay
// floating point): y[n] = sum_k (q[n][k] - 8) * s[n][k/G] * x[k], with fp16
// x and s, exact dequantization and fp32 accumulation, plus two fused
// epilogues (SiLU-gated gate/up, lm_head argmax).
//
// Design (one GEMV is a pure HBM stream: 0.52 bytes per weight against 2
// flops, far below the chip's ridge point, so the kernel is shaped for
// bandwidth, not for MFMA):
//   * A wave owns one "unit" at a time: one W4T4 tile of 4 rows (plain,
//     argmax) or the gate tile and the matching up tile (gate/up, 8 rows).
//     Its 64 lanes stride along k in 8-input blocks, so every weight load is a
//     16-byte global load and a wave instruction reads 1 KiB of contiguous
//     packed weights per tile.
//   * The 16 bytes a lane loads are the same 8 inputs of the tile's 4 rows,
//     so one 16-byte LDS read of x serves 4 (or 8) rows.  x is staged once per
//     workgroup in LDS; the grid is sized to the resident capacity and waves
//     walk units with a grid stride, so the staging is amortised.
//   * Unpacking costs 5 integer ops per 8 nibbles (masks 0x000F000F /
//     0x00F000F0 OR-ed into the fraction of fp16 1024.0, before and after a
//     shift by 8), 4 packed-fp16 ops to remove the bias exactly (1024+q-1032
//     and (1024+16q)/16-72 are both exactly q-8), and 4 v_dot2_f32_f16 whose
//     products are exact in fp32.  One fma per row and block applies the
//     group scale.  This is the gfx950 counterpart of the pages' lesson that
//     a byte-permute unpack beat an integer dot product for these shapes
//     ("Technical Details" bullet 4): keep the per-weight instruction count
//     low, stay in floating point for the activations.
//   * Per-row sums are reduced across the wave with DPP row operations and
//     four lane reads; no LDS is used for the reduction.
//   * Tail rows are masked, never returned early: every wave reaches every
//     barrier (the pages' warp-specialisation bug, "Technical Details"
//     bullet 4, was a barrier inside a divergent branch).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "w4_internal.h"

namespace w4i {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kDepth = 8;  // 16-byte weight loads in flight per lane and tile

struct KernelArgs {
    const uint4* pw;
    const uint2* ps;
    const uint4* x;
    void* out;
    int32_t* argmax;
    uint8_t* ws;
    int64_t n;           // logical rows (gate/up: 2I)
    int64_t units;       // wave units
    int64_t tiles_half;  // gate/up: tiles per half
    int32_t kb;          // k / 8
    int32_t ng;          // k / G
    int32_t gshift;      // log2(G / 8)
};

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
    float p = __builtin_amdgcn_fdot2(va, as_h2(xv.x), 0.0f, false);
    p = __builtin_amdgcn_fdot2(vb, as_h2(xv.y), p, false);
    p = __builtin_amdgcn_fdot2(vc, as_h2(xv.z), p, false);
    p = __builtin_amdgcn_fdot2(ve, as_h2(xv.w), p, false);
    return p;
}

__device__ __forceinline__ float half_lo(uint32_t v) { return (float)as_h2(v)[0]; }
__device__ __forceinline__ float half_hi(uint32_t v) { return (float)as_h2(v)[1]; }

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane receives the same bits (each DPP step
// adds a lane to its mirror image, so all lanes of a row add the same two
// values, and fp addition is commutative).
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ bool better(float v, int32_t i, float bv, int32_t bi)
{
    return v > bv || (v == bv && i < bi);
}

template <int U, int EPI>
__global__ void __launch_bounds__(kBlockThreads) gemv_w4_kernel(KernelArgs a)
{
    extern __shared__ uint4 xs[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    for (int i = tid; i < a.kb; i += kBlockThreads) xs[i] = a.x[i];
    __syncthreads();

    const int iters = (a.kb + 63) >> 6;
    const uint32_t magic = opaque_magic();
    float best_v = -__builtin_inff();
    int32_t best_i = INT32_MAX;

    for (int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + wave; unit < a.units;
         unit += (int64_t)gridDim.x * kWavesPerBlock) {
        const uint4* wp[U];
        const uint2* sp[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tile = (EPI == kEpiGateUp) ? unit + u * a.tiles_half : unit * U + u;
            wp[u] = a.pw + tile * a.kb;
            sp[u] = a.ps + tile * a.ng;
        }
        float acc[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] = 0.0f;

        for (int i0 = 0; i0 < iters; i0 += kDepth) {
            uint4 w[kDepth][U];
            uint2 s[kDepth][U];
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int j = (i0 + d) * 64 + lane;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (j < a.kb) {
                        w[d][u] = wp[u][j];
                        s[d][u] = sp[u][j >> a.gshift];
                    } else {
                        w[d][u] = make_uint4(0, 0, 0, 0);
                        s[d][u] = make_uint2(0, 0);
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < kDepth; ++d) {
                const int j = (i0 + d) * 64 + lane;
                if (j < a.kb) {
                    const uint4 xv = xs[j];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        acc[u][0] = __builtin_fmaf(dot8(w[d][u].x, xv, magic), half_lo(s[d][u].x), acc[u][0]);
                        acc[u][1] = __builtin_fmaf(dot8(w[d][u].y, xv, magic), half_hi(s[d][u].x), acc[u][1]);
                        acc[u][2] = __builtin_fmaf(dot8(w[d][u].z, xv, magic), half_lo(s[d][u].y), acc[u][2]);
                        acc[u][3] = __builtin_fmaf(dot8(w[d][u].w, xv, magic), half_hi(s[d][u].y), acc[u][3]);
                    }
                }
            }
        }

#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] = wave_sum(acc[u][r]);

        if constexpr (EPI == kEpiGateUp) {
            const int64_t half = a.n >> 1;
            uint16_t* h = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t j = unit * 4 + r;
                if (j < half && lane == r) {
                    const float g = acc[0][r];
                    const float up = acc[1][r];
                    const float silu = g / (1.0f + __expf(-g));
                    const _Float16 hv = (_Float16)(silu * up);
                    h[j] = __builtin_bit_cast(uint16_t, hv);
                }
            }
        } else {
            float* y = reinterpret_cast<float*>(a.out);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = unit * 4 + r;
                if (row < a.n) {
                    if (lane == r) y[row] = acc[0][r];
                    if constexpr (EPI == kEpiArgmax) {
                        if (better(acc[0][r], (int32_t)row, best_v, best_i)) {
                            best_v = acc[0][r];
                            best_i = (int32_t)row;
                        }
                    }
                }
            }
        }
    }

    if constexpr (EPI == kEpiArgmax) {
        // Deterministic two-level argmax: each block publishes its best
        // (value, row) to the workspace; the last block to finish (counted
        // with one device-scope atomic) reduces the partials in index order
        // and re-arms the counter, so the workspace is reusable and the
        // result is independent of block scheduling.
        __shared__ float red_v[kBlockThreads];
        __shared__ int32_t red_i[kBlockThreads];
        __shared__ int is_last;
        uint32_t* counter = reinterpret_cast<uint32_t*>(a.ws);
        float* part_v = reinterpret_cast<float*>(a.ws + kArgmaxHeaderBytes);
        int32_t* part_i = reinterpret_cast<int32_t*>(a.ws + kArgmaxHeaderBytes) + kArgmaxMaxBlocks;
        if (lane == 0) {
            red_v[wave] = best_v;
            red_i[wave] = best_i;
        }
        __syncthreads();
        if (tid == 0) {
            float bv = red_v[0];
            int32_t bi = red_i[0];
            for (int w = 1; w < kWavesPerBlock; ++w)
                if (better(red_v[w], red_i[w], bv, bi)) {
                    bv = red_v[w];
                    bi = red_i[w];
                }
            part_v[blockIdx.x] = bv;
            part_i[blockIdx.x] = bi;
            __threadfence();
            const uint32_t done = atomicAdd(counter, 1u);
            is_last = (done == gridDim.x - 1) ? 1 : 0;
        }
        __syncthreads();
        if (is_last) {
            __threadfence();
            float bv = -__builtin_inff();
            int32_t bi = INT32_MAX;
            for (int b = tid; b < (int)gridDim.x; b += kBlockThreads) {
                const float v = __builtin_nontemporal_load(part_v + b);
                const int32_t i = __builtin_nontemporal_load(part_i + b);
                if (better(v, i, bv, bi)) {
                    bv = v;
                    bi = i;
                }
            }
            red_v[tid] = bv;
            red_i[tid] = bi;
            __syncthreads();
            for (int stride = kBlockThreads / 2; stride > 0; stride >>= 1) {
                if (tid < stride && better(red_v[tid + stride], red_i[tid + stride], red_v[tid], red_i[tid])) {
                    red_v[tid] = red_v[tid + stride];
                    red_i[tid] = red_i[tid + stride];
                }
                __syncthreads();
            }
            if (tid == 0) {
                a.argmax[0] = (red_i[0] == INT32_MAX) ? -1 : red_i[0];
                atomicExch(counter, 0u);
            }
        }
    }
}

const void* kernel_for(int32_t epi)
{
    switch (epi) {
        case kEpiPlain: return reinterpret_cast<const void*>(&gemv_w4_kernel<1, kEpiPlain>);
        case kEpiArgmax: return reinterpret_cast<const void*>(&gemv_w4_kernel<1, kEpiArgmax>);
        case kEpiGateUp: return reinterpret_cast<const void*>(&gemv_w4_kernel<2, kEpiGateUp>);
        default: return nullptr;
    }
}

// Resident workgroups per device for a kernel and LDS size (cached).
hipError_t resident_blocks(const void* fn, size_t lds, int* out)
{
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, size_t>, int> cache;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const auto key = std::make_tuple(dev, fn, lds);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            *out = it->second;
            return hipSuccess;
        }
    }
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlockThreads, lds);
    if (err != hipSuccess) return err;
    if (per_cu < 1) per_cu = 1;
    const int total = cus * per_cu;
    {
        std::lock_guard<std::mutex> lock(mu);
        cache[key] = total;
    }
    *out = total;
    return hipSuccess;
}

}  // namespace

hipError_t prepare_gemv(const GemvCall& c)
{
    const void* fn = kernel_for(c.epi);
    if (!fn) return hipErrorInvalidValue;
    int resident = 0;
    return resident_blocks(fn, (size_t)(c.k / 8) * 16, &resident);
}

hipError_t launch_gemv(const GemvCall& c, hipStream_t stream)
{
    const bool gateup = c.epi == kEpiGateUp;
    KernelArgs a;
    a.pw = static_cast<const uint4*>(c.pw);
    a.ps = static_cast<const uint2*>(c.ps);
    a.x = static_cast<const uint4*>(c.x);
    a.out = c.out;
    a.argmax = c.argmax;
    a.ws = static_cast<uint8_t*>(c.ws);
    a.n = c.n;
    a.kb = (int32_t)(c.k / 8);
    a.ng = (int32_t)(c.k / c.group);
    int gshift = 0;
    while ((8 << gshift) < c.group) ++gshift;
    a.gshift = gshift;
    const int64_t tiles = tiles_for(c.n, gateup);
    a.tiles_half = gateup ? tiles / 2 : 0;
    a.units = gateup ? tiles / 2 : tiles;

    const void* fn = kernel_for(c.epi);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = (size_t)a.kb * 16;
    int resident = 0;
    hipError_t err = resident_blocks(fn, lds, &resident);
    if (err != hipSuccess) return err;
    int64_t grid = (a.units + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid > resident) grid = resident;
    if (c.epi == kEpiArgmax && grid > kArgmaxMaxBlocks) grid = kArgmaxMaxBlocks;
    if (grid < 1) grid = 1;
    void* args[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kBlockThreads), args, lds, stream);
}

}  // namespace w4i
