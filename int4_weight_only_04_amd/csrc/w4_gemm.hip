// Prefill GEMM over the INT4 weights: Y[m][n] = sum_k X[m][k] * w[n][k] for a
// block of prompt tokens (the 512-token prompt whose first-token latency the
// pages report: "How To Build Your Own LLM Runtime From Scratch",
// aitrending.vip, "Technical Details", performance-metrics bullet), with
// w[n][k] = (q[n][k] - 8) * s[n][k / G] read from the same W4T4 packed
// buffers as the decode GEMV.
//
// At M = 512 the product is a dense contraction (about 2000 flop per weight
// byte), so it runs on the matrix cores: each workgroup stages an M-tile of
// X and an N-tile of W, dequantized to fp16, in LDS and four waves multiply
// them with v_mfma_f32_32x32x16_f16 (fp16 operands, exact products, fp32
// accumulation).  Dequantizing rounds each weight once to fp16, a relative
// error of at most 2^-11 per weight, inside the 1e-3 * sum|w x| tolerance.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"

namespace w4i {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16x_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct GemmArgs {
    const uint4* pw;     // packed weights, 16 B per (tile, 8-input block)
    const uint2* ps;     // packed scales, 8 B per (tile, group)
    const uint4* x;      // fp16 [m][k] as 16-byte chunks (k / 8 per row)
    void* out;           // fp32 [m][n], or fp16 [m][n/2] for gate/up
    int64_t m;           // token rows
    int64_t n;           // weight rows (gate/up: 2I)
    int64_t tiles;       // W4T4 tiles
    int64_t tiles_half;  // gate/up: tiles per half
    int32_t kb;          // k / 8
    int32_t ng;          // k / G
    int32_t gshift;      // log2(G / 8)
    int32_t steps;       // ceil(kb / 8): k steps of 64 inputs
    int32_t splits;      // k ranges (blockIdx.z); > 1 writes fp32 partials [splits][m][n]
};

constexpr int kStepK = 64;                  // inputs per k step
constexpr int kRowHalves = kStepK + 8;      // LDS row: 64 fp16 + 16 B pad (conflict-free 16-B reads)
constexpr int kThreads = 256;               // 2 x 2 waves

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

// One 32-bit word of a W4T4 block holds the 8 nibbles of one row for 8
// consecutive inputs; slot p sits at bits [4p, 4p+4) and holds input 2p
// (p < 4) or 2(p-4)+1 (p >= 4), so the masks below pick input pairs
// (0,1), (2,3) / (4,5), (6,7) as fp16 lanes 1024+q or 1024+16q.  Returns
// the 8 weights (q - 8) * s rounded once to fp16, in input order.
__device__ __forceinline__ u32x4_t dequant_word(uint32_t d, uint32_t s2)
{
    const h2_t s = as_h2(s2);
    const h2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t d8 = d >> 8;
    const h2_t p01 = as_h2((d & 0x000F000Fu) | 0x64006400u) + lo_bias;
    const h2_t p23 = __builtin_elementwise_fma(as_h2((d & 0x00F000F0u) | 0x64006400u), sixteenth, hi_bias);
    const h2_t p45 = as_h2((d8 & 0x000F000Fu) | 0x64006400u) + lo_bias;
    const h2_t p67 = __builtin_elementwise_fma(as_h2((d8 & 0x00F000F0u) | 0x64006400u), sixteenth, hi_bias);
    u32x4_t r;
    r.x = as_u32(p01 * s);
    r.y = as_u32(p23 * s);
    r.z = as_u32(p45 * s);
    r.w = as_u32(p67 * s);
    return r;
}

// BM x BN output tile per workgroup (BM in {64, 128}, BN = 128; for gate/up
// the 128 weight rows are 64 gate rows and the matching 64 up rows).  Wave
// (wm, wn) owns a (BM/2) x (BN/2) quarter as (BM/64) x 2 blocks of 32 x 32;
// for gate/up its two n blocks are a gate block and the up block of the same
// outputs, so both land in the same lanes and registers.
//
// Pipeline: the global loads of k step s+RING go out while step s is
// computed (a ring of RING register slots, the loop unrolled by RING so every
// slot index is a constant).  With NBUF = 2 the LDS tiles are double-buffered,
// so one barrier per k step separates a step's LDS writes from its MFMA reads,
// and two 128-row workgroups share a CU.  With NBUF = 1 a second barrier per
// step keeps the next step's writes behind the current step's reads; the
// halved LDS and a 2-slot ring (within 168 registers) let three workgroups
// share a CU, which the gate/up shape (1184 workgroups, 1.5 rounds of 768
// instead of 2.3 rounds of 512) turns into a shorter kernel.  Loads are never
// predicated: past-the-end addresses are clamped in bounds and the values
// masked when stored to LDS (k tail: x and the scale zeroed, so the weight is
// 0; rows past m are read from the last row and never written out).
template <int BM, int BN, int EPI, int RING, int NBUF>
__global__ void __launch_bounds__(kThreads, NBUF == 2 ? 2 : 3) gemm_w4_kernel(GemmArgs a)
{
    constexpr int kRing = RING;
    static_assert(RING % 2 == 0, "consecutive k steps alternate LDS buffers by slot parity");
    static_assert(NBUF == 1 || NBUF == 2, "one or two LDS buffers");
    constexpr int MB = BM / 64;
    constexpr int NB = BN / 64;
    constexpr int XCHUNKS = BM * 8 / kThreads;          // 16-B chunks of X per thread per step
    constexpr int WITEMS = BN / 4 * 8;                   // (tile, block) items of W per step
    static_assert(BN == 128 && WITEMS == kThreads, "one W item per thread");
    __shared__ __attribute__((aligned(16))) _Float16 xs[NBUF][BM * kRowHalves];
    __shared__ __attribute__((aligned(16))) _Float16 wsm[NBUF][BN * kRowHalves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    // first output column of the tile (gate/up: first h column, 64 per tile)
    const int64_t c0 = (int64_t)blockIdx.x * (EPI == kEpiGateUp ? BN / 2 : BN);

    // X: chunk c = tid + kThreads * i -> tile row c / 8, 16-byte column c % 8
    int64_t xrow_off[XCHUNKS];
#pragma unroll
    for (int i = 0; i < XCHUNKS; ++i) {
        const int c = tid + kThreads * i;
        int64_t row = m0 + c / 8;
        if (row >= a.m) row = a.m - 1;
        xrow_off[i] = row * a.kb + (c % 8);
    }
    // W: thread tid -> LDS tile tt = tid / 8 (4 rows), 8-input block jj = tid % 8
    const int tt = tid / 8;
    const int jj = tid % 8;
    int64_t ptile;
    bool wok;
    if constexpr (EPI == kEpiGateUp) {
        const int64_t t = (int64_t)blockIdx.x * 16 + (tt % 16);  // tile within the half
        wok = t < a.tiles_half;
        ptile = (tt < 16 ? t : a.tiles_half + t);
    } else {
        ptile = (int64_t)blockIdx.x * (BN / 4) + tt;
        wok = ptile < a.tiles;
    }
    if (!wok) ptile = 0;
    const uint4* wbase = a.pw + ptile * a.kb;
    const uint2* sbase = a.ps + ptile * a.ng;

    struct Slot {
        uint4 x[XCHUNKS];
        uint4 w;
        uint2 s;
    };
    Slot ring[kRing];

    // k range of this split
    const int s_begin = (int)((int64_t)blockIdx.z * a.steps / a.splits);
    const int s_end = (int)((int64_t)(blockIdx.z + 1) * a.steps / a.splits);
    const int nsteps = s_end - s_begin;

    auto issue = [&](Slot& sl, int step) {
        if (step >= s_end) step = s_end - 1;  // in bounds, never stored
        const int blk0 = step * 8;
#pragma unroll
        for (int i = 0; i < XCHUNKS; ++i) {
            int blk = blk0 + ((tid + kThreads * i) % 8);
            if (blk >= a.kb) blk = a.kb - 1;
            sl.x[i] = a.x[xrow_off[i] - ((tid + kThreads * i) % 8) + blk];
        }
        int wblk = blk0 + jj;
        if (wblk >= a.kb) wblk = a.kb - 1;
        sl.w = wbase[wblk];
        sl.s = sbase[wblk >> a.gshift];
    };
    auto lstore = [&](const Slot& sl, int step, int b) {
        const int blk0 = step * 8;
#pragma unroll
        for (int i = 0; i < XCHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const uint32_t keep = 0u - (uint32_t)(blk0 + (c % 8) < a.kb);
            const uint4 v = make_uint4(sl.x[i].x & keep, sl.x[i].y & keep, sl.x[i].z & keep, sl.x[i].w & keep);
            *reinterpret_cast<uint4*>(&xs[b][(c / 8) * kRowHalves + (c % 8) * 8]) = v;
        }
        const uint32_t keep = 0u - (uint32_t)(wok && blk0 + jj < a.kb);
        const uint32_t wd[4] = {sl.w.x, sl.w.y, sl.w.z, sl.w.w};
        const uint32_t sx = sl.s.x & keep, sy = sl.s.y & keep;
        const uint32_t sd[4] = {sx & 0xFFFFu, sx >> 16, sy & 0xFFFFu, sy >> 16};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t s2 = sd[r] | (sd[r] << 16);
            *reinterpret_cast<u32x4_t*>(&wsm[b][(tt * 4 + r) * kRowHalves + jj * 8]) = dequant_word(wd[r], s2);
        }
    };

    f16x_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LDS rows each lane reads for its MFMA operands
    int arow[MB], brow[NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) arow[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if constexpr (EPI == kEpiGateUp)
            brow[j] = j * 64 + wn * 32 + (lane & 31);  // j = 0: gate rows, j = 1: up rows
        else
            brow[j] = wn * (BN / 2) + j * 32 + (lane & 31);
    }
    const int kofs = 8 * (lane >> 5);
    // One k step of 64 inputs: four MFMA rounds of 16 inputs.  The operands of
    // round kk + 1 are read from LDS into the second register set while round
    // kk's MFMAs run (issued one read after each MFMA), and the wave raises its
    // priority for the step (to 1; its LDS stores and loads run at 2, the rest
    // at 0) so that a SIMD issues MFMAs ahead of other waves' dequantization.
    auto mfma_step = [&](int b) {
        constexpr int KK = kStepK / 16;
        h8_t av[2][MB], bv[2][NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) av[0][i] = *reinterpret_cast<const h8_t*>(&xs[b][arow[i] * kRowHalves + kofs]);
#pragma unroll
        for (int j = 0; j < NB; ++j) bv[0][j] = *reinterpret_cast<const h8_t*>(&wsm[b][brow[j] * kRowHalves + kofs]);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            if (kk + 1 < KK) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    av[nxt][i] = *reinterpret_cast<const h8_t*>(&xs[b][arow[i] * kRowHalves + (kk + 1) * 16 + kofs]);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    bv[nxt][j] = *reinterpret_cast<const h8_t*>(&wsm[b][brow[j] * kRowHalves + (kk + 1) * 16 + kofs]);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
            if (kk + 1 < KK) {
                // alternate: one LDS read, one MFMA
#pragma unroll
                for (int q = 0; q < MB + NB; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

#pragma unroll
    for (int u = 0; u < kRing; ++u) issue(ring[u], s_begin + u);
    // whole groups of kRing steps: a branch-free body, so the compiler can wait
    // for exactly one slot's loads before each LDS store
    const int whole = nsteps - nsteps % kRing;
    for (int base = 0; base < whole; base += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            // keep each step's work in place: hoisting a later slot's dequant
            // above this point would make it wait for that slot's loads
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (NBUF == 1) __syncthreads();  // the previous step's reads are done
            // the LDS stores and the next global loads run above the MFMA
            // phase's priority: a workgroup reaches its barrier sooner and
            // the loads go out early
            __builtin_amdgcn_s_setprio(2);
            lstore(ring[u], s_begin + base + u, (u & 1) % NBUF);
            issue(ring[u], s_begin + base + u + kRing);
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            mfma_step((u & 1) % NBUF);
        }
    }
    // the last nsteps % kRing steps (their slots are the first ones of the ring)
#pragma unroll
    for (int u = 0; u < kRing - 1; ++u) {
        if (whole + u < nsteps) {
            if constexpr (NBUF == 1) __syncthreads();
            __builtin_amdgcn_s_setprio(2);
            lstore(ring[u], s_begin + whole + u, (u & 1) % NBUF);
            __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            mfma_step((u & 1) % NBUF);
        }
    }

    // ---- epilogue: register r of lane l holds row 8(r/4) + 4(l/32) + r%4, column l%32 of its block
    const int col_in = lane & 31;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
            if (row >= a.m) continue;
            if constexpr (EPI == kEpiGateUp) {
                const int64_t half = a.n >> 1;
                const int64_t j = c0 + wn * 32 + col_in;
                if (j < half) {
                    const float g = acc[i][0][r];
                    const float silu = g / (1.0f + __expf(-g));
                    const _Float16 hv = (_Float16)(silu * acc[i][1][r]);
                    reinterpret_cast<_Float16*>(a.out)[row * half + j] = hv;
                }
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int64_t col = c0 + wn * (BN / 2) + j * 32 + col_in;
                    if (col < a.n)
                        reinterpret_cast<float*>(a.out)[(int64_t)blockIdx.z * a.m * a.n + row * a.n + col] = acc[i][j][r];
                }
            }
        }
    }
}

// y = sum of the split partials, in split order (deterministic).  A thread
// owns E elements, 256 apart so that every load instruction of a wave reads
// 256 consecutive floats, and issues all E x S loads before adding: one
// memory round trip per thread instead of one per element and split.
constexpr int kReduceThreads = 256;

template <int S, int E>
__global__ void __launch_bounds__(kReduceThreads) gemm_reduce_kernel(const float* __restrict__ part,
                                                                     float* __restrict__ y, int64_t count)
{
    const int64_t base = (int64_t)blockIdx.x * (kReduceThreads * E) + threadIdx.x;
    float v[E][S];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = base + e * kReduceThreads;
        const int64_t ic = i < count ? i : count - 1;   // in bounds; the sum is not stored
#pragma unroll
        for (int sp = 0; sp < S; ++sp) v[e][sp] = part[(int64_t)sp * count + ic];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = base + e * kReduceThreads;
        float t = v[e][0];
#pragma unroll
        for (int sp = 1; sp < S; ++sp) t += v[e][sp];
        if (i < count) y[i] = t;
    }
}

template <int S>
hipError_t launch_reduce(const float* part, float* y, int64_t count, hipStream_t stream)
{
    constexpr int E = S <= 4 ? 8 : 4;   // at most 32 loads in flight per thread
    const int64_t blocks = (count + kReduceThreads * E - 1) / (kReduceThreads * E);
    if (blocks < 1 || blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    void* rargs[] = {&part, &y, &count};
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_reduce_kernel<S, E>), dim3((unsigned)blocks),
                           dim3(kReduceThreads), rargs, 0, stream);
}

struct GemmPlan {
    const void* fn;
    dim3 grid;
    GemmArgs args;
};

GemmPlan make_gemm_plan(const GemmCall& c)
{
    const bool gateup = c.epi == kEpiGateUp;
    GemmPlan p{};
    GemmArgs& a = p.args;
    a.pw = static_cast<const uint4*>(c.pw);
    a.ps = static_cast<const uint2*>(c.ps);
    a.x = static_cast<const uint4*>(c.x);
    a.out = c.out;
    a.m = c.m;
    a.n = c.n;
    a.kb = (int32_t)(c.k / 8);
    a.ng = (int32_t)(c.k / c.group);
    int gshift = 0;
    while ((8 << gshift) < c.group) ++gshift;
    a.gshift = gshift;
    a.steps = (a.kb + 7) / 8;
    a.tiles = tiles_for(c.n, gateup);
    a.tiles_half = gateup ? a.tiles / 2 : 0;
    const GemmShape sh = choose_gemm_shape(c.epi, c.m, c.n);
    const int64_t cols = gateup ? c.n / 2 : c.n;
    const int64_t per_tile = gateup ? sh.bn / 2 : sh.bn;
    a.splits = gemm_splits(c.epi, c.m, c.n, c.k);
    if (a.splits > 1) a.out = c.ws;
    p.grid = dim3((unsigned)((cols + per_tile - 1) / per_tile), (unsigned)((c.m + sh.bm - 1) / sh.bm),
                  (unsigned)a.splits);
    if (gateup)
        p.fn = sh.bm == 128 ? reinterpret_cast<const void*>(&gemm_w4_kernel<128, 128, kEpiGateUp, 2, 1>)
                            : reinterpret_cast<const void*>(&gemm_w4_kernel<64, 128, kEpiGateUp, 4, 2>);
    else
        p.fn = sh.bm == 128 ? reinterpret_cast<const void*>(&gemm_w4_kernel<128, 128, kEpiPlain, 2, 2>)
                            : reinterpret_cast<const void*>(&gemm_w4_kernel<64, 128, kEpiPlain, 4, 2>);
    return p;
}

}  // namespace

hipError_t launch_gemm(const GemmCall& c, hipStream_t stream)
{
    GemmPlan p = make_gemm_plan(c);
    if (!p.fn) return hipErrorInvalidValue;
    void* args[] = {&p.args};
    hipError_t err = hipLaunchKernel(p.fn, p.grid, dim3(kThreads), args, 0, stream);
    if (err != hipSuccess || p.args.splits == 1) return err;
    const float* part = static_cast<const float*>(c.ws);
    float* y = static_cast<float*>(c.out);
    const int64_t count = c.m * c.n;
    switch (p.args.splits) {
        case 2: return launch_reduce<2>(part, y, count, stream);
        case 3: return launch_reduce<3>(part, y, count, stream);
        case 4: return launch_reduce<4>(part, y, count, stream);
        case 5: return launch_reduce<5>(part, y, count, stream);
        case 6: return launch_reduce<6>(part, y, count, stream);
        case 7: return launch_reduce<7>(part, y, count, stream);
        case 8: return launch_reduce<8>(part, y, count, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4i
