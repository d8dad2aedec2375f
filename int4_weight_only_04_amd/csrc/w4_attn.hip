// Decode attention over a paged KV cache: the step between the QKV and o_proj
// projections of a decode token ("How To Build Your Own LLM Runtime From
// Scratch", aitrending.vip, "Technical Details", architecture bullet: paged
// KV cache and attention).  For query head h with KV head g = h / group:
//
//   s[t] = scale * q[h] . K[t][g],  p = softmax over t < ctx,  o[h] = sum_t p[t] V[t][g]
//
// Token t sits in physical page page_table[t / page] at slot t % page; the
// caches are fp16 [num_pages][n_kv][page][128].
//
// Two kernels.  The first splits the context into chunks of 128 tokens; a
// workgroup of 8 waves takes one chunk of one KV head, so K and V are read
// once for all the query heads that share them, and writes the chunk's
// softmax max, sum and unnormalised fp32 output.  The second merges the chunks in chunk order
// (deterministic).  The context length is read from device memory, so a
// captured graph replays unchanged from token to token; the grid is sized for
// max_ctx, and a chunk past the context exits before reading the cache (the
// combine uses only the chunks below the context).  A chunk's
// softmax covers every token in it, the page's tail included: all waves reach
// every barrier, and tokens past the context are masked, never skipped with
// an early exit (the barrier-in-a-branch mistake the pages describe corrupted
// exactly those tails: noticiai.com.br, "As tres licoes", lesson 1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"

namespace w4i {
namespace {

constexpr int kDim = 128;          // head dimension
constexpr int kChunk = 128;        // tokens per workgroup
constexpr int kAttnThreads = 512;  // 8 waves
constexpr int kWaves = kAttnThreads / 64;

struct AttnArgs {
    const uint4* q;          // fp16 [n_heads][128], 16 per head (not used with the fused rotary embedding)
    const uint4* kc;         // fp16 cache, 16 uint4 per token row
    const uint32_t* vc;      // fp16 cache, 64 words per token row
    const int32_t* table;    // page table
    const int32_t* ctx_ptr;  // device context length
    float* part_o;           // [chunks][n_heads][128]
    float* part_ml;          // [chunks][n_heads][2]: max, sum
    uint16_t* out;           // fp16 [n_heads][128]
    float scale;
    int32_t max_ctx;
    int32_t n_heads;
    int32_t n_kv;
    int32_t page_shift;
    int32_t num_pages;
    // fused rotary embedding + KV append (ROPE kernels): q and the new
    // token's k, v come from the fp32 QKV projection at position *pos
    const float* qkv;        // [(n_heads + 2 n_kv) * 128]: q heads, k heads, v heads
    const float* bias;       // same length, or null
    const int32_t* pos;
    int32_t* ctx_out;        // <- pos + 1 (the combine kernel's context length)
    uint16_t* q_out;         // fp16 [n_heads][128] or null (written by the chunk-0 workgroups)
    uint4* kc_w;             // the caches, written at the new token's slot
    uint32_t* vc_w;
    double theta;
    const float2* rope_cs;   // (cos, sin) per (position, pair)
};

__device__ __forceinline__ int clamp_ctx(const AttnArgs& a)
{
    int c = *a.ctx_ptr;
    if (c < 1) c = 1;
    if (c > a.max_ctx) c = a.max_ctx;
    return c;
}

// cache row index (in token rows) of token t of KV head g, from the raw
// page-table entry pg of t's page
__device__ __forceinline__ int64_t cache_row_of(const AttnArgs& a, int pg, int t, int g)
{
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);  // never read outside the cache
    return ((int64_t)pg * a.n_kv + g) * (1 << a.page_shift) + (t & ((1 << a.page_shift) - 1));
}

__device__ __forceinline__ int64_t cache_row(const AttnArgs& a, int t, int g)
{
    return cache_row_of(a, a.table[t >> a.page_shift], t, g);
}

__device__ __forceinline__ void half8_to_float(uint4 v, float (&f)[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
        f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
}

// Sum over each row of 16 lanes with DPP row shifts (no LDS traffic): lane 15
// of the row ends with the total.
__device__ __forceinline__ float row16_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xF, 0xF, true));
    return v;
}

// Maximum over each row of 16 lanes (lane 15 of the row ends with it); a lane
// whose source lies outside the row keeps its own value.
__device__ __forceinline__ float row16_max(float v)
{
#define W4A_MAX_STEP(ctrl)                                                                             \
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),      \
                                                                     __builtin_bit_cast(int, v), ctrl, \
                                                                     0xF, 0xF, false)))
    W4A_MAX_STEP(0x111);
    W4A_MAX_STEP(0x112);
    W4A_MAX_STEP(0x114);
    W4A_MAX_STEP(0x118);
#undef W4A_MAX_STEP
    return v;
}

// lane 15 + 16r of v, for the four rows r (uniform values)
__device__ __forceinline__ void row_totals(float v, float (&r)[4])
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        r[q] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * q + 15));
}

// the value of this lane's row among four uniform row values
__device__ __forceinline__ float of_row(const float (&r)[4], int lane)
{
    const int q = lane >> 4;
    return q == 0 ? r[0] : (q == 1 ? r[1] : (q == 2 ? r[2] : r[3]));
}

// Whole-wave maximum and sum (uniform results), from the row reductions and
// four lane reads: no LDS traffic.  The sum adds the rows in a fixed order.
__device__ __forceinline__ float wave_max(float v)
{
    float r[4];
    row_totals(row16_max(v), r);
    return fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
}

__device__ __forceinline__ float wave_sum(float v)
{
    float r[4];
    row_totals(row16_sum(v), r);
    return ((r[0] + r[1]) + r[2]) + r[3];
}

__device__ __forceinline__ float round_half(float v) { return (float)(_Float16)v; }

// Rotary embedding of the pair (i, i + 64) of the 128-wide head starting at
// row `base` of the QKV projection (plus bias), at position pos, with the
// (cos, sin) table of launch_rope_table (double-precision angles rounded to
// fp32, as the standalone rotary kernel computes them); rotation in fp32.
__device__ __forceinline__ void rope_pair(const AttnArgs& a, int64_t base, int i, int pos, float& r0, float& r1)
{
    float x0 = a.qkv[base + i], x1 = a.qkv[base + i + 64];
    if (a.bias) {
        x0 += a.bias[base + i];
        x1 += a.bias[base + i + 64];
    }
    const float2 t = a.rope_cs[(int64_t)pos * 64 + i];
    r0 = x0 * t.x - x1 * t.y;
    r1 = x1 * t.x + x0 * t.y;
}

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h4_t as_h4(uint32_t lo, uint32_t hi)
{
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    u2_t w;
    w.x = lo;
    w.y = hi;
    return __builtin_bit_cast(h4_t, w);
}

// Sum and maximum over the four 16-lane rows, per column (lanes l, l ^ 16,
// l ^ 32, l ^ 48): two lane-half swaps, every lane gets the result, and the
// lanes of one column add the same operands in the same order.
__device__ __forceinline__ float cols_sum(float v)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    const float p = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, p),
                                                    false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

__device__ __forceinline__ float cols_max(float v)
{
    const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    const float p = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, p), __builtin_bit_cast(uint32_t, p),
                                                    false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// GQ query heads per KV head (1..8).  Wave w of a workgroup takes the
// chunk's tokens [16w, 16w + 16) and runs both products of its part on the
// matrix cores (v_mfma_f32_16x16x16_f16: fp16 operands, exact products,
// fp32 sums), the query heads padded to 16 with zeros:
//   * scores S^T = K Q^T: the 128 dimensions are the reduction; lane
//     (row r = lane / 16, column c = lane % 16) supplies token c's K and head
//     c's q at dimensions 32 r + 4 s + (0..3) in step s, so each lane reads
//     64 contiguous bytes of one K row, and the result leaves lane (r, c)
//     with tokens 4r .. 4r + 3 of head c;
//   * that is the operand layout of P in O = P V, so the softmax weights
//     stay in registers (rounded to fp16 for the product; the sum of weights
//     is taken over the same rounded values);
//   * V is staged in LDS (each wave its own 16 rows, masked tokens as zeros,
//     padded rows so the four row groups fall in different banks), and
//     lane (r, c) reads tokens 4r .. 4r + 3 of dimension 16 n + c for tile n.
// The eight waves' parts are merged once, rescaled to the chunk maximum.
// ROPE: the query heads and the new token's key are rotated here from the
// QKV projection (fp16-rounded, as the stored q and cache are), and the new
// token's k and v are appended to the cache by the workgroup whose chunk
// holds it; that workgroup uses them directly, and no other workgroup reads
// that slot.
template <int GQ, bool ROPE>
__global__ void __launch_bounds__(kAttnThreads) attn_partial_kernel(AttnArgs a)
{
    constexpr int kVRow = kDim / 2 + 2;  // LDS words per staged V row (2 words of padding)
    __shared__ uint32_t s_v[kWaves][16][kVRow];
    __shared__ float s_o[kWaves][GQ][kDim];
    __shared__ float s_m[kWaves][GQ];     // per wave: its 16 tokens' maximum and sum of weights, per head
    __shared__ float s_l[kWaves][GQ];
    __shared__ float s_q[ROPE ? GQ : 1][kDim];
    __shared__ float s_knew[ROPE ? kDim : 1];
    __shared__ uint32_t s_vnew[ROPE ? kDim / 2 : 1];

    const int chunk = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t0 = chunk * kChunk;
    const int col = lane & 15;   // MFMA column: this lane's K token, q head, V dimension within a tile
    const int rg = lane >> 4;    // MFMA row group
    float* po = a.part_o + ((int64_t)chunk * a.n_heads + (int64_t)g * GQ) * kDim;
    float* pml = a.part_ml + ((int64_t)chunk * a.n_heads + (int64_t)g * GQ) * 2;

    // ---- first round, issued together: the context length (or position),
    // the page-table entries of this lane's K row and of the wave's 16 V rows
    // (tokens past max_ctx use the last one; the table holds an entry for
    // every token below max_ctx, so these reads are in bounds whatever the
    // context) and q.  Only then is the context length waited for: a chunk
    // past the context ends here, before any K/V traffic (the combine never
    // uses its partial).  Second round: the K and V rows, all issued before
    // any math (past the context they are masked below).  The length is
    // read as a vector load, through an index the compiler cannot fold, so
    // that it goes out first and the exit test waits for it alone (vector
    // loads are counted in issue order), not for the loads issued after it.
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const int raw_len = (ROPE ? a.pos : a.ctx_ptr)[zero];
    const int tk = t0 + wave * 16 + col;
    const int tkc = tk < a.max_ctx ? tk : a.max_ctx - 1;
    const int kpg = a.table[tkc >> a.page_shift];
    int vpg[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = t0 + wave * 16 + j;
        vpg[j] = a.table[(t < a.max_ctx ? t : a.max_ctx - 1) >> a.page_shift];
    }
    uint4 qv[4];
    if constexpr (!ROPE) {
        const int hq = col < GQ ? col : 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) qv[m] = a.q[(int64_t)(g * GQ + hq) * (kDim / 8) + rg * 4 + m];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int len = __builtin_amdgcn_readfirstlane(raw_len);  // the same in every lane
    int ctx, pos = -1;
    if constexpr (ROPE) {
        pos = len < 0 ? 0 : (len >= a.max_ctx ? a.max_ctx - 1 : len);
        ctx = pos + 1;
    } else {
        ctx = len < 1 ? 1 : (len > a.max_ctx ? a.max_ctx : len);
    }
    if (t0 >= ctx) return;  // whole workgroup, before any barrier
    const int64_t krow = cache_row_of(a, kpg, tkc, g);
    int64_t vrow[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = t0 + wave * 16 + j;
        vrow[j] = cache_row_of(a, vpg[j], t < a.max_ctx ? t : a.max_ctx - 1, g);
    }
    uint4 kv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) kv[m] = a.kc[krow * (kDim / 8) + rg * 4 + m];
    uint32_t vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) vv[j] = a.vc[vrow[j] * (kDim / 2) + lane];
    const bool has_new = ROPE && pos >= t0 && pos < t0 + kChunk;  // uniform per workgroup
    if constexpr (ROPE) {
        // rotate this workgroup's query heads (GQ x 64 pairs over 512
        // threads) and, in the workgroup holding the new token, its k and v
        if (t0 < ctx) {
            // at most one pair per thread (GQ <= 8): every load first, then the math
            constexpr int kPairs = (GQ * 64 + kAttnThreads - 1) / kAttnThreads;
            float x0[kPairs], x1[kPairs];
            float2 cs[kPairs];
#pragma unroll
            for (int k = 0; k < kPairs; ++k) {
                const int p = tid + k * kAttnThreads;
                if (p < GQ * 64) {
                    const int64_t base = (int64_t)(g * GQ + p / 64) * kDim;
                    const int i = p % 64;
                    x0[k] = a.qkv[base + i];
                    x1[k] = a.qkv[base + i + 64];
                    if (a.bias) {
                        x0[k] += a.bias[base + i];
                        x1[k] += a.bias[base + i + 64];
                    }
                    cs[k] = a.rope_cs[(int64_t)pos * 64 + i];
                }
            }
#pragma unroll
            for (int k = 0; k < kPairs; ++k) {
                const int p = tid + k * kAttnThreads;
                if (p < GQ * 64) {
                    const int h = p / 64, i = p % 64;
                    s_q[h][i] = round_half(x0[k] * cs[k].x - x1[k] * cs[k].y);
                    s_q[h][i + 64] = round_half(x1[k] * cs[k].x + x0[k] * cs[k].y);
                }
            }
            if (has_new) {
                if (tid < 64) {
                    float r0, r1;
                    rope_pair(a, (int64_t)(a.n_heads + g) * kDim, tid, pos, r0, r1);
                    s_knew[tid] = round_half(r0);
                    s_knew[tid + 64] = round_half(r1);
                } else if (tid < 128) {
                    const int w = tid - 64;  // dimensions 2w, 2w + 1
                    const int64_t vb = (int64_t)(a.n_heads + a.n_kv + g) * kDim + 2 * w;
                    float v0 = a.qkv[vb], v1 = a.qkv[vb + 1];
                    if (a.bias) {
                        v0 += a.bias[vb];
                        v1 += a.bias[vb + 1];
                    }
                    s_vnew[w] = pack_half2(v0, v1);
                }
            }
        }
        if (chunk == 0 && g == 0 && tid == 0 && a.ctx_out) *a.ctx_out = ctx;
        __syncthreads();
        if (has_new) {
            // append the new token to the cache (the stale slot was loaded
            // above; its registers are replaced below)
            const int64_t row = cache_row(a, pos, g);
            if (tid < 64) {
                reinterpret_cast<uint32_t*>(a.kc_w)[row * (kDim / 2) + tid] =
                    pack_half2(s_knew[2 * tid], s_knew[2 * tid + 1]);
            } else if (tid < 128) {
                a.vc_w[row * (kDim / 2) + (tid - 64)] = s_vnew[tid - 64];
            }
        }
        if (chunk == 0 && a.q_out) {
            for (int i = tid; i < GQ * kDim; i += kAttnThreads)
                a.q_out[(int64_t)g * GQ * kDim + i] = __builtin_bit_cast(uint16_t, (_Float16)s_q[i / kDim][i % kDim]);
        }
        const int hq = col < GQ ? col : 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float* qs = &s_q[hq][rg * 32 + m * 8];
            qv[m] = make_uint4(pack_half2(qs[0], qs[1]), pack_half2(qs[2], qs[3]), pack_half2(qs[4], qs[5]),
                               pack_half2(qs[6], qs[7]));
        }
        if (tk == pos) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float* ks = &s_knew[rg * 32 + m * 8];
                kv[m] = make_uint4(pack_half2(ks[0], ks[1]), pack_half2(ks[2], ks[3]), pack_half2(ks[4], ks[5]),
                                   pack_half2(ks[6], ks[7]));
            }
        }
    }

    // ---- stage this wave's V rows (tokens past the context as zeros, so a
    // row holding an infinity contributes exactly 0); only this wave reads
    // them, and a wave's LDS accesses complete in order
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = t0 + wave * 16 + j;
        const uint32_t keep = 0u - (uint32_t)(t < ctx);
        const uint32_t vw = (ROPE && t == pos) ? s_vnew[lane] : vv[j];
        s_v[wave][j][lane] = vw & keep;
    }

    // ---- scores S^T = K Q^T (heads past GQ get q = 0)
    const uint32_t qkeep = 0u - (uint32_t)(col < GQ);
    f4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const uint4& k4 = kv[st >> 1];
        const uint4& q4 = qv[st >> 1];
        const h4_t ka = (st & 1) ? as_h4(k4.z, k4.w) : as_h4(k4.x, k4.y);
        const h4_t qb = (st & 1) ? as_h4(q4.z & qkeep, q4.w & qkeep) : as_h4(q4.x & qkeep, q4.y & qkeep);
        sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(ka, qb, sacc, 0, 0, 0);
    }

    // ---- softmax over the wave's 16 tokens, per head (column): lane (r, c)
    // holds tokens 4r .. 4r + 3 of head c
    float sc[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + wave * 16 + rg * 4 + i;
        sc[i] = (t < ctx && col < GQ) ? sacc[i] * a.scale : -__builtin_inff();
        mx = fmaxf(mx, sc[i]);
    }
    const float m = cols_max(mx);
    float e[4], lsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // a token past the context, or a head past GQ, weighs exactly 0
        e[i] = (float)(_Float16)(sc[i] == -__builtin_inff() ? 0.0f : __expf(sc[i] - m));
        lsum += e[i];
    }
    const float l = cols_sum(lsum);
    const h4_t pa = as_h4(pack_half2(e[0], e[1]), pack_half2(e[2], e[3]));

    // ---- this wave's unnormalised output O = P V, 8 tiles of 16 dimensions
    const _Float16* vrowp = reinterpret_cast<const _Float16*>(&s_v[wave][rg * 4][0]);
    f4_t oacc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        h4_t vb;
#pragma unroll
        for (int i = 0; i < 4; ++i) vb[i] = vrowp[i * (2 * kVRow) + n * 16 + col];
        oacc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, f4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    }
    // lane (r, c) holds heads 4r .. 4r + 3 of dimensions 16 n + c
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = rg * 4 + i;
        if (h < GQ) {
#pragma unroll
            for (int n = 0; n < 8; ++n) s_o[wave][h][n * 16 + col] = oacc[n][i];
        }
    }
    if (rg == 0 && col < GQ) {
        s_m[wave][col] = m;
        s_l[wave][col] = l;
    }
    __syncthreads();

    // ---- the chunk's partial: the eight waves' parts rescaled to the chunk
    // maximum (finite: the chunk's first token is inside the context) and
    // added in wave order; a wave without a token in the context has maximum
    // -inf, weight 0 and sum 0
    for (int i = tid; i < GQ * kDim; i += kAttnThreads) {
        const int h = i / kDim, d = i % kDim;
        float mm = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][h]);
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o = __builtin_fmaf(__expf(s_m[w][h] - mm), s_o[w][h][d], o);
        po[i] = o;
    }
    if (tid < GQ) {
        float mm = s_m[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_m[w][tid]);
        float ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ls = __builtin_fmaf(__expf(s_m[w][tid] - mm), s_l[w][tid], ls);
        pml[2 * tid] = mm;
        pml[2 * tid + 1] = ls;
    }
}

// One workgroup of eight waves per query head; thread (j, d) = (tid / 128,
// tid % 128) adds dimension d over the chunks j, j + 4, ... in chunk order.
// Every wave finds the chunks' global maximum and sum of weights itself
// (lane c holds chunk c; row reductions and lane reads, uniform results), the
// chunk weights come from lane c by a lane read, and the four chunk lanes'
// sums meet once in LDS, added in a fixed order.
constexpr int kCombThreads = 512;

// The combine for workspaces of at most 4 NL chunks: every load in one
// round, with addresses that do not depend on the context length, so they
// travel together with its load: the lane's chunk (max, sum) and this
// thread's NL partials (chunks j, j + 4, ...).  Chunks past the context hold
// whatever an earlier call left there; they are only ever selected away,
// never multiplied.
template <int NL>
__device__ __forceinline__ void one_round(const AttnArgs& a, int h, int lane, int j, int cap, const float2* ml,
                                          const float* po, int64_t ostride, float& o, float& l)
{
    const int c = lane < cap ? lane : cap - 1;
    const float2 mc = ml[(int64_t)c * a.n_heads + h];
    float ov[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int cc = j + 4 * i;
        ov[i] = po[(int64_t)(cc < cap ? cc : cap - 1) * ostride];
    }
    // only now wait for the context length
    __builtin_amdgcn_sched_barrier(0);
    const int nch = (clamp_ctx(a) + kChunk - 1) / kChunk;   // 1 .. cap
    const float m = wave_max(lane < nch ? mc.x : -__builtin_inff());
    const float f = lane < nch ? __expf(mc.x - m) : 0.0f;
    l = wave_sum(f * (lane < nch ? mc.y : 0.0f));
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int cc = j + 4 * i;
        if (cc < nch) {
            const float fi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), cc));
            o = __builtin_fmaf(fi, ov[i], o);
        }
    }
}

__global__ void __launch_bounds__(kCombThreads) attn_combine_kernel(AttnArgs a)
{
    __shared__ float part[4][kDim];
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int d = tid & (kDim - 1);
    const int j = __builtin_amdgcn_readfirstlane(tid >> 7);  // uniform: a wave lies in one chunk lane
    const int cap = (a.max_ctx + kChunk - 1) / kChunk;  // chunks the workspace holds
    const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
    const float* po = a.part_o + (int64_t)h * kDim + d;
    const int64_t ostride = (int64_t)a.n_heads * kDim;
    float o = 0.0f, l;
    if (cap <= 32) {
        one_round<8>(a, h, lane, j, cap, ml, po, ostride, o, l);
    } else if (cap <= 64) {
        one_round<16>(a, h, lane, j, cap, ml, po, ostride, o, l);
    } else {
        // longer contexts: the maximum over all chunks first, then blocks of 64
        const int nch = (clamp_ctx(a) + kChunk - 1) / kChunk;
        float mx = -__builtin_inff();
        for (int c0 = 0; c0 < nch; c0 += 64) {
            const int c = c0 + lane;
            mx = fmaxf(mx, c < nch ? ml[(int64_t)c * a.n_heads + h].x : -__builtin_inff());
        }
        const float m = wave_max(mx);
        l = 0.0f;
        for (int c0 = 0; c0 < nch; c0 += 64) {
            const int c = c0 + lane;
            const float2 mc = ml[(int64_t)(c < nch ? c : nch - 1) * a.n_heads + h];
            const float f = c < nch ? __expf(mc.x - m) : 0.0f;
            l += wave_sum(f * (c < nch ? mc.y : 0.0f));
            for (int i = j; i < 64 && c0 + i < nch; i += 4) {
                const float fi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i));
                o = __builtin_fmaf(fi, po[(int64_t)(c0 + i) * ostride], o);
            }
        }
    }
    part[j][d] = o;
    __syncthreads();
    if (j == 0) {
        const float t = ((part[0][d] + part[1][d]) + part[2][d]) + part[3][d];
        a.out[(int64_t)h * kDim + d] = __builtin_bit_cast(uint16_t, (_Float16)(t / l));
    }
}

}  // namespace

int64_t attn_chunks(int32_t max_ctx)
{
    return (max_ctx + kChunk - 1) / kChunk;
}

size_t attn_workspace_bytes(int32_t n_heads, int32_t max_ctx)
{
    return (size_t)attn_chunks(max_ctx) * (size_t)n_heads * (kDim + 2) * sizeof(float);
}

template <bool ROPE>
const void* partial_fn(int group)
{
    switch (group) {
        case 1: return reinterpret_cast<const void*>(&attn_partial_kernel<1, ROPE>);
        case 2: return reinterpret_cast<const void*>(&attn_partial_kernel<2, ROPE>);
        case 3: return reinterpret_cast<const void*>(&attn_partial_kernel<3, ROPE>);
        case 4: return reinterpret_cast<const void*>(&attn_partial_kernel<4, ROPE>);
        case 5: return reinterpret_cast<const void*>(&attn_partial_kernel<5, ROPE>);
        case 6: return reinterpret_cast<const void*>(&attn_partial_kernel<6, ROPE>);
        case 7: return reinterpret_cast<const void*>(&attn_partial_kernel<7, ROPE>);
        case 8: return reinterpret_cast<const void*>(&attn_partial_kernel<8, ROPE>);
        default: return nullptr;
    }
}

hipError_t launch_attn(const AttnCall& c, hipStream_t stream)
{
    AttnArgs a{};
    a.q = static_cast<const uint4*>(c.q);
    a.kc = static_cast<const uint4*>(c.k_cache);
    a.vc = static_cast<const uint32_t*>(c.v_cache);
    a.table = c.page_table;
    a.ctx_ptr = c.ctx_len;
    const int64_t chunks = attn_chunks(c.max_ctx);
    a.part_o = static_cast<float*>(c.ws);
    a.part_ml = a.part_o + chunks * c.n_heads * kDim;
    a.out = c.out;
    a.scale = c.scale;
    a.max_ctx = c.max_ctx;
    a.n_heads = c.n_heads;
    a.n_kv = c.n_kv;
    int shift = 0;
    while ((1 << shift) < c.page_size) ++shift;
    a.page_shift = shift;
    a.num_pages = c.num_pages;
    const int group = c.n_heads / c.n_kv;
    if (c.rope) {
        const RopeCall& r = *c.rope;
        if (!r.table || !r.qkv || !r.pos || !r.k_cache || !r.v_cache || !r.ctx_out) return hipErrorInvalidValue;
        a.qkv = r.qkv;
        a.bias = r.bias;
        a.pos = r.pos;
        a.ctx_out = r.ctx_out;
        a.q_out = r.q_out;
        a.kc_w = reinterpret_cast<uint4*>(r.k_cache);
        a.vc_w = reinterpret_cast<uint32_t*>(r.v_cache);
        a.theta = r.theta;
        a.rope_cs = r.table;
        a.ctx_ptr = r.ctx_out;  // the combine kernel's context length
    }
    const void* fn = c.rope ? partial_fn<true>(group) : partial_fn<false>(group);
    if (!fn) return hipErrorInvalidValue;
    void* args[] = {&a};
    hipError_t err = hipLaunchKernel(fn, dim3((unsigned)chunks, (unsigned)c.n_kv), dim3(kAttnThreads), args, 0, stream);
    if (err != hipSuccess) return err;
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_combine_kernel), dim3((unsigned)c.n_heads),
                           dim3(kCombThreads), args, 0, stream);
}

}  // namespace w4i
