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
// Two kernels.  The first splits the context into chunks of 64 tokens; a
// workgroup takes one chunk of one KV head, so K and V are read once for all
// the query heads that share them, and writes the chunk's softmax max, sum
// and unnormalised fp32 output.  The second merges the chunks in chunk order
// (deterministic).  The context length is read from device memory, so a
// captured graph replays unchanged from token to token; the grid is sized for
// max_ctx, and a chunk past the context exits before reading the cache (the
// combine reads only the chunks below the context).  A chunk's
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
constexpr int kChunk = 64;         // tokens per workgroup
constexpr int kAttnThreads = 256;  // 4 waves

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

// cache row index (in token rows) of token t of KV head g
__device__ __forceinline__ int64_t cache_row(const AttnArgs& a, int t, int g)
{
    int pg = a.table[t >> a.page_shift];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);  // never read outside the cache
    return ((int64_t)pg * a.n_kv + g) * (1 << a.page_shift) + (t & ((1 << a.page_shift) - 1));
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

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
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

// GQ query heads per KV head (1..8).  ROPE: the query heads and the new
// token's key are rotated here from the QKV projection (fp16-rounded, as the
// stored q and cache are), and the new token's k and v are appended to the
// cache by the workgroup whose chunk holds it; that workgroup uses them
// directly, and no other workgroup reads that slot.
template <int GQ, bool ROPE>
__global__ void __launch_bounds__(kAttnThreads) attn_partial_kernel(AttnArgs a)
{
    __shared__ float s_sc[GQ][kChunk];
    __shared__ float s_o[4][GQ][kDim];
    __shared__ float s_m[GQ];
    __shared__ float s_l[GQ];
    __shared__ float s_q[ROPE ? GQ : 1][kDim];
    __shared__ float s_knew[ROPE ? kDim : 1];
    __shared__ uint32_t s_vnew[ROPE ? kDim / 2 : 1];

    const int chunk = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int t0 = chunk * kChunk;
    float* po = a.part_o + ((int64_t)chunk * a.n_heads + (int64_t)g * GQ) * kDim;
    float* pml = a.part_ml + ((int64_t)chunk * a.n_heads + (int64_t)g * GQ) * 2;

    // ---- first round: the context length (or position) and the page-table
    // entries of this lane's K and V rows; a chunk past the context ends
    // here, before any K/V traffic (the combine never reads its partial).
    // Second round: q and the K row slices and V words, all issued before any
    // math (rows of tokens past max_ctx are read from the last one; past the
    // context they are masked below).
    const int dpart = lane & 15;
    const int tq = lane >> 4;
    int64_t krow[4], vrow[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + wave * 16 + i * 4 + tq;
        krow[i] = cache_row(a, t < a.max_ctx ? t : a.max_ctx - 1, g);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int t = t0 + wave * 16 + j;
        vrow[j] = cache_row(a, t < a.max_ctx ? t : a.max_ctx - 1, g);
    }
    int ctx, pos = -1;
    if constexpr (ROPE) {
        pos = *a.pos;
        pos = pos < 0 ? 0 : (pos >= a.max_ctx ? a.max_ctx - 1 : pos);
        ctx = pos + 1;
    } else {
        ctx = clamp_ctx(a);
    }
    if (t0 >= ctx) return;  // whole workgroup, before any barrier
    uint4 qv[ROPE ? 1 : GQ];
    if constexpr (!ROPE) {
#pragma unroll
        for (int h = 0; h < GQ; ++h) qv[h] = a.q[(int64_t)(g * GQ + h) * (kDim / 8) + dpart];
    }
    uint4 kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = a.kc[krow[i] * (kDim / 8) + dpart];
    uint32_t vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) vv[j] = a.vc[vrow[j] * (kDim / 2) + lane];
    const bool has_new = ROPE && pos >= t0 && pos < t0 + kChunk;  // uniform per workgroup
    if constexpr (ROPE) {
        // rotate this workgroup's query heads (GQ x 64 pairs over 256
        // threads) and, in the workgroup holding the new token, its k and v
        if (t0 < ctx) {
            // at most two pairs per thread (GQ <= 8): every load first, then the math
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
                    s_vnew[w] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
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
                    (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s_knew[2 * tid]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s_knew[2 * tid + 1]) << 16);
            } else if (tid < 128) {
                a.vc_w[row * (kDim / 2) + (tid - 64)] = s_vnew[tid - 64];
            }
        }
        if (chunk == 0 && a.q_out) {
            for (int i = tid; i < GQ * kDim; i += kAttnThreads)
                a.q_out[(int64_t)g * GQ * kDim + i] = __builtin_bit_cast(uint16_t, (_Float16)s_q[i / kDim][i % kDim]);
        }
    }
    // ---- scores: 16 lanes per token, 8 dimensions per lane, 4 tokens per wave step
    float qr[GQ][8];
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        if constexpr (ROPE) {
#pragma unroll
            for (int j = 0; j < 8; ++j) qr[h][j] = s_q[h][8 * dpart + j];
        } else {
            half8_to_float(qv[h], qr[h]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tl = wave * 16 + i * 4 + tq;
        const bool valid = t0 + tl < ctx;
        float kf[8];
        half8_to_float(kv[i], kf);
        if (ROPE && t0 + tl == pos) {
#pragma unroll
            for (int j = 0; j < 8; ++j) kf[j] = s_knew[8 * dpart + j];
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            float d = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) d = __builtin_fmaf(qr[h][j], kf[j], d);
            d = row16_sum(d);  // total in lane 15 of each 16-lane row
            if (dpart == 15) s_sc[h][tl] = valid ? d * a.scale : -__builtin_inff();
        }
    }
    __syncthreads();

    // ---- chunk softmax: one wave per head, one lane per token
    for (int h = wave; h < GQ; h += 4) {
        const float v = s_sc[h][lane];
        const float m = wave_max(v);
        const float e = v == -__builtin_inff() ? 0.0f : __expf(v - m);
        const float l = wave_sum(e);
        s_sc[h][lane] = e;
        if (lane == 0) {
            s_m[h] = m;
            s_l[h] = l;
        }
    }
    __syncthreads();

    // ---- unnormalised output: wave w takes tokens [16w, 16w+16), lane = 2 dimensions
    float acc[GQ][2];
#pragma unroll
    for (int h = 0; h < GQ; ++h) acc[h][0] = acc[h][1] = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int tl = wave * 16 + j;
        // a token past the context (weight 0) contributes exactly 0, even if
        // the row it was read from holds an infinity
        const uint32_t keep = 0u - (uint32_t)(t0 + tl < ctx);
        const uint32_t vw = (ROPE && t0 + tl == pos) ? s_vnew[lane] : vv[j];
        const float v0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(vw & keep & 0xFFFFu));
        const float v1 = (float)__builtin_bit_cast(_Float16, (uint16_t)((vw & keep) >> 16));
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float w = s_sc[h][tl];  // 0 for tokens past the context
            acc[h][0] = __builtin_fmaf(w, v0, acc[h][0]);
            acc[h][1] = __builtin_fmaf(w, v1, acc[h][1]);
        }
    }
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
        s_o[wave][h][2 * lane] = acc[h][0];
        s_o[wave][h][2 * lane + 1] = acc[h][1];
    }
    __syncthreads();
    for (int i = tid; i < GQ * kDim; i += kAttnThreads) {
        const int h = i / kDim, d = i % kDim;
        po[i] = ((s_o[0][h][d] + s_o[1][h][d]) + s_o[2][h][d]) + s_o[3][h][d];
    }
    if (tid < GQ) {
        pml[2 * tid] = s_m[tid];
        pml[2 * tid + 1] = s_l[tid];
    }
}

// One workgroup per query head: the chunk maxima and sums are reduced across
// the workgroup, then thread (d, j) sums dimension d over the chunks j, j+8,
// ... with independent loads, and the eight partial sums meet in LDS in a
// fixed order.
constexpr int kCombThreads = 1024;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kCombThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(kCombThreads) attn_combine_kernel(AttnArgs a)
{
    constexpr int J = kCombThreads / kDim;  // 8 chunk lanes per dimension
    constexpr int kMaxPer = 8;              // chunks per thread held in registers
    __shared__ float red[kCombThreads / 64];
    __shared__ float part[J][kDim];
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int d = tid & (kDim - 1);
    const int j = tid / kDim;
    const int chunks = (a.max_ctx + kChunk - 1) / kChunk;
    const int ctx = clamp_ctx(a);
    const int nch = (ctx + kChunk - 1) / kChunk;
    // the first J * kMaxPer chunks: loads issued together, before the maxima
    float mv[kMaxPer], lv[kMaxPer], ov[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        int c = j + J * i;
        if (c >= chunks) c = chunks - 1;  // in bounds; masked below
        const float* ml = a.part_ml + ((int64_t)c * a.n_heads + h) * 2;
        mv[i] = ml[0];
        lv[i] = ml[1];
        ov[i] = a.part_o[((int64_t)c * a.n_heads + h) * kDim + d];
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i)
        if (j + J * i < nch) mx = fmaxf(mx, mv[i]);
    for (int c = j + J * kMaxPer; c < nch; c += J) mx = fmaxf(mx, a.part_ml[((int64_t)c * a.n_heads + h) * 2]);
    mx = block_reduce(mx, red, true);
    float l = 0.0f, o = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        if (j + J * i < nch) {
            const float f = __expf(mv[i] - mx);
            l = __builtin_fmaf(f, lv[i], l);
            o = __builtin_fmaf(f, ov[i], o);
        }
    }
    for (int c = j + J * kMaxPer; c < nch; c += J) {
        const float* ml = a.part_ml + ((int64_t)c * a.n_heads + h) * 2;
        const float f = __expf(ml[0] - mx);
        l = __builtin_fmaf(f, ml[1], l);
        o = __builtin_fmaf(f, a.part_o[((int64_t)c * a.n_heads + h) * kDim + d], o);
    }
    // every dimension's thread group holds the same l partials: sum them over j only
    part[j][d] = o;
    if (d == 0) red[j] = l;  // red is free again after block_reduce
    __syncthreads();
    if (j == 0) {
        float t = part[0][d], ls = red[0];
#pragma unroll
        for (int q = 1; q < J; ++q) {
            t += part[q][d];
            ls += red[q];
        }
        a.out[(int64_t)h * kDim + d] = __builtin_bit_cast(uint16_t, (_Float16)(t / ls));
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
