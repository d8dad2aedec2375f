// Glue kernels of a full decode step around the INT4 projections and the
// paged attention: embedding lookup, residual add + RMSNorm, and the rotary
// embedding with the KV-cache append (the position advance runs in the
// lm_head argmax's finalize kernel).  The pages' runtime is
// a Qwen2.5-Coder-7B decoding stack ("How To Build Your Own LLM Runtime From
// Scratch", aitrending.vip, TL;DR and "Technical Details"); its glue is read
// as the Qwen2-family pre-norm decoder:
//
//   h = E[token];  per layer:  x = rmsnorm(h) g1;  q,k,v = x Wqkv;  rope(q, k);
//   append k, v;  h += o_proj(attn(q));  x = rmsnorm(h) g2;  h += down(silu(gate) up)
//   then x = rmsnorm(h) g_f and the next token is argmax(x Wlm).
//
// The token id, the position and the attention's context length live in
// device memory and are advanced on the device, so one captured graph of
// the whole step replays token after token with no host work in between.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"
#include "w4_wave.h"

namespace w4i {
namespace {

constexpr int kNormThreads = 1024;

__device__ __forceinline__ float half_to_float(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t float_to_half(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// h[i] = table[token][i] (fp16 -> fp32); an id outside the table is clamped.
__global__ void __launch_bounds__(256) embed_kernel(const uint16_t* __restrict__ table, int64_t vocab, int64_t hidden,
                                                    const int32_t* __restrict__ token, float* __restrict__ h)
{
    int64_t t = *token;
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    const uint16_t* row = table + t * hidden;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hidden; i += (int64_t)gridDim.x * blockDim.x)
        h[i] = half_to_float(row[i]);
}

// One workgroup: h += y (fp32, when y is given), then
// x = fp16(h * g / sqrt(mean(h^2) + eps)).  The sum of squares is reduced in a
// fixed order (per-thread strided sums, then a tree: DPP row sums and the four
// row totals, then the waves in order), so it is deterministic.
__global__ void __launch_bounds__(kNormThreads) add_rmsnorm_kernel(float* __restrict__ h, const float* __restrict__ y,
                                                                   const uint16_t* __restrict__ gamma, int64_t n,
                                                                   float eps, uint16_t* __restrict__ x)
{
    __shared__ float red[kNormThreads / 64];
    const int tid = threadIdx.x;
    float ss = 0.0f;
    for (int64_t i = tid; i < n; i += kNormThreads) {
        float v = h[i];
        if (y) {
            v += y[i];
            h[i] = v;
        }
        ss = __builtin_fmaf(v, v, ss);
    }
    ss = wave::wave_sum_tree(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += red[w];
    const float r = 1.0f / sqrtf(tot / (float)n + eps);
    for (int64_t i = tid; i < n; i += kNormThreads) x[i] = float_to_half(h[i] * r * half_to_float(gamma[i]));
}


// One workgroup: h = table[token] (fp16 -> fp32), then the first layer's
// RMSNorm x = fp16(h * g / sqrt(mean(h^2) + eps)), the same reduction as
// add_rmsnorm_kernel.
__global__ void __launch_bounds__(kNormThreads) embed_rmsnorm_kernel(const uint16_t* __restrict__ table, int64_t vocab,
                                                                     int64_t n, const int32_t* __restrict__ token,
                                                                     const uint16_t* __restrict__ gamma, float eps,
                                                                     float* __restrict__ h, uint16_t* __restrict__ x)
{
    __shared__ float red[kNormThreads / 64];
    int64_t t = *token;
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    const uint16_t* row = table + t * n;
    const int tid = threadIdx.x;
    float ss = 0.0f;
    for (int64_t i = tid; i < n; i += kNormThreads) {
        const float v = half_to_float(row[i]);
        h[i] = v;
        ss = __builtin_fmaf(v, v, ss);
    }
    ss = wave::wave_sum_tree(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += red[w];
    const float r = 1.0f / sqrtf(tot / (float)n + eps);
    for (int64_t i = tid; i < n; i += kNormThreads) x[i] = float_to_half(h[i] * r * half_to_float(gamma[i]));
}

// Vector forms of the two norm kernels, used when n % 4 == 0 and
// n <= 16 x kNormThreads with aligned buffers: each thread owns up to
// kNormVec float4 of the vector, issues every load (h, y or the embedding
// row, gamma) before any arithmetic, keeps the values in registers and
// writes h and x once -- one memory round trip instead of one per strided
// iteration.  The sum of squares is reduced in a fixed order.
constexpr int kNormVec = 4;

__device__ __forceinline__ float block_sum(float v, float* red)
{
    // each wave's total through DPP row sums and lane reads (depth 6, as a
    // 6-level butterfly), without the LDS round trips of lane shuffles
    v = wave::wave_sum_tree(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += red[w];
    return tot;
}

__device__ __forceinline__ float4 f4_from_halves(uint2 g)
{
    return make_float4(half_to_float((uint16_t)(g.x & 0xFFFFu)), half_to_float((uint16_t)(g.x >> 16)),
                       half_to_float((uint16_t)(g.y & 0xFFFFu)), half_to_float((uint16_t)(g.y >> 16)));
}

__device__ __forceinline__ uint2 halves_from_f4(float4 v)
{
    return make_uint2((uint32_t)float_to_half(v.x) | ((uint32_t)float_to_half(v.y) << 16),
                      (uint32_t)float_to_half(v.z) | ((uint32_t)float_to_half(v.w) << 16));
}

// x = fp16(v * r * gamma) for this thread's float4s, r from the block sum of squares.
__device__ __forceinline__ void finish_norm4(const float4 (&v)[kNormVec], const uint2 (&g)[kNormVec], float ss,
                                             int32_t n4, float eps, uint2* __restrict__ x4, float* red)
{
    const float tot = block_sum(ss, red);
    const float r = 1.0f / sqrtf(tot / (float)(4 * n4) + eps);
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int i = u * kNormThreads + threadIdx.x;
        if (i < n4) {
            const float4 gv = f4_from_halves(g[u]);
            x4[i] = halves_from_f4(make_float4(v[u].x * r * gv.x, v[u].y * r * gv.y, v[u].z * r * gv.z,
                                               v[u].w * r * gv.w));
        }
    }
}

__global__ void __launch_bounds__(kNormThreads) add_rmsnorm4_kernel(float4* __restrict__ h, const float4* __restrict__ y,
                                                                    const uint2* __restrict__ gamma, int32_t n4,
                                                                    float eps, uint2* __restrict__ x)
{
    __shared__ float red[kNormThreads / 64];
    float4 v[kNormVec], yv[kNormVec];
    uint2 g[kNormVec];
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int i = u * kNormThreads + threadIdx.x;
        if (i < n4) {
            v[u] = h[i];
            if (y) yv[u] = y[i];
            g[u] = gamma[i];
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int i = u * kNormThreads + threadIdx.x;
        if (i < n4) {
            if (y) {
                v[u] = make_float4(v[u].x + yv[u].x, v[u].y + yv[u].y, v[u].z + yv[u].z, v[u].w + yv[u].w);
                h[i] = v[u];
            }
            ss = __builtin_fmaf(v[u].x, v[u].x, ss);
            ss = __builtin_fmaf(v[u].y, v[u].y, ss);
            ss = __builtin_fmaf(v[u].z, v[u].z, ss);
            ss = __builtin_fmaf(v[u].w, v[u].w, ss);
        }
    }
    finish_norm4(v, g, ss, n4, eps, x, red);
}

__global__ void __launch_bounds__(kNormThreads) embed_rmsnorm4_kernel(const uint16_t* __restrict__ table, int64_t vocab,
                                                                      const int32_t* __restrict__ token,
                                                                      const uint2* __restrict__ gamma, int32_t n4,
                                                                      float eps, float4* __restrict__ h,
                                                                      uint2* __restrict__ x)
{
    __shared__ float red[kNormThreads / 64];
    int64_t t = *token;
    t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
    const uint2* row = reinterpret_cast<const uint2*>(table + t * (int64_t)(4 * n4));
    float4 v[kNormVec];
    uint2 e[kNormVec], g[kNormVec];
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int i = u * kNormThreads + threadIdx.x;
        if (i < n4) {
            e[u] = row[i];
            g[u] = gamma[i];
        }
    }
    float ss = 0.0f;
#pragma unroll
    for (int u = 0; u < kNormVec; ++u) {
        const int i = u * kNormThreads + threadIdx.x;
        if (i < n4) {
            v[u] = f4_from_halves(e[u]);
            h[i] = v[u];
            ss = __builtin_fmaf(v[u].x, v[u].x, ss);
            ss = __builtin_fmaf(v[u].y, v[u].y, ss);
            ss = __builtin_fmaf(v[u].z, v[u].z, ss);
            ss = __builtin_fmaf(v[u].w, v[u].w, ss);
        }
    }
    finish_norm4(v, g, ss, n4, eps, x, red);
}

bool norm4_ok(int64_t n, const void* h, const void* y, const void* gamma, const void* x)
{
    auto al = [](const void* p, uintptr_t b) { return (reinterpret_cast<uintptr_t>(p) & (b - 1)) == 0; };
    return n % 4 == 0 && n / 4 <= (int64_t)kNormVec * kNormThreads && al(h, 16) && (!y || al(y, 16)) &&
           al(gamma, 8) && al(x, 8);
}

// One workgroup per head of q and k (v heads ride along with k); thread i < 64
// rotates the pair (i, i + 64) by pos * theta^(-2i/128) after the optional
// bias is added.  The angle and its sine and cosine are evaluated in double
// (the angle reaches the context length in radians), the rotation in fp32.
// k and v go to the cache slot of token pos.
__global__ void __launch_bounds__(64) rope_append_kernel(RopeCall a, int page_shift)
{
    const int hd = blockIdx.x;  // 0..n_heads-1: q heads; then n_kv k heads
    const int i = threadIdx.x;
    int pos = *a.pos;
    pos = pos < 0 ? 0 : (pos >= a.max_ctx ? a.max_ctx - 1 : pos);
    const double ang = (double)pos * pow(a.theta, -2.0 * (double)i / 128.0);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const int64_t base = (int64_t)hd * 128;
    float x0 = a.qkv[base + i], x1 = a.qkv[base + i + 64];
    if (a.bias) {
        x0 += a.bias[base + i];
        x1 += a.bias[base + i + 64];
    }
    const float r0 = x0 * c - x1 * s;
    const float r1 = x1 * c + x0 * s;
    if (hd < a.n_heads) {
        a.q_out[base + i] = float_to_half(r0);
        a.q_out[base + i + 64] = float_to_half(r1);
        return;
    }
    const int g = hd - a.n_heads;
    int pg = a.page_table[pos >> page_shift];
    pg = pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
    const int64_t row = ((int64_t)pg * a.n_kv + g) * ((int64_t)1 << page_shift) + (pos & ((1 << page_shift) - 1));
    a.k_cache[row * 128 + i] = float_to_half(r0);
    a.k_cache[row * 128 + i + 64] = float_to_half(r1);
    const int64_t vb = (int64_t)(a.n_heads + a.n_kv + g) * 128;
    float v0 = a.qkv[vb + i], v1 = a.qkv[vb + i + 64];
    if (a.bias) {
        v0 += a.bias[vb + i];
        v1 += a.bias[vb + i + 64];
    }
    a.v_cache[row * 128 + i] = float_to_half(v0);
    a.v_cache[row * 128 + i + 64] = float_to_half(v1);
    if (a.ctx_out && g == 0 && i == 0) *a.ctx_out = pos + 1;
}

__global__ void __launch_bounds__(256) rope_table_kernel(double theta, int32_t max_ctx, float2* table)
{
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= (int64_t)max_ctx * 64) return;
    const int pos = (int)(k / 64), i = (int)(k % 64);
    const double ang = (double)pos * pow(theta, -2.0 * (double)i / 128.0);
    double sn, cs;
    sincos(ang, &sn, &cs);
    table[k] = make_float2((float)cs, (float)sn);
}

}  // namespace

hipError_t launch_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token, float* h,
                        hipStream_t stream)
{
    const int64_t blocks = (hidden + 255) / 256 < 64 ? (hidden + 255) / 256 : 64;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, vocab, hidden, token, h);
    return hipGetLastError();
}

hipError_t launch_embed_rmsnorm(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token,
                                const uint16_t* gamma, float eps, float* h, uint16_t* x, hipStream_t stream)
{
    if (norm4_ok(hidden, h, nullptr, gamma, x) && (reinterpret_cast<uintptr_t>(table) & 7u) == 0) {
        hipLaunchKernelGGL(embed_rmsnorm4_kernel, dim3(1), dim3(kNormThreads), 0, stream, table, vocab, token,
                           reinterpret_cast<const uint2*>(gamma), (int32_t)(hidden / 4), eps,
                           reinterpret_cast<float4*>(h), reinterpret_cast<uint2*>(x));
        return hipGetLastError();
    }
    hipLaunchKernelGGL(embed_rmsnorm_kernel, dim3(1), dim3(kNormThreads), 0, stream, table, vocab, hidden, token, gamma,
                       eps, h, x);
    return hipGetLastError();
}

hipError_t launch_add_rmsnorm(float* h, const float* y, const uint16_t* gamma, int64_t n, float eps, uint16_t* x,
                              hipStream_t stream)
{
    if (norm4_ok(n, h, y, gamma, x)) {
        hipLaunchKernelGGL(add_rmsnorm4_kernel, dim3(1), dim3(kNormThreads), 0, stream, reinterpret_cast<float4*>(h),
                           reinterpret_cast<const float4*>(y), reinterpret_cast<const uint2*>(gamma), (int32_t)(n / 4),
                           eps, reinterpret_cast<uint2*>(x));
        return hipGetLastError();
    }
    hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(1), dim3(kNormThreads), 0, stream, h, y, gamma, n, eps, x);
    return hipGetLastError();
}

hipError_t launch_rope_append(const RopeCall& c, hipStream_t stream)
{
    int shift = 0;
    while ((1 << shift) < c.page_size) ++shift;
    hipLaunchKernelGGL(rope_append_kernel, dim3((unsigned)(c.n_heads + c.n_kv)), dim3(64), 0, stream, c, shift);
    return hipGetLastError();
}

hipError_t launch_rope_table(double theta, int32_t max_ctx, float2* table, hipStream_t stream)
{
    const int64_t n = (int64_t)max_ctx * 64;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, theta, max_ctx, table);
    return hipGetLastError();
}

}  // namespace w4i
