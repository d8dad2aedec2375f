// Glue kernels of a full decode step around the INT4 projections and the
// paged attention: embedding lookup, residual add + RMSNorm, rotary embedding
// with the KV-cache append, and the position advance.  The pages' runtime is
// a Qwen2.5-Coder-7B decoding stack ("How To Build Your Own LLM Runtime From
// Scratch", aitrending.vip, TL;DR and "Technical Details"); its glue is read
// as the Qwen2-family pre-norm decoder:
//
//   h = E[token];  per layer:  x = rmsnorm(h) g1;  q,k,v = x Wqkv;  rope(q, k);
//   append k, v;  h += o_proj(attn(q));  x = rmsnorm(h) g2;  h += down(silu(gate) up)
//   then x = rmsnorm(h) g_f and the next token is argmax(x Wlm).
//
// The token id, the position and the attention's context length live in
// device memory and are advanced by these kernels, so one captured graph of
// the whole step replays token after token with no host work in between.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"

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
// fixed order (per-thread strided sums, then a tree), so it is deterministic.
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
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += red[w];
    const float r = 1.0f / sqrtf(tot / (float)n + eps);
    for (int64_t i = tid; i < n; i += kNormThreads) x[i] = float_to_half(h[i] * r * half_to_float(gamma[i]));
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

__global__ void __launch_bounds__(64) advance_kernel(int32_t* pos)
{
    if (threadIdx.x == 0) *pos = *pos + 1;
}

}  // namespace

hipError_t launch_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token, float* h,
                        hipStream_t stream)
{
    const int64_t blocks = (hidden + 255) / 256 < 64 ? (hidden + 255) / 256 : 64;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, table, vocab, hidden, token, h);
    return hipGetLastError();
}

hipError_t launch_add_rmsnorm(float* h, const float* y, const uint16_t* gamma, int64_t n, float eps, uint16_t* x,
                              hipStream_t stream)
{
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

hipError_t launch_advance(int32_t* pos, hipStream_t stream)
{
    hipLaunchKernelGGL(advance_kernel, dim3(1), dim3(64), 0, stream, pos);
    return hipGetLastError();
}

}  // namespace w4i
