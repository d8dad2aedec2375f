// extern "C" entry points of the INT4 weight-only GEMV library: argument
// validation, error reporting, the host packer entry, single-GEMV launches
// and the per-token sweep (eager launches or one captured HIP graph).
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>
#include <vector>

#include "w4.h"
#include "w4_abi_util.h"
#include "w4_internal.h"

namespace w4i {
int64_t pack_w4t4(const uint8_t* q, const uint16_t* s, int64_t n, int64_t k, int32_t group,
                  bool gateup, uint8_t* pw, uint8_t* ps);
}

using namespace w4i;

namespace w4i {

namespace {
thread_local std::string g_last_error;
}

w4_status fail(w4_status code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

w4_status hip_fail(hipError_t err, const char* what)
{
    return fail(W4_EHIP, "%s failed: %s (%d)", what, hipGetErrorString(err), (int)err);
}

const char* last_error()
{
    return g_last_error.c_str();
}

}  // namespace w4i

namespace {

w4_status ok()
{
    return W4_OK;
}

w4_status check_shape(int64_t n, int64_t k, int32_t group, bool gateup, const char* who)
{
    if (n < 1) return fail(W4_ESHAPE, "%s: n=%lld must be >= 1", who, (long long)n);
    if (k < 8) return fail(W4_ESHAPE, "%s: k=%lld must be >= 8", who, (long long)k);
    if (k > kMaxK) return fail(W4_ESHAPE, "%s: k=%lld exceeds %lld", who, (long long)k, (long long)kMaxK);
    if (group < 8 || (group & (group - 1)) != 0)
        return fail(W4_ESHAPE, "%s: group=%d must be a power of two >= 8", who, group);
    if (group > k || k % group != 0)
        return fail(W4_ESHAPE, "%s: k=%lld must be a multiple of group=%d", who, (long long)k, group);
    if (gateup && n % 2 != 0)
        return fail(W4_ESHAPE, "%s: gate/up n_total=%lld must be even", who, (long long)n);
    if (tiles_for(n, gateup) > ((int64_t)1 << 40))
        return fail(W4_ESHAPE, "%s: n=%lld too large", who, (long long)n);
    return W4_OK;
}

void sizes(int64_t n, int64_t k, int32_t group, bool gateup, size_t* wb, size_t* sb)
{
    const int64_t tiles = tiles_for(n, gateup);
    *wb = (size_t)(tiles * (k / 8) * 16);
    *sb = (size_t)(tiles * (k / group) * 8);
}

w4_status validate_gemv(const GemvCall& c, const char* who)
{
    const bool gateup = c.epi == kEpiGateUp;
    w4_status st = check_shape(c.n, c.k, c.group, gateup, who);
    if (st != W4_OK) return st;
    const void* in = c.norm_h ? static_cast<const void*>(c.norm_h) : c.x;
    if (!c.pw || !c.ps || !in || !c.out)
        return fail(W4_EINVAL, "%s: null pointer (packed_w=%p packed_s=%p x=%p out=%p)", who, c.pw,
                    c.ps, in, c.out);
    if (!aligned16(c.pw) || !aligned16(c.ps) || !aligned16(in))
        return fail(W4_EALIGN, "%s: packed_w, packed_s and x (or h) must be 16-byte aligned", who);
    if (c.norm_h) {
        if (c.xs) return fail(W4_EINVAL, "%s: the RMSNorm prologue takes fp16 activations only", who);
        if (!c.norm_gamma || !c.norm_ss) return fail(W4_EINVAL, "%s: null gamma or ss_part", who);
        if (!aligned16(c.norm_gamma) || !aligned16(c.norm_ss) || (c.x_out && !aligned16(c.x_out)))
            return fail(W4_EALIGN, "%s: gamma, ss_part and x_out must be 16-byte aligned", who);
        if (c.norm_parts < 1 || c.norm_parts > kMaxNormParts)
            return fail(W4_ESHAPE, "%s: parts=%lld must be in [1, %lld]", who, (long long)c.norm_parts,
                        (long long)kMaxNormParts);
        if (!(c.norm_eps >= 0.0f) || !isfinite(c.norm_eps))
            return fail(W4_EINVAL, "%s: eps=%g must be finite and >= 0", who, c.norm_eps);
    }
    if (c.h_out) {
        if (c.epi != kEpiPlain) return fail(W4_EINVAL, "%s: the residual epilogue is for plain GEMVs", who);
        if (!c.h_in || !c.ss_out) return fail(W4_EINVAL, "%s: null h_in or ss_part", who);
        if (!aligned_to(c.h_in, 4) || !aligned_to(c.h_out, 4) || !aligned16(c.ss_out) || !aligned_to(c.out, 4))
            return fail(W4_EALIGN, "%s: h_in, h_out and y must be 4-byte, ss_part 16-byte aligned", who);
    }
    if (c.epi == kEpiArgmax) {
        if (!c.argmax || !c.ws)
            return fail(W4_EINVAL, "%s: argmax needs argmax and workspace pointers", who);
        if (!aligned16(c.ws)) return fail(W4_EALIGN, "%s: workspace must be 16-byte aligned", who);
        if (c.n > INT32_MAX - 1)
            return fail(W4_ESHAPE, "%s: argmax needs n < 2^31-1 (int32 index)", who);
    }
    return W4_OK;
}

w4_status validate_gemm(const GemmCall& c, const char* who)
{
    const bool gateup = c.epi == kEpiGateUp;
    w4_status st = check_shape(c.n, c.k, c.group, gateup, who);
    if (st != W4_OK) return st;
    if (c.m < 1 || c.m > ((int64_t)1 << 20))
        return fail(W4_ESHAPE, "%s: m=%lld must be in [1, 2^20]", who, (long long)c.m);
    if (!c.pw || !c.ps || !c.x || !c.out)
        return fail(W4_EINVAL, "%s: null pointer (packed_w=%p packed_s=%p x=%p out=%p)", who, c.pw,
                    c.ps, c.x, c.out);
    if (!aligned16(c.pw) || !aligned16(c.ps) || !aligned16(c.x))
        return fail(W4_EALIGN, "%s: packed_w, packed_s and x must be 16-byte aligned", who);
    if ((reinterpret_cast<uintptr_t>(c.out) & (gateup ? 1u : 3u)) != 0)
        return fail(W4_EALIGN, "%s: output must be aligned to its element size", who);
    return W4_OK;
}

w4_status check_gemm_workspace(const GemmCall& c, size_t ws_bytes, const char* who)
{
    const size_t need = gemm_workspace_bytes(c.epi, c.m, c.n, c.k);
    if (need == 0) return W4_OK;
    if (!c.ws) return fail(W4_EINVAL, "%s: this shape needs a workspace of %zu bytes", who, need);
    if (ws_bytes < need) return fail(W4_EINVAL, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, need);
    if (!aligned16(c.ws)) return fail(W4_EALIGN, "%s: workspace must be 16-byte aligned", who);
    return W4_OK;
}

}  // namespace

namespace w4i {

w4_status check_gemv(const GemvCall& c, const char* who)
{
    return validate_gemv(c, who);
}

}  // namespace w4i

extern "C" {

const char* w4_status_string(w4_status status)
{
    switch (status) {
        case W4_OK: return "W4_OK";
        case W4_EINVAL: return "W4_EINVAL";
        case W4_ESHAPE: return "W4_ESHAPE";
        case W4_EALIGN: return "W4_EALIGN";
        case W4_EHIP: return "W4_EHIP";
        case W4_ENOMEM: return "W4_ENOMEM";
        case W4_ECAPTURE: return "W4_ECAPTURE";
        default: return "W4_UNKNOWN";
    }
}

const char* w4_last_error(void)
{
    return last_error();
}

int32_t w4_abi_version(void)
{
    return 1;
}

w4_status w4_packed_size(int64_t n, int64_t k, int32_t group, int32_t layout, size_t* weight_bytes,
                         size_t* scale_bytes)
{
    try {
        if (!weight_bytes || !scale_bytes) return fail(W4_EINVAL, "w4_packed_size: null output");
        if (layout != W4_LAYOUT_PLAIN && layout != W4_LAYOUT_GATEUP)
            return fail(W4_EINVAL, "w4_packed_size: unknown layout %d", layout);
        const bool gateup = layout == W4_LAYOUT_GATEUP;
        w4_status st = check_shape(n, k, group, gateup, "w4_packed_size");
        if (st != W4_OK) return st;
        sizes(n, k, group, gateup, weight_bytes, scale_bytes);
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_packed_size: internal exception");
    }
}

w4_status w4_pack(const uint8_t* q, const uint16_t* scales, int64_t n, int64_t k, int32_t group,
                  int32_t layout, void* packed_w, size_t packed_w_bytes, void* packed_s,
                  size_t packed_s_bytes)
{
    try {
        if (!q || !scales || !packed_w || !packed_s) return fail(W4_EINVAL, "w4_pack: null pointer");
        if (layout != W4_LAYOUT_PLAIN && layout != W4_LAYOUT_GATEUP)
            return fail(W4_EINVAL, "w4_pack: unknown layout %d", layout);
        const bool gateup = layout == W4_LAYOUT_GATEUP;
        w4_status st = check_shape(n, k, group, gateup, "w4_pack");
        if (st != W4_OK) return st;
        size_t wb, sb;
        sizes(n, k, group, gateup, &wb, &sb);
        if (packed_w_bytes != wb || packed_s_bytes != sb)
            return fail(W4_EINVAL, "w4_pack: buffer sizes %zu/%zu, expected %zu/%zu", packed_w_bytes,
                        packed_s_bytes, wb, sb);
        const int64_t bad = pack_w4t4(q, scales, n, k, group, gateup, static_cast<uint8_t*>(packed_w),
                                      static_cast<uint8_t*>(packed_s));
        if (bad >= 0)
            return fail(W4_EINVAL, "w4_pack: q[%lld][%lld] = %u is not a 4-bit value",
                        (long long)(bad / k), (long long)(bad % k), (unsigned)q[bad]);
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(W4_ENOMEM, "w4_pack: out of host memory");
    } catch (...) {
        return fail(W4_EINVAL, "w4_pack: internal exception");
    }
}

w4_status w4_gemv_workspace_size(int64_t n, int64_t k, int32_t group, int32_t with_argmax,
                                 size_t* bytes)
{
    try {
        if (!bytes) return fail(W4_EINVAL, "w4_gemv_workspace_size: null output");
        w4_status st = check_shape(n, k, group, false, "w4_gemv_workspace_size");
        if (st != W4_OK) return st;
        GemvCall c{};
        c.n = n;
        c.k = k;
        c.group = group;
        c.epi = kEpiArgmax;
        *bytes = with_argmax ? argmax_workspace_bytes(launch_grid(c)) : 0;
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_workspace_size: internal exception");
    }
}

w4_status w4_gemv(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                  int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                  int32_t group, void* stream)
{
    try {
        GemvCall c{packed_w, packed_s, x, y, argmax, workspace, n, k, group,
                   argmax ? kEpiArgmax : kEpiPlain};
        w4_status st = validate_gemv(c, "w4_gemv");
        if (st != W4_OK) return st;
        if (argmax && workspace_bytes < argmax_workspace_bytes(launch_grid(c)))
            return fail(W4_EINVAL, "w4_gemv: workspace of %zu bytes, need %zu", workspace_bytes,
                        argmax_workspace_bytes(launch_grid(c)));
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv: internal exception");
    }
}

w4_status w4_gemv_argmax_noalloc(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                                 int32_t* argmax, int64_t n, int64_t k, int32_t group, void* stream)
{
    try {
        const char* who = "w4_gemv_argmax_noalloc";
        if (!argmax) return fail(W4_EINVAL, "%s: null argmax", who);
        // validated with a placeholder workspace address; the real one is the
        // library's static scratch, looked up below
        GemvCall c{packed_w, packed_s, x, y, argmax, reinterpret_cast<void*>(uintptr_t{256}), n, k, group,
                   kEpiArgmax};
        w4_status st = validate_gemv(c, who);
        if (st != W4_OK) return st;
        const size_t need = argmax_workspace_bytes(launch_grid(c));
        if (need > kNoAllocScratchBytes)
            return fail(W4_ESHAPE, "%s: n=%lld k=%lld needs %zu bytes of scratch, the static scratch holds %zu", who,
                        (long long)n, (long long)k, need, kNoAllocScratchBytes);
        void* ws = nullptr;
        hipError_t err = noalloc_scratch(&ws);
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_argmax_noalloc scratch lookup");
        c.ws = ws;
        err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_argmax_noalloc launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_argmax_noalloc: internal exception");
    }
}

w4_status w4_gemv_gateup_silu(const void* packed_w, const void* packed_s, const uint16_t* x,
                              uint16_t* h, int64_t n_total, int64_t k, int32_t group, void* stream)
{
    try {
        GemvCall c{packed_w, packed_s, x, h, nullptr, nullptr, n_total, k, group, kEpiGateUp};
        w4_status st = validate_gemv(c, "w4_gemv_gateup_silu");
        if (st != W4_OK) return st;
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_gateup_silu launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_gateup_silu: internal exception");
    }
}

w4_status w4_residual_parts(int64_t n, int64_t k, int32_t group, int64_t* parts)
{
    try {
        if (!parts) return fail(W4_EINVAL, "w4_residual_parts: null output");
        w4_status st = check_shape(n, k, group, false, "w4_residual_parts");
        if (st != W4_OK) return st;
        *parts = residual_parts(n, k, group);
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_residual_parts: internal exception");
    }
}

w4_status w4_gemv_residual(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                           const float* h_in, float* h_out, float* ss_part, int64_t n, int64_t k, int32_t group,
                           void* stream)
{
    try {
        const char* who = "w4_gemv_residual";
        if (!h_out) return fail(W4_EINVAL, "%s: null h_out", who);
        GemvCall c{packed_w, packed_s, x, y, nullptr, nullptr, n, k, group, kEpiPlain};
        c.h_in = h_in;
        c.h_out = h_out;
        c.ss_out = ss_part;
        w4_status st = validate_gemv(c, who);
        if (st != W4_OK) return st;
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_residual launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_residual: internal exception");
    }
}

w4_status w4_gemv_rmsnorm(const void* packed_w, const void* packed_s, const float* h, const uint16_t* gamma,
                          const float* ss_part, int64_t parts, float eps, uint16_t* x_out, float* y,
                          int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                          int32_t group, void* stream)
{
    try {
        const char* who = "w4_gemv_rmsnorm";
        if (!h) return fail(W4_EINVAL, "%s: null h", who);
        GemvCall c{packed_w, packed_s, nullptr, y, argmax, workspace, n, k, group, argmax ? kEpiArgmax : kEpiPlain};
        c.norm_h = h;
        c.norm_gamma = gamma;
        c.norm_ss = ss_part;
        c.norm_parts = parts;
        c.norm_eps = eps;
        c.x_out = x_out;
        w4_status st = validate_gemv(c, who);
        if (st != W4_OK) return st;
        if (argmax && workspace_bytes < argmax_workspace_bytes(launch_grid(c)))
            return fail(W4_EINVAL, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes,
                        argmax_workspace_bytes(launch_grid(c)));
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_rmsnorm launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_rmsnorm: internal exception");
    }
}

w4_status w4_gemv_gateup_silu_rmsnorm(const void* packed_w, const void* packed_s, const float* h,
                                      const uint16_t* gamma, const float* ss_part, int64_t parts, float eps,
                                      uint16_t* x_out, uint16_t* h_mlp, int64_t n_total, int64_t k, int32_t group,
                                      void* stream)
{
    try {
        const char* who = "w4_gemv_gateup_silu_rmsnorm";
        if (!h) return fail(W4_EINVAL, "%s: null h", who);
        GemvCall c{packed_w, packed_s, nullptr, h_mlp, nullptr, nullptr, n_total, k, group, kEpiGateUp};
        c.norm_h = h;
        c.norm_gamma = gamma;
        c.norm_ss = ss_part;
        c.norm_parts = parts;
        c.norm_eps = eps;
        c.x_out = x_out;
        w4_status st = validate_gemv(c, who);
        if (st != W4_OK) return st;
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_gateup_silu_rmsnorm launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_gateup_silu_rmsnorm: internal exception");
    }
}

w4_status w4_quantize_act8(const uint16_t* x, int64_t k, int32_t group, int8_t* codes, float* scales, void* stream)
{
    try {
        const char* who = "w4_quantize_act8";
        if (!x || !codes || !scales) return fail(W4_EINVAL, "%s: null pointer", who);
        w4_status st = check_shape(1, k, group, false, who);
        if (st != W4_OK) return st;
        if (!aligned16(x) || !aligned_to(codes, 8) || !aligned_to(scales, 4))
            return fail(W4_EALIGN, "%s: x must be 16-byte, codes 8-byte, scales 4-byte aligned", who);
        hipError_t err = launch_act8_quantize(x, k, group, codes, scales, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_quantize_act8 launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_quantize_act8: internal exception");
    }
}

w4_status w4_gemv_a8(const void* packed_w, const void* packed_s, const int8_t* codes, const float* act_scales,
                     float* y, int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                     int32_t group, void* stream)
{
    try {
        GemvCall c{packed_w, packed_s, codes, y, argmax, workspace, n, k, group, argmax ? kEpiArgmax : kEpiPlain,
                   act_scales};
        w4_status st = validate_gemv(c, "w4_gemv_a8");
        if (st != W4_OK) return st;
        if (!act_scales) return fail(W4_EINVAL, "w4_gemv_a8: null act_scales");
        if (!aligned_to(act_scales, 4)) return fail(W4_EALIGN, "w4_gemv_a8: act_scales must be 4-byte aligned");
        if (argmax && workspace_bytes < argmax_workspace_bytes(launch_grid(c)))
            return fail(W4_EINVAL, "w4_gemv_a8: workspace of %zu bytes, need %zu", workspace_bytes,
                        argmax_workspace_bytes(launch_grid(c)));
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_a8 launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_a8: internal exception");
    }
}

w4_status w4_gemv_gateup_silu_a8(const void* packed_w, const void* packed_s, const int8_t* codes,
                                 const float* act_scales, uint16_t* h, int64_t n_total, int64_t k, int32_t group,
                                 void* stream)
{
    try {
        GemvCall c{packed_w, packed_s, codes, h, nullptr, nullptr, n_total, k, group, kEpiGateUp, act_scales};
        w4_status st = validate_gemv(c, "w4_gemv_gateup_silu_a8");
        if (st != W4_OK) return st;
        if (!act_scales) return fail(W4_EINVAL, "w4_gemv_gateup_silu_a8: null act_scales");
        if (!aligned_to(act_scales, 4))
            return fail(W4_EALIGN, "w4_gemv_gateup_silu_a8: act_scales must be 4-byte aligned");
        hipError_t err = launch_gemv(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemv_gateup_silu_a8 launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemv_gateup_silu_a8: internal exception");
    }
}

w4_status w4_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream)
{
    try {
        const char* who = "w4_read_probe";
        if (!buf || !sink) return fail(W4_EINVAL, "%s: null pointer", who);
        if (bytes == 0 || bytes % 16 != 0 || bytes / 16 > ((size_t)1 << 40))
            return fail(W4_ESHAPE, "%s: bytes=%zu must be a positive multiple of 16", who, bytes);
        if (!aligned16(buf) || !aligned_to(sink, 4)) return fail(W4_EALIGN, "%s: buf must be 16-byte aligned", who);
        hipError_t err = launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_read_probe launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_read_probe: internal exception");
    }
}

w4_status w4_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t group, size_t* bytes)
{
    try {
        if (!bytes) return fail(W4_EINVAL, "w4_gemm_workspace_size: null output");
        w4_status st = check_shape(n, k, group, false, "w4_gemm_workspace_size");
        if (st != W4_OK) return st;
        if (m < 1 || m > ((int64_t)1 << 20))
            return fail(W4_ESHAPE, "w4_gemm_workspace_size: m=%lld must be in [1, 2^20]", (long long)m);
        *bytes = gemm_workspace_bytes(kEpiPlain, m, n, k);
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemm_workspace_size: internal exception");
    }
}

w4_status w4_gemm(const void* packed_w, const void* packed_s, const uint16_t* x, float* y, void* workspace,
                  size_t workspace_bytes, int64_t m, int64_t n, int64_t k, int32_t group, void* stream)
{
    try {
        GemmCall c{packed_w, packed_s, x, y, workspace, m, n, k, group, kEpiPlain};
        w4_status st = validate_gemm(c, "w4_gemm");
        if (st != W4_OK) return st;
        st = check_gemm_workspace(c, workspace_bytes, "w4_gemm");
        if (st != W4_OK) return st;
        hipError_t err = launch_gemm(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemm launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemm: internal exception");
    }
}

w4_status w4_gemm_gateup_silu(const void* packed_w, const void* packed_s, const uint16_t* x,
                              uint16_t* h, int64_t m, int64_t n_total, int64_t k, int32_t group,
                              void* stream)
{
    try {
        GemmCall c{packed_w, packed_s, x, h, nullptr, m, n_total, k, group, kEpiGateUp};
        w4_status st = validate_gemm(c, "w4_gemm_gateup_silu");
        if (st != W4_OK) return st;
        hipError_t err = launch_gemm(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_gemm_gateup_silu launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_gemm_gateup_silu: internal exception");
    }
}

w4_status w4_attn_decode_workspace_size(int32_t n_heads, int32_t max_ctx, size_t* bytes)
{
    try {
        if (!bytes) return fail(W4_EINVAL, "w4_attn_decode_workspace_size: null output");
        if (n_heads < 1 || max_ctx < 1 || max_ctx > kAttnMaxCtx)
            return fail(W4_ESHAPE, "w4_attn_decode_workspace_size: n_heads=%d max_ctx=%d", n_heads, max_ctx);
        *bytes = attn_workspace_bytes(n_heads, max_ctx);
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_attn_decode_workspace_size: internal exception");
    }
}

w4_status w4_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* page_table, int32_t num_pages, const int32_t* ctx_len, int32_t max_ctx,
                         uint16_t* out, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size,
                         float scale, void* workspace, size_t workspace_bytes, void* stream)
{
    try {
        const char* who = "w4_attn_decode";
        if (!q || !k_cache || !v_cache || !page_table || !ctx_len || !out || !workspace)
            return fail(W4_EINVAL, "%s: null pointer", who);
        w4_status st = check_kv_shape(n_heads, n_kv_heads, head_dim, page_size, max_ctx, num_pages, who);
        if (st != W4_OK) return st;
        if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) ||
            (reinterpret_cast<uintptr_t>(out) & 1u) || (reinterpret_cast<uintptr_t>(page_table) & 3u) ||
            (reinterpret_cast<uintptr_t>(ctx_len) & 3u))
            return fail(W4_EALIGN, "%s: q, caches and workspace must be 16-byte aligned", who);
        const size_t need = attn_workspace_bytes(n_heads, max_ctx);
        if (workspace_bytes < need)
            return fail(W4_EINVAL, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
        AttnCall c{q, k_cache, v_cache, page_table, ctx_len, out, workspace, scale, max_ctx, n_heads, n_kv_heads,
                   page_size, num_pages};
        hipError_t err = launch_attn(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_attn_decode launch");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_attn_decode: internal exception");
    }
}

}  // extern "C"

struct w4_sweep {
    std::vector<GemvCall> calls;
    int32_t mode = 0;             // W4_SWEEP_EAGER / _GRAPH / _PERSISTENT / _PERSISTENT_EAGER
    bool use_graph = false;       // the launches are replayed from `exec`
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    // persistent modes
    void* dev = nullptr;          // phase table + control block + tagged input words
    PersistArgs pargs{};
    struct Final {
        const float* part_v;
        const int32_t* part_i;
        int32_t* out;
    };
    std::vector<Final> finals;    // argmax finalize per lm_head projection
};

namespace {

w4_status desc_to_call(const w4_proj_desc& d, int32_t idx, GemvCall* out)
{
    int32_t epi;
    switch (d.kind) {
        case W4_PROJ_PLAIN: epi = kEpiPlain; break;
        case W4_PROJ_GATEUP_SILU: epi = kEpiGateUp; break;
        case W4_PROJ_LMHEAD_ARGMAX: epi = kEpiArgmax; break;
        default: return fail(W4_EINVAL, "sweep projection %d: unknown kind %d", idx, d.kind);
    }
    *out = GemvCall{d.packed_w, d.packed_s, d.x, d.out, d.argmax, d.workspace, d.n, d.k, d.group, epi};
    char who[64];
    snprintf(who, sizeof who, "sweep projection %d", idx);
    w4_status st = validate_gemv(*out, who);
    if (st != W4_OK) return st;
    if (epi == kEpiArgmax && d.workspace_bytes < argmax_workspace_bytes(launch_grid(*out)))
        return fail(W4_EINVAL, "%s: workspace of %zu bytes, need %zu", who, d.workspace_bytes,
                    argmax_workspace_bytes(launch_grid(*out)));
    return W4_OK;
}

w4_status launch_persistent(const w4_sweep& sw, hipStream_t stream)
{
    hipError_t err = launch_persist(sw.pargs, stream);
    if (err != hipSuccess) return hip_fail(err, "persistent sweep launch");
    for (const auto& f : sw.finals) {
        err = launch_argmax_finalize(f.part_v, f.part_i, sw.pargs.nwg, f.out, stream);
        if (err != hipSuccess) return hip_fail(err, "persistent sweep argmax finalize");
    }
    return W4_OK;
}

// Build the persistent sweep's device state: the phase table (same unit and
// split shape per projection as the launch table of the one-kernel path), the
// control block and the tagged input words.  Fails with W4_ESHAPE for sweeps
// the persistent kernel does not cover.
w4_status persist_setup(w4_sweep* sw, const w4_proj_desc* projs)
{
    const char* who = "w4_decode_linear_sweep_create (persistent)";
    const int32_t count = (int32_t)sw->calls.size();
    if (count > kPMaxPhases) return fail(W4_ESHAPE, "%s: %d projections, at most %d", who, count, kPMaxPhases);
    for (int32_t i = 0; i < count; ++i) {
        const GemvCall& c = sw->calls[(size_t)i];
        if (c.k % 512 != 0 || c.k / 8 > kPMaxKb)
            return fail(W4_ESHAPE, "%s: projection %d: k=%lld must be a multiple of 512 and at most %d", who, i,
                        (long long)c.k, kPMaxKb * 8);
        if (c.group < 64 || c.group > 512)
            return fail(W4_ESHAPE, "%s: projection %d: group=%d must be in [64, 512]", who, i, c.group);
    }
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
    int cus = 0, coop = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (err != hipSuccess) return hip_fail(err, "hipDeviceGetAttribute");
    if (!coop) return fail(W4_EINVAL, "%s: the device does not support cooperative launches", who);
    int per_cu = 0;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, persist_kernel_fn(), persist_threads(), 0);
    if (err != hipSuccess) return hip_fail(err, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (per_cu < 1 || cus < 8) return fail(W4_EINVAL, "%s: the kernel does not fit on a CU (%d per CU, %d CUs)", who,
                                           per_cu, cus);
    const int32_t nwg = cus;
    std::vector<PersistPhase> ph((size_t)count);
    int32_t max_words = 1;
    for (int32_t i = 0; i < count; ++i) {
        const GemvCall& c = sw->calls[(size_t)i];
        const int32_t words = (int32_t)(c.k / 2);
        if ((words + nwg - 1) / nwg > kPStageWords)
            return fail(W4_ESHAPE, "%s: projection %d: k=%lld too long for %d workgroups", who, i, (long long)c.k,
                        nwg);
        if (words > max_words) max_words = words;
        const bool gateup = c.epi == kEpiGateUp;
        PersistPhase& P = ph[(size_t)i];
        P.pw = static_cast<const uint4*>(c.pw);
        P.ps = static_cast<const uint2*>(c.ps);
        P.x = static_cast<const uint16_t*>(c.x);
        P.out = c.out;
        P.n = c.n;
        P.tiles = tiles_for(c.n, gateup);
        P.tiles_half = gateup ? P.tiles / 2 : 0;
        P.kb = (int32_t)(c.k / 8);
        P.iters = (int32_t)(c.k / 512);
        P.ng = (int32_t)(c.k / c.group);
        int32_t gshift = 0;
        while ((8 << gshift) < c.group) ++gshift;
        P.gshift = gshift;
        P.epi = c.epi;
        const LaunchConfig cfg = choose_config(c.epi, gateup ? P.tiles / 2 : P.tiles, P.iters);
        P.utiles = gateup ? 2 : cfg.tiles;
        P.split = cfg.split;
        const int64_t units = gateup ? P.tiles / 2 : (P.tiles + cfg.tiles - 1) / cfg.tiles;
        if (units > INT32_MAX) return fail(W4_ESHAPE, "%s: projection %d too tall", who, i);
        P.units = (int32_t)units;
        P.sc_dwords = 2 * (512 / c.group);
        if (c.epi == kEpiArgmax) {
            const w4_proj_desc& d = projs[i];
            if (d.workspace_bytes < argmax_workspace_bytes(nwg))
                return fail(W4_EINVAL, "%s: projection %d: workspace of %zu bytes, need %zu", who, i,
                            d.workspace_bytes, argmax_workspace_bytes(nwg));
            uint8_t* ws = static_cast<uint8_t*>(c.ws);
            P.part_v = reinterpret_cast<float*>(ws);
            P.part_i = reinterpret_cast<int32_t*>(ws + argmax_index_offset(nwg));
            sw->finals.push_back({P.part_v, P.part_i, c.argmax});
        }
    }
    const size_t ph_bytes = ((sizeof(PersistPhase) * (size_t)count) + 255) & ~(size_t)255;
    const size_t hand_bytes = 2 * (size_t)max_words * 8;
    err = hipMalloc(&sw->dev, ph_bytes + kPersistCtrlBytes + hand_bytes);
    if (err != hipSuccess) return hip_fail(err, "hipMalloc (persistent sweep state)");
    uint8_t* base = static_cast<uint8_t*>(sw->dev);
    err = hipMemset(base + ph_bytes, 0, kPersistCtrlBytes + hand_bytes);
    if (err == hipSuccess) err = hipMemcpy(base, ph.data(), sizeof(PersistPhase) * (size_t)count, hipMemcpyHostToDevice);
    const unsigned long long ticks = kPersistTicksPerSecond / 5;   // 200 ms watchdog
    if (err == hipSuccess)
        err = hipMemcpy(base + ph_bytes + kPersistCtrlWatchdogOffset, &ticks, sizeof ticks, hipMemcpyHostToDevice);
    if (err != hipSuccess) return hip_fail(err, "persistent sweep state upload");
    sw->pargs.ph = reinterpret_cast<const PersistPhase*>(base);
    sw->pargs.nph = count;
    sw->pargs.nwg = nwg;
    sw->pargs.ctrl = reinterpret_cast<unsigned*>(base + ph_bytes);
    sw->pargs.hand = reinterpret_cast<unsigned long long*>(base + ph_bytes + kPersistCtrlBytes);
    sw->pargs.hand_words = max_words;
    return W4_OK;
}

w4_status launch_all(const std::vector<GemvCall>& calls, hipStream_t stream)
{
    for (size_t i = 0; i < calls.size(); ++i) {
        hipError_t err = launch_gemv(calls[i], stream);
        if (err != hipSuccess) {
            char what[64];
            snprintf(what, sizeof what, "sweep launch %zu", i);
            return hip_fail(err, what);
        }
    }
    return W4_OK;
}

}  // namespace

extern "C" {

w4_status w4_decode_linear_sweep_create(const w4_proj_desc* projs, int32_t count, int32_t mode,
                                        w4_sweep** out)
{
    try {
        if (!out) return fail(W4_EINVAL, "w4_decode_linear_sweep_create: null output");
        *out = nullptr;
        if (!projs || count < 1)
            return fail(W4_EINVAL, "w4_decode_linear_sweep_create: need at least one projection");
        if (mode < W4_SWEEP_EAGER || mode > W4_SWEEP_PERSISTENT_EAGER)
            return fail(W4_EINVAL, "w4_decode_linear_sweep_create: unknown mode %d", mode);
        w4_sweep* sw = new w4_sweep();
        sw->mode = mode;
        sw->use_graph = mode == W4_SWEEP_GRAPH || mode == W4_SWEEP_PERSISTENT;
        sw->calls.resize((size_t)count);
        for (int32_t i = 0; i < count; ++i) {
            w4_status st = desc_to_call(projs[i], i, &sw->calls[(size_t)i]);
            if (st != W4_OK) {
                delete sw;
                return st;
            }
        }
        const bool persistent = mode == W4_SWEEP_PERSISTENT || mode == W4_SWEEP_PERSISTENT_EAGER;
        if (persistent) {
            w4_status st = persist_setup(sw, projs);
            if (st != W4_OK) {
                if (sw->dev) (void)hipFree(sw->dev);
                delete sw;
                return st;
            }
        }
        if (sw->use_graph) {
            hipStream_t cap = nullptr;
            hipError_t err = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
            if (err != hipSuccess) {
                if (sw->dev) (void)hipFree(sw->dev);
                delete sw;
                return hip_fail(err, "hipStreamCreateWithFlags");
            }
            err = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
            if (err != hipSuccess) {
                (void)hipStreamDestroy(cap);
                if (sw->dev) (void)hipFree(sw->dev);
                delete sw;
                return fail(W4_ECAPTURE, "hipStreamBeginCapture failed: %s", hipGetErrorString(err));
            }
            w4_status st = persistent ? launch_persistent(*sw, cap) : launch_all(sw->calls, cap);
            hipGraph_t graph = nullptr;
            hipError_t end_err = hipStreamEndCapture(cap, &graph);
            (void)hipStreamDestroy(cap);
            if (st != W4_OK || end_err != hipSuccess) {
                if (graph) (void)hipGraphDestroy(graph);
                if (sw->dev) (void)hipFree(sw->dev);
                delete sw;
                if (st != W4_OK) return st;
                return fail(W4_ECAPTURE, "hipStreamEndCapture failed: %s", hipGetErrorString(end_err));
            }
            hipGraphExec_t exec = nullptr;
            err = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
            if (err != hipSuccess) {
                (void)hipGraphDestroy(graph);
                if (sw->dev) (void)hipFree(sw->dev);
                delete sw;
                return fail(W4_ECAPTURE, "hipGraphInstantiate failed: %s", hipGetErrorString(err));
            }
            sw->graph = graph;
            sw->exec = exec;
        }
        *out = sw;
        return ok();
    } catch (const std::bad_alloc&) {
        return fail(W4_ENOMEM, "w4_decode_linear_sweep_create: out of host memory");
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_linear_sweep_create: internal exception");
    }
}

w4_status w4_decode_linear_sweep(w4_sweep* sweep, void* stream)
{
    try {
        if (!sweep) return fail(W4_EINVAL, "w4_decode_linear_sweep: null handle");
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (sweep->use_graph) {
            hipError_t err = hipGraphLaunch(sweep->exec, s);
            if (err != hipSuccess) return hip_fail(err, "hipGraphLaunch");
            return ok();
        }
        if (sweep->mode == W4_SWEEP_PERSISTENT_EAGER) return launch_persistent(*sweep, s);
        return launch_all(sweep->calls, s);
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_linear_sweep: internal exception");
    }
}

w4_status w4_decode_linear_sweep_destroy(w4_sweep* sweep)
{
    try {
        if (!sweep) return ok();
        if (sweep->exec) (void)hipGraphExecDestroy(sweep->exec);
        if (sweep->graph) (void)hipGraphDestroy(sweep->graph);
        if (sweep->dev) (void)hipFree(sweep->dev);
        delete sweep;
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_linear_sweep_destroy: internal exception");
    }
}

w4_status w4_decode_linear_sweep_status(w4_sweep* sweep, int32_t* timed_out)
{
    try {
        if (!sweep || !timed_out) return fail(W4_EINVAL, "w4_decode_linear_sweep_status: null argument");
        *timed_out = 0;
        if (!sweep->dev) return ok();
        hipError_t err = hipDeviceSynchronize();
        if (err != hipSuccess) return hip_fail(err, "hipDeviceSynchronize");
        uint32_t word = 0;
        uint8_t* ctrl = reinterpret_cast<uint8_t*>(sweep->pargs.ctrl);
        err = hipMemcpy(&word, ctrl + kPersistCtrlErrorOffset, sizeof word, hipMemcpyDeviceToHost);
        if (err != hipSuccess) return hip_fail(err, "hipMemcpy (sweep status)");
        if (word) {
            const uint32_t zero = 0;
            err = hipMemcpy(ctrl + kPersistCtrlErrorOffset, &zero, sizeof zero, hipMemcpyHostToDevice);
            if (err != hipSuccess) return hip_fail(err, "hipMemcpy (sweep status clear)");
        }
        *timed_out = word ? 1 : 0;
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_linear_sweep_status: internal exception");
    }
}

w4_status w4_decode_linear_sweep_set_watchdog(w4_sweep* sweep, double seconds)
{
    try {
        if (!sweep) return fail(W4_EINVAL, "w4_decode_linear_sweep_set_watchdog: null handle");
        if (!(seconds > 0.0) || !(seconds <= 60.0))
            return fail(W4_EINVAL, "w4_decode_linear_sweep_set_watchdog: seconds=%g must be in (0, 60]", seconds);
        if (!sweep->dev) return fail(W4_EINVAL, "w4_decode_linear_sweep_set_watchdog: not a persistent sweep");
        unsigned long long ticks = (unsigned long long)(seconds * (double)kPersistTicksPerSecond);
        if (ticks < 1) ticks = 1;
        hipError_t err = hipDeviceSynchronize();
        if (err == hipSuccess)
            err = hipMemcpy(reinterpret_cast<uint8_t*>(sweep->pargs.ctrl) + kPersistCtrlWatchdogOffset, &ticks,
                            sizeof ticks, hipMemcpyHostToDevice);
        if (err != hipSuccess) return hip_fail(err, "hipMemcpy (sweep watchdog)");
        return ok();
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_linear_sweep_set_watchdog: internal exception");
    }
}

}  // extern "C"
