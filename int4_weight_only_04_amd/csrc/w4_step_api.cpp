// extern "C" entry points of the decode-step glue (embedding, residual add +
// RMSNorm, rotary embedding + KV append) and the full decode-step handle that
// chains them with the INT4 projections and the paged attention, eagerly or
// as one captured HIP graph.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>

#include <functional>
#include <new>
#include <vector>

#include "w4.h"
#include "w4_abi_util.h"
#include "w4_internal.h"

using namespace w4i;

namespace w4i {

w4_status check_kv_shape(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_ctx,
                         int32_t num_pages, const char* who)
{
    if (head_dim != kAttnHeadDim) return fail(W4_ESHAPE, "%s: head_dim=%d must be 128", who, head_dim);
    if (n_kv_heads < 1 || n_heads < n_kv_heads || n_heads % n_kv_heads != 0 || n_heads / n_kv_heads > 8)
        return fail(W4_ESHAPE, "%s: n_heads=%d must be 1..8 times n_kv_heads=%d", who, n_heads, n_kv_heads);
    if (page_size < 1 || page_size > 4096 || (page_size & (page_size - 1)) != 0)
        return fail(W4_ESHAPE, "%s: page_size=%d must be a power of two <= 4096", who, page_size);
    if (max_ctx < 1 || max_ctx > kAttnMaxCtx || num_pages < 1)
        return fail(W4_ESHAPE, "%s: max_ctx=%d num_pages=%d", who, max_ctx, num_pages);
    return W4_OK;
}

}  // namespace w4i

namespace {

w4_status check_norm(int64_t n, float eps, const char* who)
{
    if (n < 1 || n > kMaxHidden) return fail(W4_ESHAPE, "%s: n=%lld must be in [1, 2^20]", who, (long long)n);
    if (!(eps >= 0.0f) || !isfinite(eps)) return fail(W4_EINVAL, "%s: eps=%g must be finite and >= 0", who, eps);
    return W4_OK;
}

w4_status check_rope(const RopeCall& c, int32_t head_dim, const char* who)
{
    w4_status st = check_kv_shape(c.n_heads, c.n_kv, head_dim, c.page_size, c.max_ctx, c.num_pages, who);
    if (st != W4_OK) return st;
    if (!(c.theta > 0.0) || !isfinite(c.theta)) return fail(W4_EINVAL, "%s: theta=%g must be > 0", who, c.theta);
    if (!c.qkv || !c.pos || !c.q_out || !c.k_cache || !c.v_cache || !c.page_table)
        return fail(W4_EINVAL, "%s: null pointer", who);
    if (!aligned_to(c.qkv, 4) || (c.bias && !aligned_to(c.bias, 4)) || !aligned_to(c.pos, 4) ||
        !aligned_to(c.q_out, 2) || !aligned_to(c.page_table, 4) || (c.ctx_out && !aligned_to(c.ctx_out, 4)))
        return fail(W4_EALIGN, "%s: pointers must be aligned to their element size", who);
    // the caches are the attention's, which reads K rows in 16-byte words
    if (!aligned_to(c.k_cache, 16) || !aligned_to(c.v_cache, 16))
        return fail(W4_EALIGN, "%s: k_cache and v_cache must be 16-byte aligned", who);
    return W4_OK;
}

}  // namespace

extern "C" {

w4_status w4_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token, float* h,
                   void* stream)
{
    try {
        const char* who = "w4_embed";
        if (!table || !token || !h) return fail(W4_EINVAL, "%s: null pointer", who);
        if (hidden < 1 || hidden > kMaxHidden || vocab < 1 || vocab > ((int64_t)1 << 31))
            return fail(W4_ESHAPE, "%s: vocab=%lld hidden=%lld", who, (long long)vocab, (long long)hidden);
        if (!aligned_to(table, 2) || !aligned_to(token, 4) || !aligned_to(h, 4))
            return fail(W4_EALIGN, "%s: pointers must be aligned to their element size", who);
        hipError_t err = launch_embed(table, vocab, hidden, token, h, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_embed launch");
        return W4_OK;
    } catch (...) {
        return fail(W4_EINVAL, "w4_embed: internal exception");
    }
}

w4_status w4_add_rmsnorm(float* h, const float* y, const uint16_t* gamma, int64_t n, float eps, uint16_t* x,
                         void* stream)
{
    try {
        const char* who = "w4_add_rmsnorm";
        if (!h || !gamma || !x) return fail(W4_EINVAL, "%s: null pointer", who);
        w4_status st = check_norm(n, eps, who);
        if (st != W4_OK) return st;
        if (!aligned_to(h, 4) || (y && !aligned_to(y, 4)) || !aligned_to(gamma, 2) || !aligned_to(x, 2))
            return fail(W4_EALIGN, "%s: pointers must be aligned to their element size", who);
        hipError_t err = launch_add_rmsnorm(h, y, gamma, n, eps, x, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_add_rmsnorm launch");
        return W4_OK;
    } catch (...) {
        return fail(W4_EINVAL, "w4_add_rmsnorm: internal exception");
    }
}

w4_status w4_rope_kv_append(const float* qkv, const float* bias, const int32_t* pos, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_dim, double theta, uint16_t* q_out,
                            uint16_t* k_cache, uint16_t* v_cache, const int32_t* page_table,
                            int32_t num_pages, int32_t page_size, int32_t max_ctx, int32_t* ctx_len,
                            void* stream)
{
    try {
        RopeCall c{qkv, bias, pos, q_out, k_cache, v_cache, page_table, ctx_len, theta,
                   n_heads, n_kv_heads, page_size, num_pages, max_ctx};
        w4_status st = check_rope(c, head_dim, "w4_rope_kv_append");
        if (st != W4_OK) return st;
        hipError_t err = launch_rope_append(c, static_cast<hipStream_t>(stream));
        if (err != hipSuccess) return hip_fail(err, "w4_rope_kv_append launch");
        return W4_OK;
    } catch (...) {
        return fail(W4_EINVAL, "w4_rope_kv_append: internal exception");
    }
}

}  // extern "C"

struct w4_step {
    struct Op {
        std::function<hipError_t(hipStream_t)> run;
        int32_t kernels;
        const char* what;
    };
    std::vector<Op> ops;
    std::vector<void*> buffers;
    bool use_graph = false;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;

    ~w4_step()
    {
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
        for (void* p : buffers) (void)hipFree(p);
    }
};

namespace {

// Stand-in for the handle's own buffers while the projections are validated
// before anything is allocated (a non-null, 16-byte aligned address that is
// never passed to a kernel).
alignas(16) uint8_t kPlaceholder[16];

w4_status run_ops(const w4_step& st, hipStream_t stream)
{
    for (size_t i = 0; i < st.ops.size(); ++i) {
        hipError_t err = st.ops[i].run(stream);
        if (err != hipSuccess) {
            char what[96];
            snprintf(what, sizeof what, "decode step launch %zu (%s)", i, st.ops[i].what);
            return hip_fail(err, what);
        }
    }
    return W4_OK;
}

struct TraceLayout {
    size_t off[W4_TRACE_FIELDS];
    size_t bytes[W4_TRACE_FIELDS];
    size_t stride;
    size_t total;
};

TraceLayout trace_layout(const w4_step_desc& d)
{
    const size_t H = (size_t)d.hidden, R = (size_t)(d.n_heads + 2 * d.n_kv_heads) * 128;
    const size_t A = (size_t)d.n_heads * 128, I = (size_t)d.inter;
    TraceLayout t{};
    t.bytes[W4_TRACE_H_IN] = 4 * H;
    t.bytes[W4_TRACE_X1] = 2 * H;
    t.bytes[W4_TRACE_QKV] = 4 * R;
    t.bytes[W4_TRACE_Q] = 2 * A;
    t.bytes[W4_TRACE_ATTN] = 2 * A;
    t.bytes[W4_TRACE_O] = 4 * H;
    t.bytes[W4_TRACE_H_MID] = 4 * H;
    t.bytes[W4_TRACE_X2] = 2 * H;
    t.bytes[W4_TRACE_M] = 2 * I;
    t.bytes[W4_TRACE_D] = 4 * H;
    size_t o = 0;
    for (int f = 0; f < W4_TRACE_FIELDS; ++f) {
        t.off[f] = o;
        o += (t.bytes[f] + 255) & ~(size_t)255;
    }
    t.stride = o;
    t.total = (size_t)d.layers * o + t.off[W4_TRACE_QKV];  // final record: h and x_f
    return t;
}

w4_status validate_step(const w4_step_desc& d)
{
    const char* who = "w4_decode_step_create";
    if (d.layers < 1 || !d.layer) return fail(W4_EINVAL, "%s: need at least one layer", who);
    if (d.hidden < 8 || d.hidden > kMaxHidden || d.hidden % 8 != 0 || d.inter < 8 || d.vocab < 1 ||
        d.vocab > INT32_MAX - 1)
        return fail(W4_ESHAPE, "%s: hidden=%d inter=%d vocab=%lld", who, d.hidden, d.inter, (long long)d.vocab);
    w4_status st = check_kv_shape(d.n_heads, d.n_kv_heads, d.head_dim, d.page_size, d.max_ctx, d.num_pages, who);
    if (st != W4_OK) return st;
    st = check_norm(d.hidden, d.rms_eps, who);
    if (st != W4_OK) return st;
    if (!(d.rope_theta > 0.0) || !isfinite(d.rope_theta))
        return fail(W4_EINVAL, "%s: rope_theta=%g must be > 0", who, d.rope_theta);
    if (!d.embed || !d.final_norm || !d.page_table || !d.token || !d.pos || !d.logits)
        return fail(W4_EINVAL, "%s: null pointer in the descriptor", who);
    if (!aligned_to(d.embed, 2) || !aligned_to(d.final_norm, 8) || !aligned_to(d.page_table, 4) ||
        !aligned_to(d.token, 4) || !aligned_to(d.pos, 4) || !aligned_to(d.logits, 4) ||
        (d.trace && !aligned_to(d.trace, 256)))
        return fail(W4_EALIGN, "%s: descriptor pointers must be aligned to their element size (trace: 256)", who);
    void* ph = kPlaceholder;
    const int64_t qkv_rows = (int64_t)(d.n_heads + 2 * d.n_kv_heads) * 128;
    const int64_t attn_dim = (int64_t)d.n_heads * 128;
    char name[64];
    for (int32_t l = 0; l < d.layers; ++l) {
        const w4_layer_desc& L = d.layer[l];
        if (!L.attn_norm || !L.mlp_norm || !L.k_cache || !L.v_cache)
            return fail(W4_EINVAL, "%s: layer %d: null norm or cache pointer", who, l);
        if (!aligned_to(L.attn_norm, 16) || !aligned_to(L.mlp_norm, 8) || !aligned_to(L.k_cache, 16) ||
            !aligned_to(L.v_cache, 16) || (L.qkv_bias && !aligned_to(L.qkv_bias, 4)))
            return fail(W4_EALIGN, "%s: layer %d: pointers must be aligned to their element size", who, l);
        const GemvCall calls[4] = {
            {L.qkv_w, L.qkv_s, ph, ph, nullptr, nullptr, qkv_rows, d.hidden, d.group, kEpiPlain},
            {L.o_w, L.o_s, ph, ph, nullptr, nullptr, d.hidden, attn_dim, d.group, kEpiPlain},
            {L.gateup_w, L.gateup_s, ph, ph, nullptr, nullptr, 2 * (int64_t)d.inter, d.hidden, d.group, kEpiGateUp},
            {L.down_w, L.down_s, ph, ph, nullptr, nullptr, d.hidden, d.inter, d.group, kEpiPlain},
        };
        static const char* const kNames[4] = {"qkv", "o_proj", "gate/up", "down"};
        for (int p = 0; p < 4; ++p) {
            snprintf(name, sizeof name, "%s: layer %d %s", who, l, kNames[p]);
            st = check_gemv(calls[p], name);
            if (st != W4_OK) return st;
        }
    }
    const GemvCall lm{d.lm_w, d.lm_s, ph, d.logits, d.token, ph, d.vocab, d.hidden, d.group,
                      kEpiArgmax};
    snprintf(name, sizeof name, "%s: lm_head", who);
    return check_gemv(lm, name);
}

}  // namespace

extern "C" {

w4_status w4_decode_step_create(const w4_step_desc* desc, int32_t use_graph, w4_step** out)
{
    try {
        const char* who = "w4_decode_step_create";
        if (!out) return fail(W4_EINVAL, "%s: null output", who);
        *out = nullptr;
        if (!desc) return fail(W4_EINVAL, "%s: null descriptor", who);
        const w4_step_desc d = *desc;
        w4_status st = validate_step(d);
        if (st != W4_OK) return st;

        w4_step* sp = new w4_step();
        w4_step& s = *sp;
        s.use_graph = use_graph != 0;
        auto alloc = [&](size_t bytes) -> void* {
            void* p = nullptr;
            if (hipMalloc(&p, bytes < 256 ? 256 : bytes) != hipSuccess) return nullptr;
            s.buffers.push_back(p);
            return p;
        };
        const int64_t qkv_rows = (int64_t)(d.n_heads + 2 * d.n_kv_heads) * 128;
        const int64_t attn_dim = (int64_t)d.n_heads * 128;
        GemvCall lm{d.lm_w, d.lm_s, nullptr, d.logits, d.token, nullptr, d.vocab, d.hidden, d.group, kEpiArgmax};
        const size_t lm_ws_bytes = argmax_workspace_bytes(launch_grid(lm));
        // The attention norm of layers 1.. is folded into their qkv projection
        // (the down projection before it adds the residual and writes partial
        // sums of squares) when those partials fit the norm prologue's one load
        // round (hidden <= 4096).  The MLP and final norms stay separate
        // kernels: folded into gate/up and lm_head they cost those kernels more
        // (three times the input bytes per workgroup) than the norm kernel
        // costs on its own.
        const int64_t parts_down = residual_parts(d.hidden, d.inter, d.group);
        const bool fuse_attn = d.layers > 1 && parts_down <= kMaxNormParts;
        float* h = static_cast<float*>(alloc((size_t)d.hidden * 4));
        float* ss = fuse_attn ? static_cast<float*>(alloc((size_t)((parts_down + 3) & ~(int64_t)3) * 4)) : nullptr;
        float* y = static_cast<float*>(alloc((size_t)d.hidden * 4));
        uint16_t* x = static_cast<uint16_t*>(alloc((size_t)d.hidden * 2));
        float* qkv = static_cast<float*>(alloc((size_t)qkv_rows * 4));
        uint16_t* q = static_cast<uint16_t*>(alloc((size_t)attn_dim * 2));
        uint16_t* ao = static_cast<uint16_t*>(alloc((size_t)attn_dim * 2));
        uint16_t* mh = static_cast<uint16_t*>(alloc((size_t)d.inter * 2));
        int32_t* ctx = static_cast<int32_t*>(alloc(16));
        void* lm_ws = alloc(lm_ws_bytes);
        void* attn_ws = alloc(attn_workspace_bytes(d.n_heads, d.max_ctx));
        float2* rope_cs = static_cast<float2*>(alloc((size_t)d.max_ctx * 64 * sizeof(float2)));
        if (!h || !y || !x || !qkv || !q || !ao || !mh || !ctx || !lm_ws || !attn_ws || !rope_cs ||
            (fuse_attn && !ss)) {
            delete sp;
            return fail(W4_EHIP, "%s: hipMalloc of the step's activation buffers failed", who);
        }
        // rotary (cos, sin) of every position, once (the handle's constant)
        if (launch_rope_table(d.rope_theta, d.max_ctx, rope_cs, nullptr) != hipSuccess ||
            hipDeviceSynchronize() != hipSuccess) {
            delete sp;
            return fail(W4_EHIP, "%s: building the rotary table failed", who);
        }
        lm.x = x;
        lm.ws = lm_ws;

        const int64_t H = d.hidden;
        const float eps = d.rms_eps;
        const TraceLayout tl = trace_layout(d);
        uint8_t* trace = static_cast<uint8_t*>(d.trace);
        // Copy `bytes` from src into trace field f of record l (traced steps only).
        auto copy = [&](int32_t l, int f, const void* src, const char* what) {
            if (!trace) return;
            void* dst = trace + (size_t)l * tl.stride + tl.off[f];
            const size_t n = tl.bytes[f];
            s.ops.push_back({[=](hipStream_t st_) {
                                 return hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, st_);
                             },
                             1, what});
        };
        // layer 0's attention norm runs with the embedding lookup
        const uint16_t* g0 = d.layer[0].attn_norm;
        s.ops.push_back({[=](hipStream_t st_) {
                             return launch_embed_rmsnorm(d.embed, d.vocab, H, d.token, g0, eps, h, x, st_);
                         },
                         1, "embed + norm"});
        copy(0, W4_TRACE_H_IN, h, "trace h");
        copy(0, W4_TRACE_X1, x, "trace x1");
        for (int32_t l = 0; l < d.layers; ++l) {
            const w4_layer_desc L = d.layer[l];
            const bool qkv_normed = fuse_attn && l > 0;
            GemvCall qkv_call{L.qkv_w, L.qkv_s, x, qkv, nullptr, nullptr, qkv_rows, H, d.group, kEpiPlain};
            if (qkv_normed) {
                // this layer's attention norm, from h and the down projection's
                // partial sums; workgroup 0 writes the normalized x for the trace
                qkv_call.x = nullptr;
                qkv_call.norm_h = h;
                qkv_call.norm_gamma = L.attn_norm;
                qkv_call.norm_ss = ss;
                qkv_call.norm_parts = parts_down;
                qkv_call.norm_eps = eps;
                qkv_call.x_out = x;
            }
            s.ops.push_back({[=](hipStream_t st_) { return launch_gemv(qkv_call, st_); }, 1, "qkv"});
            if (qkv_normed) copy(l, W4_TRACE_X1, x, "trace x1");
            copy(l, W4_TRACE_QKV, qkv, "trace qkv");
            // rotary embedding and the KV append run inside the attention's
            // first kernel (q, and the new token's k and v, from the fp32 QKV
            // output); it also writes q for the trace and ctx = pos + 1
            const RopeCall rc{qkv,         L.qkv_bias,   d.pos,       q,           L.k_cache,
                              L.v_cache,   d.page_table, ctx,         d.rope_theta, d.n_heads,
                              d.n_kv_heads, d.page_size, d.num_pages, d.max_ctx,   rope_cs};
            const AttnCall ac{q, L.k_cache, L.v_cache, d.page_table, ctx, ao, attn_ws,
                              (float)(1.0 / sqrt((double)kAttnHeadDim)), d.max_ctx, d.n_heads, d.n_kv_heads,
                              d.page_size, d.num_pages, nullptr};
            s.ops.push_back({[=](hipStream_t st_) {
                                 AttnCall fused = ac;
                                 fused.rope = &rc;
                                 return launch_attn(fused, st_);
                             },
                             2, "rope + kv append + attention"});
            copy(l, W4_TRACE_Q, q, "trace q");
            copy(l, W4_TRACE_ATTN, ao, "trace attn");
            const GemvCall o_call{L.o_w, L.o_s, ao, y, nullptr, nullptr, H, attn_dim, d.group, kEpiPlain};
            s.ops.push_back({[=](hipStream_t st_) { return launch_gemv(o_call, st_); }, 1, "o_proj"});
            copy(l, W4_TRACE_O, y, "trace o");
            s.ops.push_back({[=](hipStream_t st_) { return launch_add_rmsnorm(h, y, L.mlp_norm, H, eps, x, st_); },
                             1, "mlp norm"});
            copy(l, W4_TRACE_H_MID, h, "trace h_mid");
            copy(l, W4_TRACE_X2, x, "trace x2");
            const GemvCall gu_call{L.gateup_w, L.gateup_s, x, mh, nullptr, nullptr, 2 * (int64_t)d.inter, H,
                                   d.group, kEpiGateUp};
            s.ops.push_back({[=](hipStream_t st_) { return launch_gemv(gu_call, st_); }, 1, "gate/up"});
            copy(l, W4_TRACE_M, mh, "trace m");
            GemvCall dn_call{L.down_w, L.down_s, mh, y, nullptr, nullptr, H, d.inter, d.group, kEpiPlain};
            const bool next_normed = fuse_attn && l + 1 < d.layers;
            if (next_normed) {
                // h += y in place, with the partial sums of squares of the new h
                dn_call.h_in = h;
                dn_call.h_out = h;
                dn_call.ss_out = ss;
            }
            s.ops.push_back({[=](hipStream_t st_) { return launch_gemv(dn_call, st_); }, 1, "down"});
            copy(l, W4_TRACE_D, y, "trace d");
            if (!next_normed) {
                const uint16_t* g_next = l + 1 < d.layers ? d.layer[l + 1].attn_norm : d.final_norm;
                s.ops.push_back({[=](hipStream_t st_) { return launch_add_rmsnorm(h, y, g_next, H, eps, x, st_); },
                                 1, l + 1 < d.layers ? "attn norm" : "final norm"});
            }
            copy(l + 1, W4_TRACE_H_IN, h, "trace h");
            if (!next_normed) copy(l + 1, W4_TRACE_X1, x, "trace x1");
        }
        // the argmax finalize also advances the position
        int32_t* pos = d.pos;
        s.ops.push_back({[=](hipStream_t st_) { return launch_gemv(lm, st_, pos); }, 2, "lm_head + argmax + advance"});

        if (s.use_graph) {
            hipStream_t cap = nullptr;
            hipError_t err = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
            if (err != hipSuccess) {
                delete sp;
                return hip_fail(err, "hipStreamCreateWithFlags");
            }
            err = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal);
            if (err != hipSuccess) {
                (void)hipStreamDestroy(cap);
                delete sp;
                return fail(W4_ECAPTURE, "hipStreamBeginCapture failed: %s", hipGetErrorString(err));
            }
            st = run_ops(s, cap);
            hipGraph_t graph = nullptr;
            hipError_t end_err = hipStreamEndCapture(cap, &graph);
            (void)hipStreamDestroy(cap);
            if (st != W4_OK || end_err != hipSuccess) {
                if (graph) (void)hipGraphDestroy(graph);
                delete sp;
                if (st != W4_OK) return st;
                return fail(W4_ECAPTURE, "hipStreamEndCapture failed: %s", hipGetErrorString(end_err));
            }
            s.graph = graph;
            err = hipGraphInstantiate(&s.exec, graph, nullptr, nullptr, 0);
            if (err != hipSuccess) {
                s.exec = nullptr;
                delete sp;
                return fail(W4_ECAPTURE, "hipGraphInstantiate failed: %s", hipGetErrorString(err));
            }
        }
        *out = sp;
        return W4_OK;
    } catch (const std::bad_alloc&) {
        return fail(W4_ENOMEM, "w4_decode_step_create: out of host memory");
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_step_create: internal exception");
    }
}

w4_status w4_decode_step(w4_step* step, void* stream)
{
    try {
        if (!step) return fail(W4_EINVAL, "w4_decode_step: null handle");
        hipStream_t s = static_cast<hipStream_t>(stream);
        if (step->use_graph) {
            hipError_t err = hipGraphLaunch(step->exec, s);
            if (err != hipSuccess) return hip_fail(err, "hipGraphLaunch");
            return W4_OK;
        }
        return run_ops(*step, s);
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_step: internal exception");
    }
}

w4_status w4_decode_step_trace_layout(const w4_step_desc* desc, size_t* offsets, size_t* layer_stride,
                                      size_t* total_bytes)
{
    try {
        if (!desc || !offsets || !layer_stride || !total_bytes)
            return fail(W4_EINVAL, "w4_decode_step_trace_layout: null argument");
        if (desc->layers < 1 || desc->hidden < 1 || desc->n_heads < 1 || desc->n_kv_heads < 0 || desc->inter < 1)
            return fail(W4_ESHAPE, "w4_decode_step_trace_layout: bad dimensions");
        const TraceLayout t = trace_layout(*desc);
        for (int f = 0; f < W4_TRACE_FIELDS; ++f) offsets[f] = t.off[f];
        *layer_stride = t.stride;
        *total_bytes = t.total;
        return W4_OK;
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_step_trace_layout: internal exception");
    }
}

w4_status w4_decode_step_launches(const w4_step* step, int32_t* count)
{
    if (!step || !count) return fail(W4_EINVAL, "w4_decode_step_launches: null argument");
    int32_t n = 0;
    for (const auto& op : step->ops) n += op.kernels;
    *count = n;
    return W4_OK;
}

w4_status w4_decode_step_destroy(w4_step* step)
{
    try {
        delete step;
        return W4_OK;
    } catch (...) {
        return fail(W4_EINVAL, "w4_decode_step_destroy: internal exception");
    }
}

}  // extern "C"
