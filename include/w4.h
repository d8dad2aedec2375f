/*
 * w4.h -- C ABI of the MI355X (gfx950) INT4 weight-only decode GEMV library.
 *
 * The operation.  "How To Build Your Own LLM Runtime From Scratch"
 * (aitrending.vip), section "Technical Details", first bullet: the runtime
 * packs its weights, stores them as INT4 and dequantizes them at run time;
 * the third page (noticiai.com.br, "As tres licoes", lesson 3) says the
 * activations stay in floating point (the INT8-activation path was removed).
 * The pages fix no quantization format; this library uses zero point 8 and one
 * fp16 scale per row and per group of G consecutive inputs:
 *
 *     w[n][k] = (q[n][k] - 8) * s[n][k / G],   q in {0..15}
 *     y[n]    = sum_k w[n][k] * x[k]            x fp16, products and sums fp32
 *
 * The decode step that runs these products once per token, for the fused QKV,
 * o_proj, fused gate/up (with a SiLU-gated epilogue), down_proj and lm_head
 * projections of each of 28 layers of a 3584-hidden / 18944-MLP / 152064-vocab
 * model (same page, section 技术解析, first bullet), is replayed as one captured
 * graph: the pages attribute a ~7x per-token gain to graph capture (section
 * "CUDA Graph Optimization" / "Technical Details", third bullet).
 *
 * Conventions for every entry point.
 *   - Every function returns a w4_status; W4_OK is 0.  On failure nothing has
 *     been launched, and w4_last_error() returns a thread-local message.
 *   - No C++ exception crosses this boundary.
 *   - "device" pointers are HIP device allocations (e.g. torch CUDA tensors
 *     on ROCm); "host" pointers are ordinary CPU memory.  The caller owns every
 *     buffer; the library never frees caller memory.
 *   - Device calls are asynchronous on the given stream (a hipStream_t passed
 *     as void*, NULL = the legacy default stream).  A device fault surfaces at
 *     the caller's next synchronization, not in the call.
 *   - Calls on different streams may run concurrently from different threads;
 *     one sweep handle must not be used by two threads at once.
 *
 * Packed layout "W4T4" (produced by w4_pack, consumed by the kernels).
 *   - Rows are grouped in tiles of 4.  Plain layout: tile t holds rows
 *     4t..4t+3 (ceil(n/4) tiles).  Gate/up layout (n = 2I): the gate half and
 *     the up half are tiled separately, gate tiles first (2*ceil(I/4) tiles),
 *     so that gate row j and up row j sit in the same slot of tiles j/4 and
 *     ceil(I/4) + j/4.  Slots beyond the logical rows are padding (nibble 8,
 *     scale +0.0, i.e. a zero weight).
 *   - Weights: the 8 inputs 8j..8j+7 of tile t occupy 16 bytes at byte offset
 *     (t * (k/8) + j) * 16; little-endian 32-bit word r of those 16 bytes holds
 *     tile row r.  Nibble slot p of a word (bits 4p..4p+3) holds input offset
 *     2p for p < 4 and 2(p-4)+1 for p >= 4, so the masks 0x000F000F and
 *     0x00F000F0 (and the same after a shift by 8) pull out the input pairs
 *     (0,1), (2,3), (4,5), (6,7) as two fp16 lanes each.
 *   - Scales: tile t, group g occupies 8 bytes at byte offset
 *     (t * (k/G) + g) * 8; the fp16 at bytes 2r..2r+1 is tile row r's scale.
 *   - Size: weight bytes = tiles * k / 2 * 4, scale bytes = tiles * (k/G) * 8.
 *
 * Shape rules (W4_ESHAPE otherwise): n >= 1; k >= 8; G a power of two with
 * 8 <= G <= k and k % G == 0; k <= 32768; gate/up: n even; argmax: n below
 * 2^31 - 1.  Device pointers must be 16-byte aligned (W4_EALIGN).
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t w4_status;

#define W4_OK 0
#define W4_EINVAL 1   /* null pointer, bad enum, nibble > 15, size mismatch */
#define W4_ESHAPE 2   /* shape outside the rules above                     */
#define W4_EALIGN 3   /* device pointer not 16-byte aligned                */
#define W4_EHIP 4     /* a HIP runtime call failed (message names it)      */
#define W4_ENOMEM 5   /* host allocation failed                            */
#define W4_ECAPTURE 6 /* graph capture / instantiation failed              */

#define W4_LAYOUT_PLAIN 0
#define W4_LAYOUT_GATEUP 1

/* Status code -> static string ("W4_OK", "W4_EINVAL", ...). */
const char* w4_status_string(w4_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* w4_last_error(void);

/* ABI version of this header: 1. */
int32_t w4_abi_version(void);

/*
 * Packed sizes of an n x k matrix with group size `group` in `layout`
 * (W4_LAYOUT_PLAIN or W4_LAYOUT_GATEUP), in bytes.  Host only, no device.
 * Outputs must be non-null.
 */
w4_status w4_packed_size(int64_t n, int64_t k, int32_t group, int32_t layout,
                         size_t* weight_bytes, size_t* scale_bytes);

/*
 * Pack logical INT4 weights into the W4T4 layout ("Technical Details",
 * first bullet: weight packing).  Host only.
 *   q        host, uint8 [n][k] row-major, every value in 0..15 (W4_EINVAL
 *            names the first offending element otherwise; the outputs are
 *            then partially written);
 *   scales   host, fp16 bit patterns [n][k/group] row-major;
 *   packed_w host, packed_w_bytes == the weight size from w4_packed_size;
 *   packed_s host, packed_s_bytes == the scale size from w4_packed_size.
 * Padding slots are written too, so the outputs are fully defined.
 */
w4_status w4_pack(const uint8_t* q, const uint16_t* scales, int64_t n, int64_t k, int32_t group,
                  int32_t layout, void* packed_w, size_t packed_w_bytes, void* packed_s,
                  size_t packed_s_bytes);

/*
 * Workspace bytes w4_gemv needs: 0 without argmax; with argmax, 8 bytes per
 * workgroup of the shape's launch (about 152 KiB for 152064 x 3584).  Host
 * only.
 */
w4_status w4_gemv_workspace_size(int64_t n, int64_t k, int32_t group, int32_t with_argmax,
                                 size_t* bytes);

/*
 * y = W x for a plain-layout packed matrix: the run-time INT4 dequantization
 * GEMV of "How To Build Your Own LLM Runtime From Scratch" (aitrending.vip),
 * "Technical Details", first bullet, with fp16 activations (third page,
 * "As tres licoes", lesson 3).  Optionally with the lm_head argmax epilogue,
 * the greedy reading of the runtime's own sampling code (first page,
 * "Industry Insight", first bullet): lowest index of the largest y; NaN never
 * wins; -1 if every y is NaN.  Device, asynchronous on `stream`; with argmax a
 * second, one-workgroup kernel on the same stream reduces the per-workgroup
 * partials.
 *   packed_w, packed_s  device, from w4_pack(..., W4_LAYOUT_PLAIN, ...);
 *   x        device, fp16 [k];
 *   y        device, fp32 [n] (written for every row);
 *   argmax   device int32 [1], or NULL for no argmax;
 *   workspace device, >= w4_gemv_workspace_size bytes when argmax != NULL
 *            (may be NULL otherwise); no initial contents are needed.  Calls
 *            that may run at the same time need separate workspaces.
 */
w4_status w4_gemv(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                  int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                  int32_t group, void* stream);

/*
 * w4_gemv with the argmax epilogue, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same outputs as w4_gemv(..., argmax, workspace, ...),
 * but the per-workgroup partials live in a static device array of the
 * library (256 KiB per GPU, held until the process ends), so no workspace is
 * passed and nothing is allocated or freed.  Every call on one GPU shares that
 * array: calls that may overlap on the same GPU (different streams, threads)
 * race and must be serialized by the caller.  The array needs no initial
 * contents.  Shapes whose launch needs more partials than the array holds
 * (more than ~520K rows at k = 3584) return W4_ESHAPE; otherwise rules and
 * errors as for w4_gemv.  Device, asynchronous on `stream`.
 */
w4_status w4_gemv_argmax_noalloc(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                                 int32_t* argmax, int64_t n, int64_t k, int32_t group, void* stream);

/*
 * Fused gate/up + SiLU: the gate/up GEMV that the pages' instruction lesson is
 * about (first page, section 技术解析, engineering-lessons bullet, item 2; third
 * page, "As tres licoes", lesson 3), with the SiLU-gated MLP epilogue of the model family
 * they name.  With I = n_total / 2, g = rows [0, I) of W x and
 * u = rows [I, 2I), h[j] = silu(g[j]) * u[j] rounded to fp16 (nearest even),
 * silu(t) = t / (1 + e^-t).  Device, asynchronous on `stream`.
 *   packed_w, packed_s  device, from w4_pack(..., W4_LAYOUT_GATEUP, ...);
 *   x  device fp16 [k];  h  device fp16 [n_total / 2].
 */
w4_status w4_gemv_gateup_silu(const void* packed_w, const void* packed_s, const uint16_t* x,
                              uint16_t* h, int64_t n_total, int64_t k, int32_t group, void* stream);

/*
 * Workspace bytes w4_gemm needs for an m x n x k product: 0 when the grid
 * already covers the chip, else the split-k partials (splits x m x n fp32,
 * splits <= 8; 28.3 MB for 512 x 4608 x 3584, split 3 ways).  Host only.
 */
w4_status w4_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t group, size_t* bytes);

/*
 * Prefill GEMM over a block of m prompt tokens (the pages report the
 * first-token latency of a 512-token prompt: "How To Build Your Own LLM
 * Runtime From Scratch", aitrending.vip, "Technical Details",
 * performance-metrics bullet): y[t][j] = sum_k x[t][k] * w[j][k] for every
 * token row t < m and weight row j < n, with w = (q - 8) * s as for w4_gemv.
 * The weights are dequantized to fp16 (rounded to nearest even) and
 * multiplied on the matrix cores with fp32 accumulation; split-k partials
 * are summed in a fixed order, so results are deterministic.  Device,
 * asynchronous on `stream` (one kernel, or two when split).
 *   packed_w, packed_s  device, from w4_pack(..., W4_LAYOUT_PLAIN, ...);
 *   x  device, fp16 [m][k] row-major (16-byte aligned);
 *   y  device, fp32 [m][n] row-major (4-byte aligned), written in full;
 *   workspace  device, >= w4_gemm_workspace_size bytes, 16-byte aligned (may
 *              be NULL when that size is 0); no initial contents; calls that
 *              may run at the same time need separate workspaces.
 * Shape rules as for w4_gemv, plus 1 <= m <= 2^20 (W4_ESHAPE otherwise).
 */
w4_status w4_gemm(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                  void* workspace, size_t workspace_bytes, int64_t m, int64_t n, int64_t k,
                  int32_t group, void* stream);

/*
 * Prefill gate/up + SiLU: with I = n_total / 2, for every token row t,
 * h[t][j] = silu(g) * u rounded to fp16, g = row t of the product with weight
 * rows [0, I), u = with rows [I, 2I).  Same arithmetic as w4_gemm.
 *   packed_w, packed_s  device, from w4_pack(..., W4_LAYOUT_GATEUP, ...);
 *   x  device fp16 [m][k] row-major;  h  device fp16 [m][n_total / 2] row-major.
 */
w4_status w4_gemm_gateup_silu(const void* packed_w, const void* packed_s, const uint16_t* x,
                              uint16_t* h, int64_t m, int64_t n_total, int64_t k, int32_t group,
                              void* stream);

/*
 * Diagnostic, not part of the method: a kernel that only reads `bytes`
 * (a positive multiple of 16) of device memory at `buf` (16-byte aligned)
 * with the same 16-byte non-temporal loads as the GEMVs' weight stream, and
 * stores a checksum word per workgroup into `sink` (device uint32 [1024],
 * contents meaningless).  Launched once per matrix of a sweep, in the same
 * order, it measures the practical ceiling of a sweep built from one kernel
 * per projection.  Device, asynchronous.
 */
w4_status w4_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * W4A8: the INT8-activation variant of the GEMV, the path the pages' runtime
 * implemented, tested and removed ("Tutorial: como construir seu proprio
 * runtime de LLM do zero", noticiai.com.br, "As tres licoes", lesson 3;
 * "How To Build Your Own LLM Runtime From Scratch", aitrending.vip,
 * "Technical Details", low-level pitfalls bullet).  The pages give no
 * quantization rule; this library quantizes x per group of G inputs (the
 * weights' G), symmetric, in binary32 with round-to-nearest-even:
 *     amax = max |x| over the group, inv = 127 / amax,
 *     c[k] = clamp(rint(x[k] * inv), -127, 127),  s_g = amax / 127
 *     (amax == 0: c = 0, s_g = 0)
 * and computes y[n] = sum_k (q[n][k] - 8) * s[n][g] * c[k] * s_g, each
 * 8-input block's integer sum exact (v_dot4_i32_i8), fp32 accumulation.
 *
 * w4_quantize_act8: codes and scales of one fp16 vector.  Device, async.
 *   x       device fp16 [k], 16-byte aligned;
 *   codes   device int8 [k], 8-byte aligned, in W4T4 block order: the bytes
 *           8j..8j+7 hold inputs 8j + (0, 4, 1, 5, 2, 6, 3, 7) (the order
 *           of the nibbles in (word & 0x0F0F0F0F) then ((word >> 4) &
 *           0x0F0F0F0F) of a packed weight word);
 *   scales  device fp32 [k / group].
 * Shape rules as for w4_gemv (k, group).
 */
w4_status w4_quantize_act8(const uint16_t* x, int64_t k, int32_t group, int8_t* codes, float* scales,
                           void* stream);

/* w4_gemv with int8 activation codes and per-group scales from
 * w4_quantize_act8 (same group) in place of fp16 x; the same outputs,
 * argmax option, workspace and rules (codes 16-byte aligned). */
w4_status w4_gemv_a8(const void* packed_w, const void* packed_s, const int8_t* codes, const float* act_scales,
                     float* y, int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                     int32_t group, void* stream);

/* w4_gemv_gateup_silu with int8 activation codes (see w4_gemv_a8). */
w4_status w4_gemv_gateup_silu_a8(const void* packed_w, const void* packed_s, const int8_t* codes,
                                 const float* act_scales, uint16_t* h, int64_t n_total, int64_t k, int32_t group,
                                 void* stream);

/*
 * Workspace bytes w4_attn_decode needs: (130 x 4) bytes per query head per
 * 128-token chunk of max_ctx (about 0.47 MB for 28 heads at 4096).  Host only.
 */
w4_status w4_attn_decode_workspace_size(int32_t n_heads, int32_t max_ctx, size_t* bytes);

/*
 * Decode attention of one new token over a paged KV cache, the step between
 * the QKV and o_proj projections ("How To Build Your Own LLM Runtime From
 * Scratch", aitrending.vip, "Technical Details", architecture bullet: paged
 * KV cache and attention).  For query head h and KV head g = h / (n_heads /
 * n_kv_heads):
 *     o[h] = sum_{t < ctx} softmax_t(scale * q[h] . K[t][g]) V[t][g]
 * with token t in physical page page_table[t / page_size], slot
 * t % page_size.  fp32 arithmetic, fp16 output (nearest even).  Device,
 * asynchronous on `stream` (two kernels).
 *   q           device fp16 [n_heads][128];
 *   k_cache, v_cache  device fp16 [num_pages][n_kv_heads][page_size][128];
 *   page_table  device int32, >= ceil(max_ctx / page_size) entries, each in
 *               [0, num_pages) (an entry outside is clamped into range: a
 *               wrong result, never a read outside the caches);
 *   ctx_len     device int32 [1]: tokens in the cache, read by the kernels
 *               (so a captured graph replays as the context grows), clamped
 *               to [1, max_ctx];
 *   out         device fp16 [n_heads][128];
 *   workspace   device, >= w4_attn_decode_workspace_size(n_heads, max_ctx)
 *               bytes, 16-byte aligned; no initial contents; calls that may
 *               run at the same time need separate workspaces.
 * Shape rules: head_dim == 128; n_heads = 1..8 x n_kv_heads; page_size a
 * power of two <= 4096; 1 <= max_ctx <= 2^20 (W4_ESHAPE otherwise).
 */
w4_status w4_attn_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                         const int32_t* page_table, int32_t num_pages, const int32_t* ctx_len,
                         int32_t max_ctx, uint16_t* out, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, int32_t page_size, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/* One projection of the per-token linear sweep. */
#define W4_PROJ_PLAIN 0         /* w4_gemv, out = float y[n]                  */
#define W4_PROJ_GATEUP_SILU 1   /* w4_gemv_gateup_silu, out = fp16 h[n/2]     */
#define W4_PROJ_LMHEAD_ARGMAX 2 /* w4_gemv with argmax, out = float y[n]      */

typedef struct w4_proj_desc {
    int32_t kind;          /* W4_PROJ_*                                      */
    int32_t group;         /* G                                              */
    int64_t n;             /* rows (gate/up: n_total = 2I)                   */
    int64_t k;             /* inputs                                         */
    const void* packed_w;  /* device                                         */
    const void* packed_s;  /* device                                         */
    const uint16_t* x;     /* device fp16 [k]                                */
    void* out;             /* device float [n] or fp16 [n/2]                 */
    int32_t* argmax;       /* device int32 [1] (LMHEAD_ARGMAX only)          */
    void* workspace;       /* device (LMHEAD_ARGMAX only)                    */
    size_t workspace_bytes;
} w4_proj_desc;

typedef struct w4_sweep w4_sweep;

/* How a sweep is issued (the `mode` of w4_decode_linear_sweep_create). */
#define W4_SWEEP_EAGER 0            /* one GEMV kernel per projection, launched one by one        */
#define W4_SWEEP_GRAPH 1            /* the same kernels captured into one HIP graph               */
#define W4_SWEEP_PERSISTENT 2       /* one persistent cooperative kernel for all projections,     */
                                    /* captured into one HIP graph                               */
#define W4_SWEEP_PERSISTENT_EAGER 3 /* the persistent kernel's launches, not captured            */

/*
 * Build the per-token sweep over `count` projections, run in array order
 * (the decode order: per layer QKV, o_proj, gate/up, down; then lm_head);
 * each projection's math starts only after the previous one has finished.
 * W4_SWEEP_GRAPH captures all launches into one HIP graph (one submission
 * per token, as the pages' "CUDA Graph Optimization" bullet describes);
 * W4_SWEEP_EAGER keeps them as eager launches, for the eager-vs-graph
 * comparison.
 *
 * W4_SWEEP_PERSISTENT runs every projection inside one cooperative kernel
 * with one workgroup per CU: while a projection finishes, each workgroup
 * already has the next projection's first weights in flight, and the next
 * projection's input reaches every workgroup as data written by the other
 * workgroups after they finished (tagged words plus arrival counters in
 * device memory), so the decode-order dependency is kept without a kernel
 * boundary.  Its outputs are bit-identical to the one-kernel path's.  It
 * covers sweeps of at most 256 projections whose every k is a multiple of
 * 512 and at most 20480, with 64 <= G <= 512 (W4_ESHAPE otherwise); lm_head workspaces then need
 * w4_gemv_workspace_size bytes for at most one workgroup per CU.  The handle
 * allocates its device state at create (phase table, control block, two
 * input buffers of k/2 8-byte words; ~160 KB for the 7B shapes).  Every wait
 * in the kernel is bounded by a watchdog (200 ms by default): on a timeout
 * the kernel ends normally, its outputs are undefined, and
 * w4_decode_linear_sweep_status reports it.  Only one persistent sweep may
 * run on a GPU at a time (it needs every CU).  On MI355X it is slower than
 * W4_SWEEP_GRAPH for the 28-layer sweep (3.27 ms against 0.91 ms): it is
 * kept as the dependency-checked single-kernel form, not as the fast path.
 *
 * Every descriptor is validated first.  The handle keeps a copy of the
 * descriptors and the graph, which bakes in every pointer: the buffers must
 * stay alive and in place until w4_decode_linear_sweep_destroy.  Capture uses
 * a private stream of the library, so create takes no stream.
 */
w4_status w4_decode_linear_sweep_create(const w4_proj_desc* projs, int32_t count,
                                        int32_t mode, w4_sweep** out);

/* Run one token's sweep on `stream` (graph launch or eager launches).  The
 * lm_head projection contributes two kernels (GEMV + argmax finalize). */
w4_status w4_decode_linear_sweep(w4_sweep* sweep, void* stream);

/* Release the handle (NULL is accepted). */
w4_status w4_decode_linear_sweep_destroy(w4_sweep* sweep);

/* Persistent modes: waits for the device, then sets *timed_out to 1 if a
 * watchdog timeout happened in any run since the last call (and clears it),
 * else 0.  Other modes: always 0.  Host, synchronizing. */
w4_status w4_decode_linear_sweep_status(w4_sweep* sweep, int32_t* timed_out);

/* Persistent modes: the watchdog bound of every wait in the kernel, in
 * seconds (0 < seconds <= 60); takes effect from the next run.  Host,
 * synchronizing.  W4_EINVAL for other modes. */
w4_status w4_decode_linear_sweep_set_watchdog(w4_sweep* sweep, double seconds);

/*
 * The glue of a full decode step.  The pages name the model (Qwen2.5-Coder-7B:
 * 28 decoder layers, hidden 3584, MLP 18944, vocabulary 152064; second page,
 * "How to Build Your Own LLM Runtime from Scratch" (brifing.si), section 7
 * "Model Dimensions and Structure") and the parts of its runtime (first page,
 * "Technical Details", architecture bullet: INT4 weights, paged KV cache,
 * attention) but not the decoder's equations.  They are read as that model
 * family's pre-norm decoder: token embedding, RMSNorm before attention and
 * before the MLP, rotary position embedding on q and k (pairs (i, i + 64) of
 * each 128-wide head), grouped KV heads, SiLU-gated MLP, residual adds in
 * fp32, a final RMSNorm and the lm_head with a greedy argmax.
 */

/*
 * Embedding lookup: h[i] = table[t][i] widened to fp32 for i < hidden, with
 * t = *token read on the device (clamped into [0, vocab): a wrong row, never
 * a read outside the table).  Device, asynchronous.
 *   table  device fp16 [vocab][hidden];  token  device int32 [1];
 *   h      device fp32 [hidden].
 * Rules: 1 <= hidden <= 2^20, vocab >= 1 (W4_ESHAPE); h 4-byte, table and
 * token naturally aligned (W4_EALIGN).
 */
w4_status w4_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token, float* h,
                   void* stream);

/*
 * Residual add and RMSNorm, one kernel: if y != NULL, h[i] += y[i] in fp32
 * (stored back to h); then
 *     x[i] = fp16( h[i] * gamma[i] / sqrt(mean_j h[j]^2 + eps) )
 * (fp32 arithmetic, one rounding to fp16 at the end, nearest even).
 * Device, asynchronous, one workgroup; the sum of squares is reduced in a
 * fixed order (deterministic).
 *   h  device fp32 [n] (read, and written when y != NULL);  y  device fp32 [n]
 *   or NULL;  gamma  device fp16 [n];  x  device fp16 [n].
 * Rules: 1 <= n <= 2^20 (W4_ESHAPE); eps >= 0 and finite (W4_EINVAL).
 */
w4_status w4_add_rmsnorm(float* h, const float* y, const uint16_t* gamma, int64_t n, float eps, uint16_t* x,
                         void* stream);

/*
 * The residual add and the RMSNorm above, folded into the projections on
 * either side of them (the same decoder reading; the fold itself is this
 * library's, not the pages').  A projection whose output feeds the residual
 * stream (o_proj, down) adds it and emits partial sums of squares; the next
 * projection (qkv, gate/up, lm_head) normalizes h itself from those partials,
 * so no separate norm kernel runs between them.
 *
 * Number of partial sums w4_gemv_residual writes for an n x k projection
 * (one per 4-row tile while n <= 65532; fewer for taller matrices).  Host only.
 * Rules as for w4_gemv (W4_ESHAPE).
 */
w4_status w4_residual_parts(int64_t n, int64_t k, int32_t group, int64_t* parts);

/*
 * y = W x as w4_gemv (no argmax), then h_out[i] = h_in[i] + y[i] in fp32
 * (i < n; h_out may be h_in) and ss_part[u] = the sum of h_out[i]^2 over the
 * rows of partial u (fp32, a fixed order), for u < w4_residual_parts(n, k,
 * group).  Device, asynchronous, one kernel.
 *   x  device fp16 [k];  y, h_in, h_out  device fp32 [n];
 *   ss_part  device fp32, 16-byte aligned, w4_residual_parts floats written.
 * Rules as for w4_gemv; y, h_in and h_out 4-byte aligned (W4_EALIGN).
 */
w4_status w4_gemv_residual(const void* packed_w, const void* packed_s, const uint16_t* x, float* y,
                           const float* h_in, float* h_out, float* ss_part, int64_t n, int64_t k, int32_t group,
                           void* stream);

/*
 * RMSNorm folded into the GEMV input: with S = the sum of ss_part[0 .. parts)
 * (fp32, a fixed order) and r = 1 / sqrt(S / k + eps),
 *     x[i] = fp16( (h[i] * r) * gamma[i] )      (fp32 products, nearest even)
 * and then y = W x exactly as w4_gemv, optionally with the argmax epilogue.
 * Every workgroup computes the same x; the first also stores it to x_out
 * when x_out != NULL.  Device, asynchronous (one kernel, two with argmax).
 *   h  device fp32 [k];  gamma  device fp16 [k];  x_out  device fp16 [k] or
 *   NULL;  ss_part  device fp32, parts values, readable up to the next
 *   multiple of 4 floats (the values past parts are ignored);
 *   y, argmax, workspace as for w4_gemv.
 * Rules as for w4_gemv; 1 <= parts <= 1024 (W4_ESHAPE); eps >= 0 and finite
 * (W4_EINVAL); h, gamma, ss_part and x_out 16-byte aligned (W4_EALIGN).
 */
w4_status w4_gemv_rmsnorm(const void* packed_w, const void* packed_s, const float* h, const uint16_t* gamma,
                          const float* ss_part, int64_t parts, float eps, uint16_t* x_out, float* y,
                          int32_t* argmax, void* workspace, size_t workspace_bytes, int64_t n, int64_t k,
                          int32_t group, void* stream);

/*
 * w4_gemv_gateup_silu with its input normalized as in w4_gemv_rmsnorm.
 *   h_mlp  device fp16 [n_total / 2], the SiLU-gated output.
 */
w4_status w4_gemv_gateup_silu_rmsnorm(const void* packed_w, const void* packed_s, const float* h,
                                      const uint16_t* gamma, const float* ss_part, int64_t parts, float eps,
                                      uint16_t* x_out, uint16_t* h_mlp, int64_t n_total, int64_t k, int32_t group,
                                      void* stream);

/*
 * Rotary embedding and KV-cache append for one new token at position
 * p = *pos (device int32, clamped into [0, max_ctx)).  qkv holds the fused
 * projection's output: n_heads query heads, then n_kv_heads key heads, then
 * n_kv_heads value heads, 128 values each; bias (same length) is added first
 * when not NULL.  Each q and k head is rotated pairwise,
 *     r[i]      = x[i] cos(a_i) - x[i + 64] sin(a_i)
 *     r[i + 64] = x[i + 64] cos(a_i) + x[i] sin(a_i),   a_i = p * theta^(-2i/128)
 * (angle, sine and cosine in double, the rotation in fp32).  Rotated q goes to
 * q_out (fp16); rotated k and the unrotated v go to the caches' slot of token
 * p: page page_table[p / page_size] (clamped into [0, num_pages)), slot
 * p % page_size.  ctx_len (when not NULL) is set to p + 1, the attention's
 * context length.  Device, asynchronous, one kernel.
 *   qkv   device fp32 [(n_heads + 2 n_kv_heads) * 128];  bias likewise or NULL;
 *   q_out device fp16 [n_heads][128];
 *   k_cache, v_cache  device fp16 [num_pages][n_kv_heads][page_size][128]
 *   (the layout w4_attn_decode reads), 16-byte aligned (W4_EALIGN
 *   otherwise);  page_table  device int32.
 * Rules as for w4_attn_decode (head_dim 128, n_heads 1..8 x n_kv_heads,
 * power-of-two page_size <= 4096, 1 <= max_ctx <= 2^20); theta > 0.
 */
w4_status w4_rope_kv_append(const float* qkv, const float* bias, const int32_t* pos, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_dim, double theta, uint16_t* q_out,
                            uint16_t* k_cache, uint16_t* v_cache, const int32_t* page_table,
                            int32_t num_pages, int32_t page_size, int32_t max_ctx, int32_t* ctx_len,
                            void* stream);

/* Weights and KV cache of one decoder layer (all device).  Packed matrices
 * come from w4_pack (plain layout unless stated). */
typedef struct w4_layer_desc {
    const uint16_t* attn_norm;  /* fp16 [hidden]                                   */
    const void* qkv_w;          /* (n_heads + 2 n_kv) * 128 rows, hidden inputs    */
    const void* qkv_s;
    const float* qkv_bias;      /* fp32 [(n_heads + 2 n_kv) * 128] or NULL          */
    const void* o_w;            /* hidden rows, n_heads * 128 inputs               */
    const void* o_s;
    const uint16_t* mlp_norm;   /* fp16 [hidden]                                   */
    const void* gateup_w;       /* gate/up layout, 2 * inter rows, hidden inputs   */
    const void* gateup_s;
    const void* down_w;         /* hidden rows, inter inputs                       */
    const void* down_s;
    uint16_t* k_cache;          /* fp16 [num_pages][n_kv][page_size][128],         */
    uint16_t* v_cache;          /* both 16-byte aligned (read in 16-byte words)    */
} w4_layer_desc;

typedef struct w4_step_desc {
    int32_t layers;
    int32_t hidden;
    int32_t n_heads;
    int32_t n_kv_heads;
    int32_t head_dim;           /* must be 128                                     */
    int32_t inter;              /* MLP width                                       */
    int64_t vocab;
    int32_t group;              /* G of every packed matrix                        */
    int32_t page_size;
    int32_t num_pages;          /* pages in each layer's cache                     */
    int32_t max_ctx;
    float rms_eps;
    double rope_theta;
    const uint16_t* embed;      /* fp16 [vocab][hidden]                            */
    const w4_layer_desc* layer; /* host array [layers], copied at create           */
    const uint16_t* final_norm; /* fp16 [hidden]                                   */
    const void* lm_w;           /* vocab rows, hidden inputs                       */
    const void* lm_s;
    const int32_t* page_table;  /* device int32, >= ceil(max_ctx / page_size), shared by the layers */
    int32_t* token;             /* device int32 [1]: input token, replaced by the argmax */
    int32_t* pos;               /* device int32 [1]: its position, incremented     */
    float* logits;              /* device fp32 [vocab], written                    */
    void* trace;                /* device, w4_decode_step_trace_layout bytes, or NULL */
} w4_step_desc;

/* Intermediate values a step copies into desc->trace (for checking each
 * stage on its own); layer l's record starts at l * layer_stride, the field
 * at offsets[field] within it (256-byte aligned).  The record at
 * layers * layer_stride holds the final residual stream (W4_TRACE_H_IN) and
 * the final norm's output (W4_TRACE_X1). */
#define W4_TRACE_H_IN 0   /* fp32 [hidden]   residual stream at the layer input  */
#define W4_TRACE_X1 1     /* fp16 [hidden]   attention-norm output               */
#define W4_TRACE_QKV 2    /* fp32 [(n_heads + 2 n_kv) * 128]  projection, no bias */
#define W4_TRACE_Q 3      /* fp16 [n_heads * 128]  rotated q                     */
#define W4_TRACE_ATTN 4   /* fp16 [n_heads * 128]  attention output              */
#define W4_TRACE_O 5      /* fp32 [hidden]   o_proj output                       */
#define W4_TRACE_H_MID 6  /* fp32 [hidden]   residual stream after attention     */
#define W4_TRACE_X2 7     /* fp16 [hidden]   MLP-norm output                     */
#define W4_TRACE_M 8      /* fp16 [inter]    silu(gate) * up                     */
#define W4_TRACE_D 9      /* fp32 [hidden]   down output                         */
#define W4_TRACE_FIELDS 10

/* Trace layout for a descriptor's dimensions (only the dimension fields are
 * read).  Host only. */
w4_status w4_decode_step_trace_layout(const w4_step_desc* desc, size_t* offsets, size_t* layer_stride,
                                      size_t* total_bytes);

typedef struct w4_step w4_step;

/*
 * Build one full decode step of the decoder read above, for batch 1:
 *     h = embed[token]
 *     per layer: x = rmsnorm(h) attn_norm;  qkv = x Wqkv (+ bias);
 *                rope + append k, v at pos;  a = attention over pos + 1 tokens;
 *                h += a Wo;  x = rmsnorm(h) mlp_norm;
 *                h += (silu(x Wgate) * (x Wup)) Wdown
 *     x = rmsnorm(h) final_norm;  logits = x Wlm;  token = argmax(logits);
 *     pos += 1
 * with the library's kernels: the embedding lookup fused with the first
 * norm; w4_gemv, w4_gemv_gateup_silu and w4_add_rmsnorm (the residual add
 * fused into the norm after o_proj, and into the final norm); from layer 1 on,
 * while hidden <= 4096, the attention norm folded into the qkv projection
 * (w4_gemv_residual for the down projection before it, w4_gemv_rmsnorm for
 * qkv), otherwise w4_add_rmsnorm there too; and w4_attn_decode with the
 * rotary embedding and KV append fused into its first kernel (q and the new
 * token's k, v taken from the fp32 QKV output, cos/sin from a per-position
 * table built at create).  Attention scale 1/sqrt(128).  Because
 * token and pos are read and advanced on the device, one call of
 * w4_decode_step per token continues the greedy decode with no host work;
 * use_graph != 0 captures the whole step as one HIP graph (one submission per
 * token, the pages' "CUDA Graph Optimization" bullet), use_graph == 0 keeps
 * eager launches for the comparison.  The handle allocates its activation
 * buffers, workspaces and the rotary table (device, at create: about 3 MB
 * for the 7B shapes at max_ctx 4096) and frees them at destroy; every pointer in the descriptor is baked in and
 * must stay valid until destroy.  pos must stay below max_ctx (at max_ctx - 1
 * the last cache slot is overwritten).  The handle is not thread-safe.
 * Rules: shapes as for the individual calls; hidden, n_heads * 128, inter
 * multiples of G; attn_norm 16-byte, mlp_norm and final_norm 8-byte aligned;
 * W4_ESHAPE / W4_EINVAL / W4_EALIGN before anything is allocated or launched.
 */
w4_status w4_decode_step_create(const w4_step_desc* desc, int32_t use_graph, w4_step** out);

/* Run one token's step on `stream` (graph launch or eager launches). */
w4_status w4_decode_step(w4_step* step, void* stream);

/* Operations one step submits (kernels, plus the trace copies when traced):
 * the graph's node count. */
w4_status w4_decode_step_launches(const w4_step* step, int32_t* count);

/* Release the handle and its buffers (NULL is accepted). */
w4_status w4_decode_step_destroy(w4_step* step);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
