// Internal declarations shared by the host-side ABI code and the HIP kernels
// of the INT4 weight-only GEMV library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace w4i {

constexpr int kTileRows = 4;          // rows per packed tile (W4T4 layout)
constexpr int kBlockThreads = 256;    // 4 waves of 64 lanes
constexpr int kWavesPerBlock = kBlockThreads / 64;
constexpr int64_t kMaxK = 32768;      // bound on k (int32 block arithmetic)

enum Epilogue : int32_t {
    kEpiPlain = 0,   // y fp32
    kEpiArgmax = 1,  // y fp32 + lowest-index argmax
    kEpiGateUp = 2,  // h fp16 = silu(gate) * up
};

struct GemvCall {
    const void* pw;      // packed weights (device)
    const void* ps;      // packed scales (device)
    const void* x;       // fp16 [k] (device)
    void* out;           // fp32 [n] or fp16 [n/2] (device)
    int32_t* argmax;     // device, argmax epilogue only
    void* ws;            // device workspace, argmax epilogue only
    int64_t n;           // logical rows (gate/up: 2I)
    int64_t k;
    int32_t group;
    int32_t epi;
    const float* xs;     // W4A8: x holds int8 codes (W4T4 block order), xs the per-group scales; null: fp16 x
    // Residual epilogue (plain only; h_out non-null): h_out[i] = h_in[i] + y[i]
    // for i < n (h_in may equal h_out), and ss_out[u] = sum of h_out^2 over the
    // rows of unit u, for u < residual_parts(n, k, group).
    const float* h_in;
    float* h_out;
    float* ss_out;
    // RMSNorm prologue (norm_h non-null; x unused): the GEMV input is
    // x = fp16(h * r * gamma) with r = 1 / sqrt(S / k + eps) and S the sum of
    // norm_parts partial sums (<= kMaxNormParts, the buffer padded to a multiple
    // of 4 floats); workgroup 0 also writes that x to x_out when non-null.
    const float* norm_h;
    const uint16_t* norm_gamma;
    const float* norm_ss;
    int64_t norm_parts;
    float norm_eps;
    uint16_t* x_out;
};

// The norm prologue reads its partial sums with four 16-byte loads per lane.
constexpr int kNormPartLoads = 4;
constexpr int64_t kMaxNormParts = 64 * 4 * kNormPartLoads;

// Number of partial sums of squares the residual epilogue of a plain n x k
// GEMV writes (one per unit of its launch shape).
int64_t residual_parts(int64_t n, int64_t k, int32_t group);

// Per-group int8 quantization of fp16 x for the W4A8 GEMV (codes in W4T4
// block order, one fp32 scale per group).
hipError_t launch_act8_quantize(const uint16_t* x, int64_t k, int32_t group, int8_t* codes, float* scales,
                                hipStream_t stream);

// Prefill GEMM: y[m][n] = sum_k x[m][k] * w[n][k] for a block of token rows
// (x fp16 [m][k] row-major; y fp32 [m][n], or h fp16 [m][n/2] for gate/up).
struct GemmCall {
    const void* pw;
    const void* ps;
    const void* x;
    void* out;
    void* ws;            // split-k partials (plain only, when gemm_splits > 1)
    int64_t m;
    int64_t n;
    int64_t k;
    int32_t group;
    int32_t epi;         // kEpiPlain or kEpiGateUp
};

hipError_t launch_gemm(const GemmCall& call, hipStream_t stream);

// Output tile of the prefill GEMM: 128 x 128 when the block has at least
// 256 token rows or the 128-row tiles alone give two workgroups per CU of the
// 256; 64 x 128 otherwise.  A 128 x 128 tile reads 2/3 of the LDS bytes per
// flop of a 64 x 128 one (each wave multiplies 64 x 64 instead of 32 x 64).
// Gate/up tiles hold 64 gate rows and the matching 64 up rows.
struct GemmShape {
    int bm;
    int bn;
};

inline GemmShape choose_gemm_shape(int32_t epi, int64_t m, int64_t n)
{
    const int64_t cols = epi == kEpiGateUp ? n / 2 : n;
    const int64_t per_tile = epi == kEpiGateUp ? 64 : 128;
    const int64_t tiles128 = ((m + 127) / 128) * ((cols + per_tile - 1) / per_tile);
    return (m >= 256 || tiles128 >= 512) ? GemmShape{128, 128} : GemmShape{64, 128};
}

// Split-k factor: when the output tiles give fewer than 256 workgroups, the k
// range is split so the grid covers the chip in one round: for 128-row tiles
// (two workgroups per CU) as many splits as fit in 512 workgroups, for 64-row
// tiles enough to reach 256; at most 8 ways and at least one 64-input step per
// split.  The partials are summed in a fixed order by a second kernel.
// Gate/up is never split (its SiLU needs the full sums).
inline int32_t gemm_splits(int32_t epi, int64_t m, int64_t n, int64_t k)
{
    if (epi == kEpiGateUp) return 1;
    const GemmShape sh = choose_gemm_shape(epi, m, n);
    const int64_t wgs = ((n + sh.bn - 1) / sh.bn) * ((m + sh.bm - 1) / sh.bm);
    if (wgs >= 256) return 1;
    const int64_t steps = (k / 8 + 7) / 8;
    int64_t s = sh.bm == 128 ? 512 / wgs : (256 + wgs - 1) / wgs;
    if (s > 8) s = 8;
    if (s > steps) s = steps;
    return (int32_t)(s < 1 ? 1 : s);
}

inline size_t gemm_workspace_bytes(int32_t epi, int64_t m, int64_t n, int64_t k)
{
    const int32_t s = gemm_splits(epi, m, n, k);
    return s > 1 ? (size_t)s * (size_t)m * (size_t)n * 4 : 0;
}

// Decode attention over a paged KV cache (head dimension 128).
struct AttnCall {
    const void* q;            // fp16 [n_heads][128]
    const void* k_cache;      // fp16 [num_pages][n_kv][page_size][128]
    const void* v_cache;
    const int32_t* page_table;
    const int32_t* ctx_len;   // device int32, clamped to [1, max_ctx]
    uint16_t* out;            // fp16 [n_heads][128]
    void* ws;
    float scale;
    int32_t max_ctx;
    int32_t n_heads;
    int32_t n_kv;
    int32_t page_size;
    int32_t num_pages;
    // Non-null: rotary embedding + KV append fused into the attention (q,
    // k, v from rope->qkv at *rope->pos; q ignored, ctx_len = rope->ctx_out
    // is written with pos + 1).  The RopeCall's caches, page table and sizes
    // must match this call's.
    const struct RopeCall* rope;
};

constexpr int32_t kAttnHeadDim = 128;
constexpr int32_t kAttnMaxCtx = 1 << 20;

int64_t attn_chunks(int32_t max_ctx);
size_t attn_workspace_bytes(int32_t n_heads, int32_t max_ctx);
hipError_t launch_attn(const AttnCall& call, hipStream_t stream);

// Glue of a full decode step (head dimension 128).
struct RopeCall {
    const float* qkv;          // fp32 [(n_heads + 2 n_kv) * 128]: q heads, k heads, v heads
    const float* bias;         // fp32, same length, or null
    const int32_t* pos;        // device int32 [1], clamped to [0, max_ctx)
    uint16_t* q_out;           // fp16 [n_heads][128]
    uint16_t* k_cache;         // fp16 [num_pages][n_kv][page_size][128]
    uint16_t* v_cache;
    const int32_t* page_table;
    int32_t* ctx_out;          // device int32 [1] <- pos + 1 (or null)
    double theta;
    int32_t n_heads;
    int32_t n_kv;
    int32_t page_size;         // power of two
    int32_t num_pages;
    int32_t max_ctx;
    // (cos, sin) of every (position < max_ctx, pair i < 64), fp32, from
    // launch_rope_table; required by the fused attention, unused by
    // launch_rope_append
    const float2* table;
};

constexpr int64_t kMaxHidden = 1 << 20;

hipError_t launch_embed(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token, float* h,
                        hipStream_t stream);
// Embedding lookup fused with the first RMSNorm: h = table[token] (fp32),
// x = fp16(h * gamma / sqrt(mean(h^2) + eps)); one workgroup.
hipError_t launch_embed_rmsnorm(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* token,
                                const uint16_t* gamma, float eps, float* h, uint16_t* x, hipStream_t stream);
hipError_t launch_add_rmsnorm(float* h, const float* y, const uint16_t* gamma, int64_t n, float eps, uint16_t* x,
                              hipStream_t stream);
hipError_t launch_rope_append(const RopeCall& call, hipStream_t stream);
// table[p * 64 + i] = (cos, sin) of p * theta^(-2i/128) for p < max_ctx,
// evaluated in double and rounded to fp32 (the rotary kernels' arithmetic).
hipError_t launch_rope_table(double theta, int32_t max_ctx, float2* table, hipStream_t stream);

// Read-only bandwidth probe: streams `bytes` (a multiple of 16, 16-byte
// aligned) with 16-byte non-temporal loads; sink holds kProbeSinkWords words.
constexpr int kProbeSinkWords = 1024;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Size of the file-scope device array that backs the allocation-free argmax
// entry point (the per-workgroup partials of one call; 8 bytes per workgroup
// plus alignment, so up to 32736 workgroups, e.g. ~520K rows at k = 3584).
constexpr size_t kNoAllocScratchBytes = 256 * 1024;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t noalloc_scratch(void** ptr);

// Persistent sweep (one cooperative kernel for every projection of a sweep;
// eligible sweeps: k a multiple of 512 and at most kPMaxKb * 8, 64 <= G <= 512,
// at most kPStageWords input words per workgroup).
constexpr int kPMaxKb = 2560;          // k / 8 bound (k <= 20480)
constexpr int kPStageWords = 128;      // input words (2 fp16 each) a workgroup forwards
constexpr int kPMaxPhases = 256;       // projections per sweep (the phase table is kept in LDS)

struct PersistPhase {
    const uint4* pw;        // packed weights
    const uint2* ps;        // packed scales
    const uint16_t* x;      // the projection's input x (fp16 [k])
    void* out;              // y fp32 [n], or h fp16 [n/2] for gate/up
    float* part_v;          // argmax: per-workgroup best value [nwg]
    int32_t* part_i;        // argmax: per-workgroup best row [nwg]
    int64_t n;              // logical rows (gate/up: 2I)
    int64_t tiles;          // tiles in the packed matrix
    int64_t tiles_half;     // gate/up: tiles per half
    int32_t units;          // units (tiles, tile pairs, or gate/up tile pairs)
    int32_t kb;             // k / 8
    int32_t iters;          // k / 512
    int32_t ng;             // k / G
    int32_t gshift;         // log2(G / 8)
    int32_t epi;            // kEpiPlain / kEpiGateUp / kEpiArgmax
    int32_t utiles;         // tiles per unit (1 or 2)
    int32_t split;          // waves per unit (same as the one-kernel path's launch table)
    int32_t sc_dwords;      // scale dwords per 512-input chunk of a tile (2 * 512 / G)
    int32_t pad[5];         // 128 bytes (the kernel copies the table to LDS in 16-byte words)
};

struct PersistArgs {
    const PersistPhase* ph;     // device array [nph]
    int32_t nph;
    int32_t nwg;                // workgroups (one per CU)
    unsigned long long* hand;   // tagged input words [2][hand_words]
    int32_t hand_words;
    unsigned* ctrl;             // control block (kPersistCtrlBytes)
};

constexpr size_t kPersistCtrlBytes = 12 * 128;
constexpr size_t kPersistCtrlErrorOffset = 10 * 128;      // uint32: nonzero after a watchdog timeout
constexpr size_t kPersistCtrlWatchdogOffset = 11 * 128;   // uint64: wait limit in 100 MHz ticks
constexpr unsigned long long kPersistTicksPerSecond = 100000000ull;   // s_memrealtime rate

const void* persist_kernel_fn();
int persist_threads();
// the launch sequence of one token: the advance kernel, then the cooperative
// persistent kernel (the argmax finalize kernels are launched by the caller)
hipError_t launch_persist(const PersistArgs& args, hipStream_t stream);
// lowest-index maximum over `count` per-workgroup (value, row) partials into
// out[0]; a non-null advance_pos is incremented once the token is written
hipError_t launch_argmax_finalize(const float* part_v, const int32_t* part_i, int32_t count, int32_t* out,
                                  hipStream_t stream, int32_t* advance_pos = nullptr);

// Launch one GEMV on `stream` (shape already validated by the caller); the
// argmax epilogue adds a one-workgroup finalize kernel on the same stream,
// which also advances `advance_pos` when it is not null.
hipError_t launch_gemv(const GemvCall& call, hipStream_t stream, int32_t* advance_pos = nullptr);

// Workgroups of the main kernel for this call (only n, k, group, epi used).
int64_t launch_grid(const GemvCall& call);

// Launch shape: a unit is TILES tiles (1 or 2) processed together by SPLIT
// waves (k split inside the workgroup), each loading DEPTH k iterations per
// round before computing.  Chosen from measurements on MI355X at the
// decode-step shapes: enough waves to cover 256 CUs (split-k for the
// projections with few rows or long k), one load round per wave where
// registers allow, and two tiles per unit for very tall matrices (lm_head),
// which halves the number of workgroups to dispatch.
struct LaunchConfig {
    int tiles;
    int split;
    int depth;
};

inline LaunchConfig choose_config(int32_t epi, int64_t tiles, int32_t iters)
{
    int per_unit = epi == kEpiGateUp ? 2 : 1;
    int split;
    if (epi == kEpiGateUp) {
        split = 2;
    } else if (tiles >= 16384) {
        split = 2;
        per_unit = 2;
    } else if (iters > 8) {
        split = 8;
    } else {
        split = 4;
    }
    while (split > 1 && split > iters) split >>= 1;
    const int per_wave = (iters + split - 1) / split;
    int depth;
    if (per_wave <= 2)
        depth = 2;
    else if (split == 8)
        depth = per_wave <= 5 ? 5 : 8;
    else
        depth = per_wave <= 4 ? 4 : 8;
    return LaunchConfig{per_unit, split, depth};
}

// Argmax workspace: per-workgroup best values (fp32), then, from a 256-byte
// aligned offset, the matching rows (int32).
inline size_t argmax_index_offset(int64_t grid)
{
    return ((size_t)grid * 4 + 255) & ~(size_t)255;
}

inline size_t argmax_workspace_bytes(int64_t grid)
{
    return argmax_index_offset(grid) + (size_t)grid * 4;
}

// Number of W4T4 tiles of an n-row matrix in the given epilogue's layout.
inline int64_t tiles_for(int64_t n, bool gateup)
{
    if (gateup) return 2 * ((n / 2 + kTileRows - 1) / kTileRows);
    return (n + kTileRows - 1) / kTileRows;
}

}  // namespace w4i
