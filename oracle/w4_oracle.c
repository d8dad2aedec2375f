/*
 * CPU oracle for the INT4 weight-only decode GEMV and its prefill GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; it is written from the definitions below and from the packed
 * layout specification (the "W4T4" layout, restated in the comments of
 * oracle_pack / oracle_unpack).
 *
 * What it computes.  The pages ("How To Build Your Own LLM Runtime From
 * Scratch", aitrending.vip, section "Technical Details", first bullet; and
 * noticiai.com.br, section "As tres licoes", third lesson) describe a decode
 * runtime whose weights are stored as INT4 and dequantized at run time while
 * activations stay in floating point.  The pages fix neither the zero point nor
 * the scale format; the reading used here (zero point 8, one fp16 scale per row
 * and per group of G consecutive inputs) is the one the workload definition
 * gives:
 *
 *     w[n][k] = (q[n][k] - 8) * s[n][floor(k / G)]          q in {0..15}
 *     y[n]    = sum_k w[n][k] * x[k]                        (plain GEMV)
 *     A[n]    = sum_k |w[n][k] * x[k]|                      (tolerance scale)
 *
 * Every dequantized weight is exact in double (a 4-bit integer times an
 * 11-bit significand), every product w*x is exact in double (at most 26
 * significant bits), and the sums are accumulated in double in increasing k,
 * so y is the exact dot product up to the rounding of a plain fp64 sum.
 *
 * Decode attention over a paged KV cache: see oracle_attn_decode.
 *
 * Prefill (a block of m prompt tokens through the same layers):
 *     Y[m][n] = sum_k X[m][k] * w[n][k]                     (one y per token)
 *
 * Fused epilogues:
 *     gate/up:  g = y[0..I), u = y[I..2I), h[j] = silu(g[j]) * u[j],
 *               silu(t) = t / (1 + exp(-t)) evaluated in double;
 *     lm_head:  argmax = lowest index of the largest y.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* IEEE 754 binary16 -> double, from the format definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes
 * subnormals (fraction * 2^-24), exponent 31 encodes inf / NaN. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -v : v;
}

/* ---------------------------------------------------------------------------
 * Packed layout "W4T4" (tile of 4 rows), restated for the oracle.
 *
 *  - Rows are grouped into tiles of 4.  Plain layout: tile t holds logical
 *    rows 4t..4t+3; there are ceil(N/4) tiles.  Gate/up layout (N = 2I): the
 *    gate half [0, I) and the up half [I, 2I) are tiled separately, gate tiles
 *    first, so tile t < ceil(I/4) holds rows 4t.., and tile ceil(I/4)+t holds
 *    rows I+4t..; each half has ceil(I/4) tiles.
 *  - Tile slots that hold no logical row are padding: nibble 8, scale +0.0.
 *  - Weights: tile t, block j (inputs 8j..8j+7) occupies 16 bytes at byte
 *    offset (t * (K/8) + j) * 16.  Bytes 4r..4r+3 of those 16, read as a
 *    little-endian 32-bit word, hold the 8 nibbles of tile row r.
 *  - Inside that word, nibble slot p sits at bits [4p, 4p+4).  The input
 *    offset e = k - 8j held by slot p is e = 2p for p < 4 and e = 2(p-4)+1
 *    for p >= 4 (so slots 0,4 hold inputs 0,1; slots 1,5 hold 2,3; slots 2,6
 *    hold 4,5; slots 3,7 hold 6,7).
 *  - Scales: tile t, group g occupies 8 bytes at byte offset
 *    (t * (K/G) + g) * 8; the fp16 at bytes 2r, 2r+1 is row r's scale.
 * ------------------------------------------------------------------------ */

/* number of tiles and the tile/slot of a logical row */
static int64_t tiles_of(int64_t n, int32_t gateup)
{
    if (gateup) {
        int64_t half = n / 2;
        return 2 * ((half + 3) / 4);
    }
    return (n + 3) / 4;
}

static void place_row(int64_t row, int64_t n, int32_t gateup, int64_t* tile, int* r)
{
    if (gateup) {
        int64_t half = n / 2;
        int64_t per_half = (half + 3) / 4;
        if (row < half) {
            *tile = row / 4;
            *r = (int)(row % 4);
        } else {
            *tile = per_half + (row - half) / 4;
            *r = (int)((row - half) % 4);
        }
    } else {
        *tile = row / 4;
        *r = (int)(row % 4);
    }
}

/* slot that holds input offset e (0..7) of a block */
static int slot_of_offset(int e)
{
    return (e % 2 == 0) ? e / 2 : 4 + e / 2;
}

int64_t oracle_packed_weight_bytes(int64_t n, int64_t k, int32_t gateup)
{
    return tiles_of(n, gateup) * (k / 8) * 16;
}

int64_t oracle_packed_scale_bytes(int64_t n, int64_t k, int32_t group, int32_t gateup)
{
    return tiles_of(n, gateup) * (k / group) * 8;
}

/* Logical (q, s) -> packed (pw, ps).  q is uint8 [n][k], s is fp16 bits
 * [n][k/group].  Returns 0 on success, -1 on a shape the layout cannot hold. */
int oracle_pack(const uint8_t* q, const uint16_t* s, int64_t n, int64_t k, int32_t group,
                int32_t gateup, uint8_t* pw, uint8_t* ps)
{
    if (n <= 0 || k <= 0 || group <= 0 || k % group != 0 || group % 8 != 0) return -1;
    if (gateup && n % 2 != 0) return -1;
    int64_t ntiles = tiles_of(n, gateup);
    int64_t nblocks = k / 8;
    int64_t ngroups = k / group;
    /* padding first: every nibble 8, every scale +0.0 */
    memset(pw, 0x88, (size_t)(ntiles * nblocks * 16));
    memset(ps, 0x00, (size_t)(ntiles * ngroups * 8));
    for (int64_t row = 0; row < n; ++row) {
        int64_t t;
        int r;
        place_row(row, n, gateup, &t, &r);
        for (int64_t j = 0; j < nblocks; ++j) {
            uint32_t word = 0;
            for (int e = 0; e < 8; ++e) {
                uint32_t nib = q[row * k + 8 * j + e] & 0xfu;
                word |= nib << (4 * slot_of_offset(e));
            }
            uint8_t* dst = pw + (t * nblocks + j) * 16 + 4 * r;
            dst[0] = (uint8_t)(word & 0xff);
            dst[1] = (uint8_t)((word >> 8) & 0xff);
            dst[2] = (uint8_t)((word >> 16) & 0xff);
            dst[3] = (uint8_t)((word >> 24) & 0xff);
        }
        for (int64_t g = 0; g < ngroups; ++g) {
            uint16_t v = s[row * ngroups + g];
            uint8_t* dst = ps + (t * ngroups + g) * 8 + 2 * r;
            dst[0] = (uint8_t)(v & 0xff);
            dst[1] = (uint8_t)(v >> 8);
        }
    }
    return 0;
}

/* Packed (pw, ps) -> logical (q, s); the inverse of oracle_pack on the
 * logical rows (padding slots are not read). */
int oracle_unpack(const uint8_t* pw, const uint8_t* ps, int64_t n, int64_t k, int32_t group,
                  int32_t gateup, uint8_t* q, uint16_t* s)
{
    if (n <= 0 || k <= 0 || group <= 0 || k % group != 0 || group % 8 != 0) return -1;
    if (gateup && n % 2 != 0) return -1;
    int64_t nblocks = k / 8;
    int64_t ngroups = k / group;
    for (int64_t row = 0; row < n; ++row) {
        int64_t t;
        int r;
        place_row(row, n, gateup, &t, &r);
        for (int64_t j = 0; j < nblocks; ++j) {
            const uint8_t* src = pw + (t * nblocks + j) * 16 + 4 * r;
            uint32_t word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) |
                            ((uint32_t)src[2] << 16) | ((uint32_t)src[3] << 24);
            for (int e = 0; e < 8; ++e)
                q[row * k + 8 * j + e] = (uint8_t)((word >> (4 * slot_of_offset(e))) & 0xfu);
        }
        for (int64_t g = 0; g < ngroups; ++g) {
            const uint8_t* src = ps + (t * ngroups + g) * 8 + 2 * r;
            s[row * ngroups + g] = (uint16_t)(src[0] | (src[1] << 8));
        }
    }
    return 0;
}

/* Reference dot products for the listed rows (rows == NULL: all n rows, in
 * order).  y[i] and a[i] receive y and A of row rows[i]. */
void oracle_gemv_rows(const uint8_t* q, const uint16_t* s, const uint16_t* x, int64_t n, int64_t k,
                      int32_t group, const int64_t* rows, int64_t nrows, double* y, double* a)
{
    int64_t ngroups = k / group;
    (void)n;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        double acc = 0.0, mag = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double w = ((double)q[row * k + kk] - 8.0) *
                       oracle_half_to_double(s[row * ngroups + kk / group]);
            double p = w * oracle_half_to_double(x[kk]);
            acc += p;
            mag += fabs(p);
        }
        y[i] = acc;
        a[i] = mag;
    }
}

void oracle_gemv(const uint8_t* q, const uint16_t* s, const uint16_t* x, int64_t n, int64_t k,
                 int32_t group, double* y, double* a)
{
    oracle_gemv_rows(q, s, x, n, k, group, NULL, n, y, a);
}

/* Same dot products, read straight from the packed buffers (each weight is
 * located with the layout rules above).  Used where the inputs are generated
 * already packed. */
void oracle_gemv_packed_rows(const uint8_t* pw, const uint8_t* ps, const uint16_t* x, int64_t n,
                             int64_t k, int32_t group, int32_t gateup, const int64_t* rows,
                             int64_t nrows, double* y, double* a)
{
    int64_t nblocks = k / 8;
    int64_t ngroups = k / group;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        int64_t t;
        int r;
        place_row(row, n, gateup, &t, &r);
        double acc = 0.0, mag = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            int64_t j = kk / 8;
            int e = (int)(kk % 8);
            const uint8_t* src = pw + (t * nblocks + j) * 16 + 4 * r;
            uint32_t word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) |
                            ((uint32_t)src[2] << 16) | ((uint32_t)src[3] << 24);
            int qv = (int)((word >> (4 * slot_of_offset(e))) & 0xfu);
            const uint8_t* sp = ps + (t * ngroups + kk / group) * 8 + 2 * r;
            double sv = oracle_half_to_double((uint16_t)(sp[0] | (sp[1] << 8)));
            double p = ((double)qv - 8.0) * sv * oracle_half_to_double(x[kk]);
            acc += p;
            mag += fabs(p);
        }
        y[i] = acc;
        a[i] = mag;
    }
}

/* Prefill product over a block of tokens (the 512-token prompt whose
 * first-token latency the pages report: "How To Build Your Own LLM Runtime
 * From Scratch", aitrending.vip, "Technical Details", performance-metrics
 * bullet; brifing.si section 6).  The prompt's tokens go through the same
 * INT4 linear layers, so each token row is the GEMV above: X holds m_total
 * fp16 rows of k inputs (row-major) and Y[m][n] = sum_k X[m][k] * w[n][k].
 * Logical inputs; y and a are [m_total][n]. */
void oracle_gemm(const uint8_t* q, const uint16_t* s, const uint16_t* xm, int64_t m_total, int64_t n,
                 int64_t k, int32_t group, double* y, double* a)
{
    for (int64_t m = 0; m < m_total; ++m)
        oracle_gemv_rows(q, s, xm + m * k, n, k, group, NULL, n, y + m * n, a + m * n);
}

/* The same product read from the packed buffers, for the listed token rows
 * and weight rows: y[i][j] and a[i][j] belong to token mrows[i] and weight
 * row ncols[j] (ncols == NULL: all n weight rows, nn == n). */
void oracle_gemm_packed(const uint8_t* pw, const uint8_t* ps, const uint16_t* xm, int64_t n, int64_t k,
                        int32_t group, int32_t gateup, const int64_t* mrows, int64_t nm,
                        const int64_t* ncols, int64_t nn, double* y, double* a)
{
    for (int64_t i = 0; i < nm; ++i) {
        int64_t m = mrows[i];
        oracle_gemv_packed_rows(pw, ps, xm + m * k, n, k, group, gateup, ncols, nn, y + i * nn, a + i * nn);
    }
}

/* Decode attention over a paged KV cache (the step between the QKV and
 * o_proj projections: "How To Build Your Own LLM Runtime From Scratch",
 * aitrending.vip, "Technical Details", architecture bullet -- paged KV cache
 * and attention; noticiai.com.br, "As tres licoes", lesson 1 -- the softmax
 * runs across KV pages and must stay correct at a page's tail).  Plain
 * scaled dot-product attention of one new token, with grouped KV heads:
 *
 *   g(h)     = h / (n_heads / n_kv)                  KV head of query head h
 *   s[h][t]  = scale * sum_d q[h][d] * K[t][g(h)][d]   for t < ctx
 *   p[h][t]  = exp(s[h][t] - max_t s[h][t]) / sum_t exp(s[h][t] - max_t s[h][t])
 *   o[h][d]  = sum_t p[h][t] * V[t][g(h)][d]
 *   A[h][d]  = sum_t p[h][t] * |V[t][g(h)][d]|        (tolerance scale)
 *
 * Token t lives in physical page page_table[t / page] at slot t % page; a
 * cache is fp16 [num_pages][n_kv][page][dim].  q is fp16 [n_heads][dim].
 * Everything in double. */
void oracle_attn_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* page_table,
                        int32_t ctx, int32_t n_heads, int32_t n_kv, int32_t dim, int32_t page, double scale,
                        double* o, double* a)
{
    int32_t group = n_heads / n_kv;
    for (int32_t h = 0; h < n_heads; ++h) {
        int32_t g = h / group;
        double mx = -HUGE_VAL;
        for (int32_t t = 0; t < ctx; ++t) {
            int64_t base = (((int64_t)page_table[t / page] * n_kv + g) * page + t % page) * dim;
            double sdot = 0.0;
            for (int32_t d = 0; d < dim; ++d)
                sdot += oracle_half_to_double(q[(int64_t)h * dim + d]) * oracle_half_to_double(kc[base + d]);
            sdot *= scale;
            if (sdot > mx) mx = sdot;
        }
        double den = 0.0;
        for (int32_t d = 0; d < dim; ++d) {
            o[(int64_t)h * dim + d] = 0.0;
            a[(int64_t)h * dim + d] = 0.0;
        }
        for (int32_t t = 0; t < ctx; ++t) {
            int64_t base = (((int64_t)page_table[t / page] * n_kv + g) * page + t % page) * dim;
            double sdot = 0.0;
            for (int32_t d = 0; d < dim; ++d)
                sdot += oracle_half_to_double(q[(int64_t)h * dim + d]) * oracle_half_to_double(kc[base + d]);
            double w = exp(sdot * scale - mx);
            den += w;
            for (int32_t d = 0; d < dim; ++d) {
                double v = oracle_half_to_double(vc[base + d]);
                o[(int64_t)h * dim + d] += w * v;
                a[(int64_t)h * dim + d] += w * fabs(v);
            }
        }
        for (int32_t d = 0; d < dim; ++d) {
            o[(int64_t)h * dim + d] /= den;
            a[(int64_t)h * dim + d] /= den;
        }
    }
}

/* Glue of a full decode step (the decoding stack of the pages' runtime --
 * "How To Build Your Own LLM Runtime From Scratch", aitrending.vip, TL;DR
 * and "Technical Details"; noticiai.com.br: attention, linear projections,
 * softmax, sampling -- read as the Qwen2-family pre-norm decoder the pages
 * name: RMSNorm, rotary position embedding, residual adds).  Double
 * precision throughout. */

/* out[i] = h[i] / sqrt(mean_j h[j]^2 + eps) * gamma[i]   (gamma fp16 bits) */
void oracle_rmsnorm(const double* h, int64_t n, const uint16_t* gamma, double eps, double* out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += h[i] * h[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) out[i] = h[i] * r * oracle_half_to_double(gamma[i]);
}

/* The same normalization with the sum of squares supplied by the caller: the
 * mean of h^2 is a sum divided by n, and that sum may have been accumulated
 * in parts (for instance per block of rows of the projection that produced h).
 *   out[i] = h[i] / sqrt(sumsq / n + eps) * gamma[i] */
void oracle_rmsnorm_given(const double* h, int64_t n, const uint16_t* gamma, double sumsq, double eps,
                          double* out)
{
    double r = 1.0 / sqrt(sumsq / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) out[i] = h[i] * r * oracle_half_to_double(gamma[i]);
}

/* Sum of squares of h in consecutive blocks of `rows` values:
 *   out[u] = sum of h[i]^2 for u * rows <= i < min(n, (u + 1) * rows) */
void oracle_sumsq_blocks(const double* h, int64_t n, int64_t rows, double* out)
{
    int64_t parts = (n + rows - 1) / rows;
    for (int64_t u = 0; u < parts; ++u) {
        double t = 0.0;
        for (int64_t i = u * rows; i < n && i < (u + 1) * rows; ++i) t += h[i] * h[i];
        out[u] = t;
    }
}

/* Rotary embedding of one head of `dim` values at position pos, rotating the
 * pairs (i, i + dim/2) by pos * theta^(-2i/dim):
 *   out[i]         = x[i] cos a - x[i + dim/2] sin a
 *   out[i + dim/2] = x[i + dim/2] cos a + x[i] sin a */
void oracle_rope(const double* x, int32_t dim, int64_t pos, double theta, double* out)
{
    int32_t half = dim / 2;
    for (int32_t i = 0; i < half; ++i) {
        double a = (double)pos * pow(theta, -2.0 * (double)i / (double)dim);
        double c = cos(a), sn = sin(a);
        out[i] = x[i] * c - x[i + half] * sn;
        out[i + half] = x[i + half] * c + x[i] * sn;
    }
}

/* silu(t) = t * sigmoid(t) = t / (1 + e^-t) */
double oracle_silu(double t)
{
    return t / (1.0 + exp(-t));
}

/* h[j] = silu(g[j]) * u[j] with g = y[0..half), u = y[half..2 half) */
void oracle_silu_gate(const double* y, int64_t half, double* h)
{
    for (int64_t j = 0; j < half; ++j) h[j] = oracle_silu(y[j]) * y[half + j];
}

/* lowest index of the maximum; NaN entries never win; -1 if none */
int64_t oracle_argmax(const double* y, int64_t n)
{
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (y[i] != y[i]) continue;
        if (best < 0 || y[i] > y[best]) best = i;
    }
    return best;
}

/* ------------------------------------------------------------------ W4A8
 * The INT8-activation variant the pages' runtime built and then removed
 * ("Tutorial: como construir seu proprio runtime de LLM do zero",
 * noticiai.com.br, "As tres licoes", lesson 3; "How To Build Your Own LLM
 * Runtime From Scratch", aitrending.vip, "Technical Details", low-level
 * pitfalls bullet).  The pages give no quantization rule; the reading is a
 * symmetric int8 code per activation with one fp32 scale per group of G
 * consecutive inputs (the weights' G), every step in binary32 with
 * round-to-nearest-even:
 *
 *     amax_g  = max_{k in g} |x[k]|
 *     inv_g   = 127 / amax_g            (binary32 division)
 *     c[k]    = clamp(rint(x[k] * inv_g), -127, 127)   (binary32 product)
 *     s_g     = amax_g / 127            (binary32 division)
 *     (amax_g == 0: c = 0 and s_g = 0)
 *
 * and the product uses the dequantized activation x^[k] = c[k] * s_g:
 *
 *     y[n] = sum_k (q[n][k] - 8) * s[n][g] * c[k] * s_g
 *
 * Each term is exact in double ((q - 8) c has at most 10 bits, s 11, s_g
 * 24), so y is the exact sum up to the rounding of a plain fp64 sum. */

/* codes (logical order) and per-group scales of an fp16 vector x[k] */
void oracle_quantize_act8(const uint16_t* x, int64_t k, int32_t group, int8_t* codes, float* scales)
{
    for (int64_t g = 0; g < k / group; ++g) {
        float amax = 0.0f;
        for (int64_t kk = g * group; kk < (g + 1) * group; ++kk) {
            float v = (float)fabs(oracle_half_to_double(x[kk]));
            if (v > amax) amax = v;
        }
        if (amax == 0.0f) {
            for (int64_t kk = g * group; kk < (g + 1) * group; ++kk) codes[kk] = 0;
            scales[g] = 0.0f;
            continue;
        }
        volatile float inv = 127.0f / amax;
        for (int64_t kk = g * group; kk < (g + 1) * group; ++kk) {
            volatile float prod = (float)oracle_half_to_double(x[kk]) * inv;
            float r = rintf(prod);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            codes[kk] = (int8_t)r;
        }
        volatile float sg = amax / 127.0f;
        scales[g] = sg;
    }
}

/* The W4T4 byte order of the codes: for each block of 8 inputs 8j..8j+7, the
 * bytes at 8j..8j+7 hold inputs 8j + (0, 4, 1, 5, 2, 6, 3, 7), which is the
 * order of the nibbles of a packed word taken as the bytes of
 * (word & 0x0F0F0F0F) followed by the bytes of ((word >> 4) & 0x0F0F0F0F). */
void oracle_act8_block_order(const int8_t* codes, int64_t k, int8_t* out)
{
    static const int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    for (int64_t j = 0; j < k / 8; ++j)
        for (int b = 0; b < 8; ++b) out[8 * j + b] = codes[8 * j + order[b]];
}

/* W4A8 dot products for the listed rows (rows == NULL: all), logical inputs,
 * codes in logical order. */
void oracle_gemv_a8_rows(const uint8_t* q, const uint16_t* s, const int8_t* codes, const float* act_scales,
                         int64_t n, int64_t k, int32_t group, const int64_t* rows, int64_t nrows, double* y,
                         double* a)
{
    int64_t ngroups = k / group;
    (void)n;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        double acc = 0.0, mag = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double w = ((double)q[row * k + kk] - 8.0) * oracle_half_to_double(s[row * ngroups + kk / group]);
            double p = w * ((double)codes[kk] * (double)act_scales[kk / group]);
            acc += p;
            mag += fabs(p);
        }
        y[i] = acc;
        a[i] = mag;
    }
}

/* The same from the packed weight buffers (W4T4 layout rules above). */
void oracle_gemv_a8_packed_rows(const uint8_t* pw, const uint8_t* ps, const int8_t* codes,
                                const float* act_scales, int64_t n, int64_t k, int32_t group, int32_t gateup,
                                const int64_t* rows, int64_t nrows, double* y, double* a)
{
    int64_t nblocks = k / 8;
    int64_t ngroups = k / group;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        int64_t t;
        int r;
        place_row(row, n, gateup, &t, &r);
        double acc = 0.0, mag = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            const uint8_t* src = pw + (t * nblocks + kk / 8) * 16 + 4 * r;
            uint32_t word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) |
                            ((uint32_t)src[2] << 16) | ((uint32_t)src[3] << 24);
            int qv = (int)((word >> (4 * slot_of_offset((int)(kk % 8)))) & 0xfu);
            const uint8_t* sp = ps + (t * ngroups + kk / group) * 8 + 2 * r;
            double sv = oracle_half_to_double((uint16_t)(sp[0] | (sp[1] << 8)));
            double p = ((double)qv - 8.0) * sv * ((double)codes[kk] * (double)act_scales[kk / group]);
            acc += p;
            mag += fabs(p);
        }
        y[i] = acc;
        a[i] = mag;
    }
}
