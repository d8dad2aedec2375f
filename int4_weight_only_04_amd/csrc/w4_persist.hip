// Persistent decode sweep: all projections of one token's linear sweep in one
// cooperative kernel, one workgroup per CU.
//
// What is computed is exactly what the graph-captured sweep computes (the same
// GEMVs, in the same decode order, with the same per-lane arithmetic and the
// same reduction order, so every output agrees with it bit for bit): per
// projection y = W x (fp32), h = silu(g) * u (fp16) for gate/up, and the
// lm_head logits with the per-workgroup partials of the argmax.  The pages
// attribute their per-token gain to issuing the whole decode step as one
// submission ("How To Build Your Own LLM Runtime From Scratch", "Technical
// Details", CUDA Graph bullet); on MI355X the cost left after graph capture is
// the kernel boundary between dependent projections (about 1.4 us of idle HBM
// plus the next kernel's first load latency, 113 times per token).  This
// kernel tries to keep HBM busy across those boundaries.  Measured on MI355X
// it is slower than the graph-captured sweep (the dependent hand-off reads
// queue behind the prefetched weights, and one workgroup per CU hides less
// latency than the many small workgroups of the one-kernel path), so it is an
// alternative mode, not the default.  Its parts:
//
//   * Projection p + 1's weights do not depend on projection p's output, only
//     its input does.  Each consumer wave walks its share of every projection,
//     in decode order, with two cursors: a load cursor that keeps the next
//     kPDepth 1 KiB weight chunks (and their scales) in flight in registers,
//     and a compute cursor.  At the end of a projection the load cursor simply
//     runs on into the next one, so while the wave waits for the next input
//     its registers fill with the next projection's weights and HBM stays busy.
//     (Streaming through LDS with LDS-DMA loads was measured first: on gfx950
//     a wave's LDS accesses interleaved with its in-flight LDS-DMA loads cut
//     the stream to ~1 TB/s, while plain 16-byte loads keep ~6-7 TB/s.)
//   * The consumer waves do the GEMV arithmetic of the one-kernel-per-
//     projection path (same unit/split shape, same k order per lane, same
//     lane reduction, same cross-wave sum order), with x read from LDS.
//   * The dependency between projections: when a workgroup's consumers finish
//     projection p, its last consumer wave stores this workgroup's slice of
//     the next projection's input as tagged 8-byte words (two fp16 values and
//     a 32-bit tag naming launch and projection) and adds one to an arrival
//     counter.  Four poller waves of every workgroup wait until the eight
//     counters show every workgroup arrived, then read the whole input, check
//     each word's tag (re-reading any that is not there yet), and copy it into
//     LDS for the consumers.  So the input of projection p + 1 is data written
//     by other workgroups after they finished projection p, as in a real
//     decode step, and no input value is used before its producer finished.
//   * Every wait is bounded by a deadline (the 100 MHz real-time counter): a
//     wave that reaches it sets the workgroup's and the device's abort words
//     and an error code the host reads; every other wait then returns, and
//     the kernel ends normally with the error reported.
//   * No workgroup barrier is used after start-up (the pollers run their own
//     loop); waves meet through LDS words only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_gemv_math.h"
#include "w4_internal.h"

namespace w4i {
namespace {

using namespace gemv_math;

constexpr int kPCons = 8;                       // consumer waves
constexpr int kPPoll = 4;                       // poller waves
constexpr int kPThreads = (kPCons + kPPoll) * 64;
constexpr int kPDepth = 10;                     // weight chunks in flight per consumer wave
constexpr int kPWordsPerLane = 40;              // tagged words per poller lane (4 * 64 * 40 >= 10240)
constexpr int kPWordBatch = 20;                 // read in two batches of 20 loads

// control block (uint32 words; each counter in its own 128-byte line)
constexpr int kCtlEpoch = 8 * 32;
constexpr int kCtlAbort = 9 * 32;
constexpr int kCtlError = 10 * 32;
constexpr int kCtlTicks = 11 * 32;              // 64-bit deadline in 100 MHz ticks

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ unsigned ld_dev(const unsigned* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev64(const unsigned long long* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned* p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(unsigned long long* p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Pointers read from the phase table are generic to the compiler; these give
// their accesses the global address space (global_* instead of flat_*).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gp(T* p)
{
    return (__attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gp(const T* p)
{
    return (const __attribute__((address_space(1))) T*)p;
}

// Non-temporal 16- and 8-byte loads through global-address-space pointers (the
// weight and scale pointers come from the LDS copy of the phase table, which
// would otherwise make them flat loads, with their extra waits).
__device__ __forceinline__ uint4 ld_nt(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load(gp(reinterpret_cast<const u32x4_t*>(p)));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p)
{
    const u32x2_t v = __builtin_nontemporal_load(gp(reinterpret_cast<const u32x2_t*>(p)));
    return make_uint2(v.x, v.y);
}

// LDS words shared by the waves of one workgroup
// Every lane reads the same word in one instruction, so the value is uniform;
// saying so (readfirstlane) keeps the branches on it, and the cursor state
// updated under them, in scalar registers.
__device__ __forceinline__ unsigned ld_wg(const unsigned* p)
{
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void st_wg(unsigned* p, unsigned v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// tag of projection q's input words in the launch with this epoch
__device__ __forceinline__ unsigned input_tag(unsigned epoch, int q) { return epoch * 4096u + (unsigned)q + 1u; }

// (phase, round) stamp for the cross-wave sums; 0 means none
__device__ __forceinline__ unsigned stamp(int p, int r) { return ((unsigned)(p + 1) << 16) | (unsigned)r; }

// LDS words the waves of a workgroup meet through.
struct Ctl {
    unsigned stage[kPStageWords];                          // this workgroup's slice of the next input
    float red[2][kPCons][2][4];                            // cross-wave partial row sums
    float best_v[kPCons];
    int best_i[kPCons];
    unsigned posted[kPCons];                               // stamp of the last partial a wave posted
    unsigned summed[kPCons];                               // owner: stamp of the last sum it formed
    unsigned xready;                                       // poller completions (kPPoll per projection)
    unsigned cseen;                                        // projection whose arrivals poller 0 has seen
    unsigned fwd_ready;                                    // projection whose staged slice is in `stage`
    unsigned pdone;                                        // consumer-wave completions (kPCons per projection)
    unsigned abort;                                        // nonzero: stop
    unsigned epoch;
    unsigned long long ticks;
};

struct Shared {
    uint4* xbuf;                // [kPMaxKb] input x of the current projection (fp16)
    Ctl* c;
    const PersistPhase* ph;     // [nph] the phase table, copied to LDS at start
};

// Bounded wait helper: poll() returns true when the wait must be abandoned.
struct Watch {
    unsigned spin;
    unsigned long long deadline;
    unsigned* ctrl;
    Shared* sh;

    __device__ __forceinline__ bool stop()
    {
        if (ld_wg(&sh->c->abort)) return true;
        ++spin;
        if ((spin & 63) == 0) {
            if (now_ticks() > deadline) {
                st_wg(&sh->c->abort, 1u);
                st_dev(ctrl + kCtlAbort, 1u);
                st_dev(ctrl + kCtlError, 1u);
                return true;
            }
            if ((spin & 4095) == 0 && __builtin_amdgcn_readfirstlane(ld_dev(ctrl + kCtlAbort))) {
                st_wg(&sh->c->abort, 1u);
                return true;
            }
        }
        __builtin_amdgcn_s_sleep(1);
        return false;
    }
};

struct Range {
    int u0, u1;      // units of this workgroup
    int slots;       // units processed side by side (kPCons / split)
    int rounds;
    int cmax;        // k iterations per wave and unit, at most
};

__device__ __forceinline__ Range range_of(const PersistPhase& P, int b, int nwg)
{
    Range r;
    r.u0 = (int)((int64_t)P.units * b / nwg);
    r.u1 = (int)((int64_t)P.units * (b + 1) / nwg);
    r.slots = kPCons / P.split;
    r.rounds = (r.u1 - r.u0 + r.slots - 1) / r.slots;
    r.cmax = (P.iters + P.split - 1) / P.split;
    return r;
}

__device__ __forceinline__ int64_t tile_of(const PersistPhase& P, int unit, int t)
{
    return P.epi == kEpiGateUp ? (int64_t)unit + (int64_t)t * P.tiles_half : (int64_t)unit * P.utiles + t;
}

// ----------------------------------------------------------------- consumers

// Where this wave's share of projection p lies: units unit0, unit0 + ustep,
// ... < u1, k iterations [it0, it1) of each, utiles tiles per unit.
struct Share {
    int unit0, u1, ustep;
    int it0, it1;
    int sp, slot;
};

__device__ __forceinline__ Share share_of(const PersistPhase& P, int w, int b, int nwg)
{
    const int S = P.split;                 // 1, 2, 4 or 8
    const int lgS = __builtin_ctz(S);
    Share sh;
    sh.slot = w >> lgS;
    sh.sp = w & (S - 1);
    // units * (b + 1) < 2^32 (units < 2^23 is checked at create)
    sh.unit0 = (int)((unsigned)P.units * (unsigned)b / (unsigned)nwg) + sh.slot;
    sh.u1 = (int)((unsigned)P.units * (unsigned)(b + 1) / (unsigned)nwg);
    sh.ustep = kPCons >> lgS;
    sh.it0 = (sh.sp * P.iters) >> lgS;
    sh.it1 = ((sh.sp + 1) * P.iters) >> lgS;
    return sh;
}

// The load cursor: this wave's chunks over every projection, in the order the
// compute side consumes them: per unit, the k iterations of its first tile,
// then those of its second tile (gate/up, two-tile lm_head units).
struct LoadCur {
    int p;
    int unit, u1, ustep, it, it0, it1, t, U;
    bool ok1;
    int64_t tile0, tile1;
    const uint4* pw;
    const uint2* ps;
    int kb, ng, gshift;
    int64_t tiles, tiles_half;
    int epi, utiles;
    const uint4* dummy_w;   // chunk loaded past the last one (never used)
    const uint2* dummy_s;
};

__device__ __forceinline__ void lc_tiles(LoadCur& c)
{
    if (c.epi == kEpiGateUp) {
        c.tile0 = c.unit;
        c.tile1 = c.unit + c.tiles_half;
        c.ok1 = true;
    } else {
        c.tile0 = (int64_t)c.unit * c.utiles;
        c.tile1 = c.tile0 + 1;
        c.ok1 = c.utiles == 2 && c.tile1 < c.tiles;
    }
}

// position at the first chunk of projection >= c.p that has work for this wave
__device__ __forceinline__ void lc_seek(LoadCur& c, const PersistArgs& a, const Shared* sh, int w, int b)
{
    for (; c.p < a.nph; ++c.p) {
        const PersistPhase& P = sh->ph[c.p];
        const Share sh = share_of(P, w, b, a.nwg);
        if (sh.unit0 >= sh.u1 || sh.it0 >= sh.it1) continue;
        c.unit = sh.unit0;
        c.u1 = sh.u1;
        c.ustep = sh.ustep;
        c.it0 = sh.it0;
        c.it1 = sh.it1;
        c.it = sh.it0;
        c.t = 0;
        c.pw = P.pw;
        c.ps = P.ps;
        c.kb = P.kb;
        c.ng = P.ng;
        c.gshift = P.gshift;
        c.tiles = P.tiles;
        c.tiles_half = P.tiles_half;
        c.epi = P.epi;
        c.utiles = P.utiles;
        c.U = P.epi == kEpiGateUp ? 2 : P.utiles;
        lc_tiles(c);
        return;
    }
}

// the next chunk within the projection; false when the cursor must move on
// to the next projection (lc_seek)
__device__ __forceinline__ bool lc_next_fast(LoadCur& c, int nph)
{
    if (c.p >= nph) return true;
    if (++c.it < c.it1) return true;
    c.it = c.it0;
    if (c.t == 0 && c.U == 2 && c.ok1) {
        c.t = 1;
        return true;
    }
    c.t = 0;
    c.unit += c.ustep;
    if (c.unit < c.u1) {
        lc_tiles(c);
        return true;
    }
    return false;
}

__device__ __forceinline__ void lc_next(LoadCur& c, const PersistArgs& a, const Shared* sh, int w, int b)
{
    if (!lc_next_fast(c, a.nph)) {
        ++c.p;
        lc_seek(c, a, sh, w, b);
    }
}

// issue the loads of the cursor's chunk (past the last one: loads of the first
// chunk of projection 0, whose values are never used, so that every slot always
// holds exactly two loads and the waits below are fixed counts)
__device__ __forceinline__ void lc_issue(const LoadCur& c, const PersistArgs& a, int lane, uint4& wv, uint2& sv)
{
    if (c.p < a.nph) {
        const int64_t tile = c.t ? c.tile1 : c.tile0;
        const int j = c.it * 64 + lane;
        wv = ld_nt(c.pw + tile * c.kb + j);
        sv = ld_nt(c.ps + tile * c.ng + (j >> c.gshift));
    } else {
        wv = ld_nt(c.dummy_w + lane);
        sv = ld_nt(c.dummy_s);
    }
}

// The compute side of a consumer wave.
struct Comp {
    int p;                       // current projection (a.nph: finished)
    Share sh;
    int unit, it, t, r, U, epi;
    bool ok1;
    int64_t tile0, tile1;
    float acc[4];      // the tile being accumulated
    float acc0[4];     // a two-tile unit: the first tile's sums
    uint4 xv;
    float bv;
    int bi;
};

__device__ __forceinline__ void cs_tiles(Comp& c, const PersistPhase& P)
{
    if (c.epi == kEpiGateUp) {
        c.tile0 = c.unit;
        c.tile1 = c.unit + P.tiles_half;
        c.ok1 = true;
    } else {
        c.tile0 = (int64_t)c.unit * P.utiles;
        c.tile1 = c.tile0 + 1;
        c.ok1 = P.utiles == 2 && c.tile1 < P.tiles;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) c.acc[q] = 0.0f;
}

// The end of projection p for this wave: the argmax partial, the arrival, and
// for the workgroup's last wave the forward of the next input.  False on abort.
__device__ __forceinline__ bool finish_phase(const PersistArgs& a, const PersistPhase& P, int p, Comp& c, int w,
                                             int lane, int b, Shared* sh, Watch& wt)
{
    if (P.epi == kEpiArgmax) {
        // this wave's best over its rows (the 4 tile rows sit in the 4 16-lane rows)
        float bv = c.bv;
        int bi = c.bi;
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if (lane == 0) {
            sh->c->best_v[w] = bv;
            sh->c->best_i[w] = bi;
        }
    }
    unsigned prev = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    if (lane == 0) prev = __hip_atomic_fetch_add(&sh->c->pdone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(kPCons * (p + 1) - 1)) return true;
    // the last consumer wave of this workgroup to finish projection p
    if (P.epi == kEpiArgmax && lane == 0) {
        float v = sh->c->best_v[0];
        int i = sh->c->best_i[0];
        for (int q = 1; q < kPCons; ++q)
            if (better(sh->c->best_v[q], sh->c->best_i[q], v, i)) {
                v = sh->c->best_v[q];
                i = sh->c->best_i[q];
            }
        gp(P.part_v)[b] = v;
        gp(P.part_i)[b] = i;
    }
    const int q = p + 1;
    if (q >= a.nph) return true;
    while (ld_wg(&sh->c->fwd_ready) < (unsigned)q)
        if (wt.stop()) return false;
    const PersistPhase& Q = sh->ph[q];
    const int nw = Q.kb * 4;
    const int w0 = (int)((int64_t)nw * b / a.nwg);
    const int w1 = (int)((int64_t)nw * (b + 1) / a.nwg);
    const unsigned long long tg = (unsigned long long)input_tag(sh->c->epoch, q) << 32;
    unsigned long long* dst = a.hand + (size_t)(q & 1) * a.hand_words;
    for (int i = lane; i < w1 - w0; i += 64) st_dev64(dst + w0 + i, tg | sh->c->stage[i]);
    if (lane == 0) __hip_atomic_fetch_add(a.ctrl + (b & 7) * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Enter projection c.p or a later one that has work for this wave (waiting for
// each one's input; projections without work are finished at once).  False on
// abort; c.p == a.nph when every projection is done.
__device__ __forceinline__ bool cs_enter(const PersistArgs& a, Comp& c, int w, int lane, int b, Shared* sh,
                                         Watch& wt)
{
    for (; c.p < a.nph; ++c.p) {
        while (ld_wg(&sh->c->xready) < (unsigned)(kPPoll * (c.p + 1)))
            if (wt.stop()) return false;
        const PersistPhase& P = sh->ph[c.p];
        c.sh = share_of(P, w, b, a.nwg);
        c.bv = -__builtin_inff();
        c.bi = INT32_MAX;
        if (c.sh.unit0 < c.sh.u1 && c.sh.it0 < c.sh.it1) {
            c.epi = P.epi;
            c.U = P.epi == kEpiGateUp ? 2 : P.utiles;
            c.unit = c.sh.unit0;
            c.it = c.sh.it0;
            c.t = 0;
            c.r = 0;
            cs_tiles(c, P);
            c.xv = sh->xbuf[c.it * 64 + lane];
            return true;
        }
        if (!finish_phase(a, P, c.p, c, w, lane, b, sh, wt)) return false;
    }
    return true;
}

// The end of a unit: the wave's row sums, the cross-wave sum and the epilogue.
// False on abort.
__device__ __forceinline__ bool finish_unit(const PersistPhase& P, Comp& c, int w, int lane, Shared* sh, Watch& wt)
{
    const int S = P.split;
    const int owner_w = c.sh.slot * S;
    const bool writer = (lane & 15) == 0;
    const int row_in_tile = reduced_row(lane);
    // a two-tile unit whose second tile exists ended on that tile: its first
    // tile's sums were saved in acc0
    const bool two = c.U == 2 && c.ok1;
    float rv[2];
    rv[0] = two ? reduce4(c.acc0[0], c.acc0[1], c.acc0[2], c.acc0[3]) : reduce4(c.acc[0], c.acc[1], c.acc[2], c.acc[3]);
    rv[1] = two ? reduce4(c.acc[0], c.acc[1], c.acc[2], c.acc[3]) : 0.0f;
    if (S > 1) {
        const int par = c.r & 1;
        // the owner must have summed this buffer's previous round
        if (c.r >= 2) {
            while (ld_wg(&sh->c->summed[owner_w]) < stamp(c.p, c.r - 2))
                if (wt.stop()) return false;
        }
        if (writer) {
            sh->c->red[par][w][0][row_in_tile] = rv[0];
            sh->c->red[par][w][1][row_in_tile] = rv[1];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (lane == 0) st_wg(&sh->c->posted[w], stamp(c.p, c.r));
        if (c.sh.sp != 0) return true;
        for (int q = 1; q < S; ++q) {
            while (ld_wg(&sh->c->posted[owner_w + q]) < stamp(c.p, c.r))
                if (wt.stop()) return false;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float s = sh->c->red[par][owner_w][t][row_in_tile];
            for (int q = 1; q < S; ++q) s += sh->c->red[par][owner_w + q][t][row_in_tile];
            rv[t] = s;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (lane == 0) st_wg(&sh->c->summed[w], stamp(c.p, c.r));
    }
    // owner: the epilogue of this unit
    if (c.epi == kEpiGateUp) {
        const int64_t jr = (int64_t)c.unit * 4 + row_in_tile;
        if (writer && jr < (P.n >> 1)) {
            const float g = rv[0];
            const float silu = g / (1.0f + __expf(-g));
            const _Float16 hv = (_Float16)(silu * rv[1]);
            gp(reinterpret_cast<uint16_t*>(P.out))[jr] = __builtin_bit_cast(uint16_t, hv);
        }
    } else {
        const auto y = gp(reinterpret_cast<float*>(P.out));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t == 1 && !c.ok1) continue;
            const int64_t row = (t ? c.tile1 : c.tile0) * 4 + row_in_tile;
            if (row < P.n) {
                if (writer) y[row] = rv[t];
                if (c.epi == kEpiArgmax && better(rv[t], (int32_t)row, c.bv, c.bi)) {
                    c.bv = rv[t];
                    c.bi = (int32_t)row;
                }
            }
        }
    }
    return true;
}

// Advance the compute cursor past the chunk just done, within the unit;
// false when the unit has ended (cs_unit_end).
__device__ __forceinline__ bool cs_next_fast(Comp& c, int lane, Shared* sh)
{
    if (++c.it < c.sh.it1) {
        c.xv = sh->xbuf[c.it * 64 + lane];
        return true;
    }
    return false;
}

// The end of a unit: its sums and epilogue, then the next unit, or the end of
// the projection and the start of the next one.  False on abort.
__device__ __forceinline__ bool cs_unit_end(const PersistArgs& a, Comp& c, int w, int lane, int b, Shared* sh,
                                            Watch& wt)
{
    if (c.t == 0 && c.U == 2 && c.ok1) {
        // the first tile of a two-tile unit is done: keep its sums, start the second
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c.acc0[q] = c.acc[q];
            c.acc[q] = 0.0f;
        }
        c.t = 1;
        c.it = c.sh.it0;
        c.xv = sh->xbuf[c.it * 64 + lane];
        return true;
    }
    c.t = 0;
    const PersistPhase& P = sh->ph[c.p];
    if (!finish_unit(P, c, w, lane, sh, wt)) return false;
    ++c.r;
    c.unit += c.sh.ustep;
    if (c.unit < c.sh.u1) {
        c.it = c.sh.it0;
        cs_tiles(c, P);
        c.xv = sh->xbuf[c.it * 64 + lane];
        return true;
    }
    if (!finish_phase(a, P, c.p, c, w, lane, b, sh, wt)) return false;
    ++c.p;
    return cs_enter(a, c, w, lane, b, sh, wt);
}

// one chunk of the arithmetic: the same per-lane operations, in the same
// order, as the one-kernel-per-projection GEMV
__device__ __forceinline__ void cs_chunk(Comp& c, const uint4& wv, const uint2& sv, uint32_t magic)
{
    c.acc[0] = __builtin_fmaf(dot8(wv.x, c.xv, magic), half_lo(sv.x), c.acc[0]);
    c.acc[1] = __builtin_fmaf(dot8(wv.y, c.xv, magic), half_hi(sv.x), c.acc[1]);
    c.acc[2] = __builtin_fmaf(dot8(wv.z, c.xv, magic), half_lo(sv.y), c.acc[2]);
    c.acc[3] = __builtin_fmaf(dot8(wv.w, c.xv, magic), half_hi(sv.y), c.acc[3]);
}

// One chunk of the steady loop in register slot d (a compile-time index, so the
// ring stays in registers): wait for it, its arithmetic, the load of the chunk
// kPDepth ahead into the same registers, and the cursors' fast steps.  False
// when a cursor needs its slow step (a new projection or the end of a unit).
template <int d, int D>
__device__ __forceinline__ bool slot_fast(const PersistArgs& a, Comp& c, LoadCur& L, uint4 (&wr)[D], uint2 (&sr)[D],
                                          uint32_t magic, int lane, Shared* sh, bool& lseek)
{
    // the chunk in slot d was issued D chunks ago; 2 * (D - 1) loads are younger
    if constexpr (D == 12)
        asm volatile("s_waitcnt vmcnt(22)" ::: "memory");
    else if constexpr (D == 10)
        asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (D == 8)
        asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else
        static_assert(D == 12 || D == 10 || D == 8, "ring depth without a written-out wait");
    cs_chunk(c, wr[d], sr[d], magic);
    lc_issue(L, a, lane, wr[d], sr[d]);
    lseek = !lc_next_fast(L, a.nph);
    const bool cok = cs_next_fast(c, lane, sh);
    return cok && !lseek;
}

template <int D>
__device__ __forceinline__ void consumer(const PersistArgs& a, int w, int lane, int b, Shared* sh, Watch& wt)
{
    static_assert(D <= 12, "the slot switch is written out for at most 12 chunks in flight");
    const uint32_t magic = opaque_magic();
    uint4 wr[D];
    uint2 sr[D];
    LoadCur L{};
    L.p = 0;
    L.dummy_w = sh->ph[0].pw;
    L.dummy_s = sh->ph[0].ps;
    lc_seek(L, a, sh, w, b);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        lc_issue(L, a, lane, wr[d], sr[d]);
        lc_next(L, a, sh, w, b);
    }
    Comp c{};
    c.p = 0;
    if (!cs_enter(a, c, w, lane, b, sh, wt) || c.p >= a.nph) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    int d = 0;
    for (;;) {
        bool lseek = false;
        bool fast = true;
        // run slots d, d + 1, ... until one needs a slow step; continue after it
        switch (d) {
#define W4P_SLOT(k)                                                                     \
    case k:                                                                             \
        if constexpr (k < D) {                                                          \
            if (!slot_fast<(k < D ? k : 0), D>(a, c, L, wr, sr, magic, lane, sh, lseek)) { \
                d = (k + 1) % D;                                                        \
                fast = false;                                                           \
                break;                                                                  \
            }                                                                           \
        }                                                                               \
        [[fallthrough]];
            W4P_SLOT(0) W4P_SLOT(1) W4P_SLOT(2) W4P_SLOT(3) W4P_SLOT(4) W4P_SLOT(5)
            W4P_SLOT(6) W4P_SLOT(7) W4P_SLOT(8) W4P_SLOT(9) W4P_SLOT(10) W4P_SLOT(11)
#undef W4P_SLOT
            default:
                d = 0;
        }
        if (fast) continue;
        if (lseek) {
            ++L.p;
            lc_seek(L, a, sh, w, b);
        }
        if (c.it >= c.sh.it1) {
            if (!cs_unit_end(a, c, w, lane, b, sh, wt) || c.p >= a.nph) break;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ----------------------------------------------------------------- pollers

__device__ __forceinline__ void poller(const PersistArgs& a, int pw, int lane, int b, Shared* sh, Watch& wt)
{
    for (int p = 0; p < a.nph; ++p) {
        const PersistPhase& P = sh->ph[p];
        const int kb = P.kb;
        if (p == 0) {
            // the first projection's input comes straight from the caller's x
            const auto x = gp(reinterpret_cast<const u32x4_t*>(P.x));
            for (int blk = pw * 64 + lane; blk < kb; blk += kPPoll * 64) {
                const u32x4_t v = x[blk];
                sh->xbuf[blk] = make_uint4(v.x, v.y, v.z, v.w);
            }
        } else {
            if (pw == 0) {
                // The arrivals cannot be complete before this workgroup's own consumers
                // have finished the previous projection: wait for that in LDS first, so
                // the device-wide counters (eight cache lines every workgroup polls) are
                // only read for the short time the hand-off is actually pending.
                while (ld_wg(&sh->c->pdone) < (unsigned)(kPCons * p))
                    if (wt.stop()) return;
                // every workgroup of group c (b % 8 == c) adds one to counter c per projection
                const unsigned nc = (unsigned)((a.nwg - (lane & 7) + 7) / 8);
                const unsigned target = nc * (unsigned)p;
                for (;;) {
                    const unsigned v = lane < 8 ? ld_dev(a.ctrl + lane * 32) : target;
                    if (__all(v >= target)) break;
                    if (wt.stop()) return;
                }
                if (lane == 0) st_wg(&sh->c->cseen, (unsigned)p);
            } else {
                while (ld_wg(&sh->c->cseen) < (unsigned)p)
                    if (wt.stop()) return;
            }
            const int nw = kb * 4;
            const unsigned tg = input_tag(sh->c->epoch, p);
            const unsigned long long* src = a.hand + (size_t)(p & 1) * a.hand_words;
            unsigned* xw = reinterpret_cast<unsigned*>(sh->xbuf);
            for (int h = 0; h < kPWordsPerLane; h += kPWordBatch) {
                const int base = pw * 64 * kPWordsPerLane + h * 64 + lane;
                if (base - lane >= nw) break;
                unsigned long long v[kPWordBatch];
#pragma unroll
                for (int i = 0; i < kPWordBatch; ++i) {
                    const int wi = base + 64 * i;
                    v[i] = wi < nw ? ld_dev64(src + wi) : ((unsigned long long)tg << 32);
                }
#pragma unroll
                for (int i = 0; i < kPWordBatch; ++i) {
                    const int wi = base + 64 * i;
                    while ((unsigned)(v[i] >> 32) != tg) {
                        if (wt.stop()) return;
                        v[i] = ld_dev64(src + wi);
                    }
                    if (wi < nw) xw[wi] = (unsigned)v[i];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) __hip_atomic_fetch_add(&sh->c->xready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        // stage this workgroup's slice of the next projection's input
        if (pw == 0 && p + 1 < a.nph) {
            const PersistPhase& Q = sh->ph[p + 1];
            const int nw = Q.kb * 4;
            const int w0 = (int)((int64_t)nw * b / a.nwg);
            const int w1 = (int)((int64_t)nw * (b + 1) / a.nwg);
            const auto xq = gp(reinterpret_cast<const unsigned*>(Q.x));
            for (int i = lane; i < w1 - w0; i += 64) sh->c->stage[i] = xq[w0 + i];
            __builtin_amdgcn_s_waitcnt(0);
            if (lane == 0) __hip_atomic_store(&sh->c->fwd_ready, (unsigned)(p + 1), __ATOMIC_RELEASE,
                                              __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

__global__ void __launch_bounds__(kPThreads) persist_sweep_kernel(PersistArgs a)
{
    __shared__ uint4 xbuf[kPMaxKb];
    __shared__ Ctl ctl;
    __shared__ PersistPhase phs[kPMaxPhases];
    Shared sh{xbuf, &ctl, phs};
    static_assert(sizeof(PersistPhase) % 16 == 0, "the phase table is copied in 16-byte words");
    {
        const uint4* src = reinterpret_cast<const uint4*>(a.ph);
        uint4* dst = reinterpret_cast<uint4*>(phs);
        const int words = a.nph * (int)(sizeof(PersistPhase) / 16);
        for (int i = threadIdx.x; i < words; i += kPThreads) dst[i] = src[i];
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.x;
    if (threadIdx.x < kPCons) {
        ctl.posted[threadIdx.x] = 0;
        ctl.summed[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0) {
        ctl.xready = 0;
        ctl.cseen = 0;
        ctl.fwd_ready = 0;
        ctl.pdone = 0;
        ctl.abort = 0;
        ctl.epoch = ld_dev(a.ctrl + kCtlEpoch);
        ctl.ticks = ld_dev64(reinterpret_cast<const unsigned long long*>(a.ctrl + kCtlTicks));
    }
    __syncthreads();
    Watch wt{0u, now_ticks() + ctl.ticks, a.ctrl, &sh};
    if (wave < kPCons)
        consumer<kPDepth>(a, wave, lane, b, &sh, wt);
    else
        poller(a, wave - kPCons, lane, b, &sh, wt);
}

// One thread: start a new launch (new tag epoch, arrival counters at zero,
// abort word clear).  Runs before the persistent kernel on the same stream.
__global__ void persist_advance_kernel(unsigned* ctrl)
{
    if (threadIdx.x != 0) return;
    st_dev(ctrl + kCtlEpoch, ld_dev(ctrl + kCtlEpoch) + 1u);
    for (int c = 0; c < 8; ++c) st_dev(ctrl + c * 32, 0u);
    st_dev(ctrl + kCtlAbort, 0u);
}

}  // namespace

const void* persist_kernel_fn()
{
    return reinterpret_cast<const void*>(&persist_sweep_kernel);
}

int persist_threads()
{
    return kPThreads;
}

hipError_t launch_persist(const PersistArgs& args, hipStream_t stream)
{
    hipLaunchKernelGGL(persist_advance_kernel, dim3(1), dim3(64), 0, stream, args.ctrl);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    PersistArgs a = args;
    void* kargs[] = {&a};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&persist_sweep_kernel), dim3((unsigned)a.nwg),
                                      dim3(kPThreads), kargs, 0, stream);
}

}  // namespace w4i
