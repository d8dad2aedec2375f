// Host packer: logical INT4 weights + fp16 scales -> W4T4 layout.
//
// "How To Build Your Own LLM Runtime From Scratch" (aitrending.vip),
// "Technical Details" bullet 1, and noticiai.com.br (intro: "pack your own
// weights"): the weights are re-laid offline for the kernels.  The layout here
// is chosen for gfx950 wave64 loads: per tile of 4 rows, each 8-input block is
// one 16-byte chunk holding the 4 rows' words, so a lane's 16-byte load
// covers the same 8 inputs for 4 rows (one LDS read of x serves all four), and
// the nibble slots inside a word are ordered so that two AND-OR masks (before
// and after a shift by 8) yield fp16 pairs that line up with x[k], x[k+1].
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "w4_internal.h"

namespace w4i {

// Slot order inside a word: input offset e -> nibble slot.  Even offsets go
// to the low half-word (slots 0..3), odd offsets to the high half-word (slots
// 4..7), so that slot pairs (p, p+4) feed one fp16x2 lane pair.
static inline uint32_t word_of(const uint8_t* q8, bool* bad)
{
    uint32_t lo = 0, hi = 0;
    uint8_t any = 0;
    for (int p = 0; p < 4; ++p) {
        const uint8_t qe = q8[2 * p];
        const uint8_t qo = q8[2 * p + 1];
        any |= (uint8_t)(qe | qo);
        lo |= (uint32_t)(qe & 0xF) << (4 * p);
        hi |= (uint32_t)(qo & 0xF) << (4 * p);
    }
    if (any & 0xF0) *bad = true;
    return lo | (hi << 16);
}

// Returns -1 on success, else the flat index of the first nibble > 15 found
// (rows are split across threads, so "first" is per the lowest bad row).
int64_t pack_w4t4(const uint8_t* q, const uint16_t* s, int64_t n, int64_t k, int32_t group,
                  bool gateup, uint8_t* pw, uint8_t* ps)
{
    const int64_t tiles = tiles_for(n, gateup);
    const int64_t kb = k / 8;
    const int64_t ng = k / group;
    const int64_t half = n / 2;
    const int64_t tiles_half = (half + kTileRows - 1) / kTileRows;

    unsigned hw = std::thread::hardware_concurrency();
    int64_t nthreads = std::max<int64_t>(1, std::min<int64_t>(hw ? hw : 1, 16));
    // small matrices: one thread
    if (n * k < (int64_t)1 << 22) nthreads = 1;
    nthreads = std::min<int64_t>(nthreads, tiles);

    std::atomic<int64_t> first_bad_row{INT64_MAX};
    auto work = [&](int64_t t0, int64_t t1) {
        for (int64_t t = t0; t < t1; ++t) {
            // logical row of each slot of tile t (-1: padding)
            int64_t rows[kTileRows];
            for (int r = 0; r < kTileRows; ++r) {
                int64_t row;
                if (gateup) {
                    const int64_t tt = t < tiles_half ? t : t - tiles_half;
                    const int64_t local = tt * kTileRows + r;
                    row = local < half ? (t < tiles_half ? local : half + local) : -1;
                } else {
                    row = t * kTileRows + r;
                    if (row >= n) row = -1;
                }
                rows[r] = row;
            }
            uint32_t* dst = reinterpret_cast<uint32_t*>(pw + t * kb * 16);
            for (int64_t j = 0; j < kb; ++j) {
                for (int r = 0; r < kTileRows; ++r) {
                    uint32_t word = 0x88888888u;
                    if (rows[r] >= 0) {
                        bool bad = false;
                        word = word_of(q + rows[r] * k + j * 8, &bad);
                        if (bad) {
                            int64_t cur = first_bad_row.load();
                            while (rows[r] < cur && !first_bad_row.compare_exchange_weak(cur, rows[r])) {
                            }
                        }
                    }
                    dst[j * kTileRows + r] = word;  // little-endian host
                }
            }
            uint16_t* sdst = reinterpret_cast<uint16_t*>(ps + t * ng * 8);
            for (int64_t g = 0; g < ng; ++g)
                for (int r = 0; r < kTileRows; ++r)
                    sdst[g * kTileRows + r] = rows[r] >= 0 ? s[rows[r] * ng + g] : (uint16_t)0;
        }
    };
    if (nthreads == 1) {
        work(0, tiles);
    } else {
        std::vector<std::thread> pool;
        const int64_t per = (tiles + nthreads - 1) / nthreads;
        for (int64_t i = 0; i < nthreads; ++i) {
            const int64_t t0 = i * per, t1 = std::min(tiles, t0 + per);
            if (t0 < t1) pool.emplace_back(work, t0, t1);
        }
        for (auto& th : pool) th.join();
    }
    const int64_t bad_row = first_bad_row.load();
    if (bad_row == INT64_MAX) return -1;
    for (int64_t kk = 0; kk < k; ++kk)
        if (q[bad_row * k + kk] > 15) return bad_row * k + kk;
    return bad_row * k;
}

}  // namespace w4i
