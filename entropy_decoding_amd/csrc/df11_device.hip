// Device half of the DFloat11-style codec: the two-phase decode kernel for
// gfx950 and the df11_decompress_* entry points.
//
// What is computed follows "70% Size, 100% Accuracy ... (DFloat11)",
// abstract: lookup tables held in on-chip memory, a two-phase kernel in which
// small auxiliary arrays fix every thread's read and write positions, and
// transformer-block-level launches; the output is bit-identical BF16.  The
// kernel's organisation is this library's own, for CDNA4.  Two tile shapes
// share the decode steps below: 64-window tiles owned by single waves (the
// default layout, df11_decode_wave: no workgroup barrier after the table
// copy, 4-8% faster on the Llama-3 blocks) and 256- or 512-window tiles owned
// by workgroups (df11_decode, a workgroup-wide scan as on the pages).
//
// * Each workgroup copies the tables into LDS once and then walks about 4
//   tiles, grid-stride; the grid is the larger of the device's resident
//   capacity and n_tiles / 4, rounded up to a multiple of 128 for the XCD
//   renumbering (xcd_grouped).  Many short-lived workgroups measured faster
//   than a resident-only grid (0.62 vs 0.65 ms on the 70B block): their
//   dispatch order keeps the addresses in flight compact.  Occupancy
//   matters: on the 70B block, 6, 5 and 4 workgroups per CU measured 5%,
//   14% and 33% slower than 7; the LDS budget (fast tables, hierarchical
//   tables 1.., staging) stays at 20 KiB so that 8 fit (8 were 2.5-3%
//   faster than 7).  A tile is
//   256*C windows of 8 bytes; thread t decodes windows C*t .. C*t + C - 1 as
//   C independent dependency chains, so each LDS lookup latency is shared by C
//   codes in flight.
// * The next tile's window bytes, gaps and bounds are loaded before the
//   current tile's stores are issued: CDNA counts loads and stores with one
//   in-order counter, so waiting for a load issued after a store would wait
//   for the store.  Bounds arrive through a vector load: a scalar load would
//   share its counter with LDS and stall the decode loops.
// * Phase 1 counts the codes that start in each window, several per step: a
//   12-bit index into the count table gives the start offsets of every code
//   wholly inside those 12 bits as a bit mask, so a step adds the popcount of
//   the mask; the starts a chain's last step finds past the window's end are
//   taken off once, after the loop.
// * A wave64 inclusive scan in DPP row shifts and row broadcasts, then an LDS
//   pass over the 4 wave totals, turns counts into offsets; the tile total
//   must equal block_out_pos[t+1] - block_out_pos[t].
// * Phase 2 walks the windows again with a 10-bit index into the
//   multi-symbol table (up to 3 exponents per step) and writes exponent bytes
//   into an LDS staging buffer at their offsets.  A step writes all 3 slots,
//   so a window's last step may spill up to 2 bytes onto the next window's
//   first two outputs; every window keeps its own first two exponents and
//   rewrites them after a barrier.
// * The decode loops are divergent loops: a lane whose chain has finished
//   leaves the loop (masked off), so it neither counts, writes nor moves,
//   and the wave runs until no lane has work.
// * The outputs are assembled 8 at a time from 8 sm bytes and 8 exponent
//   bytes with byte permutes; the lanes of a wave store 1 KiB contiguously.
// Codes longer than the fast tables' index walk the hierarchical 8-bit
// tables from level 1 (the fast entry names the level-1 table), up to level
// 3 for 32-bit codes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "df11.h"
#include "df11_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMultiOff = 0;                                        // uint32[1024]
constexpr uint32_t kCountOff = kMultiOff + 4u * (1u << DF11_MULTI_BITS);  // uint16[4096]
constexpr uint32_t kLutOff = kCountOff + 2u * (1u << DF11_COUNT_BITS);    // uint16[n][256]
constexpr uint32_t kBadCount = 1u << 20;  // added to a window's count when it is corrupt
// Tiles per wave-tile workgroup slot when the grid is larger than the resident
// capacity.  FP8 units, bound by the decode's VALU work, copy the tables less
// often with 6 (1-2% faster than 4 on the 70B block); BF16 units measured the
// same within noise from 3 to 4 and slower with 6 or 8.
constexpr uint32_t kTilesPerWorkgroup = 4, kTilesPerWorkgroupFp8 = 6;
// Workgroup b runs on XCD b % 8, and each XCD has its own L2.  Blocks of
// 8 * kXcdRun workgroups are renumbered so that every XCD takes kXcdRun
// consecutive ids: neighbouring tiles, which share the 128-byte lines at
// their boundaries, then mostly meet in one L2 (HBM reads on the 70B block
// fell from 4.6% to 0.5% above the algorithmic bytes), while all XCDs still
// work on one compact address range (one contiguous range per XCD measured
// 4% slower).  The grid is a multiple of 8 * kXcdRun, so this is a bijection.
constexpr uint32_t kXcds = 8, kXcdRun = 16, kXcdBlock = kXcds * kXcdRun;

struct KArgs {
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *bop;
    const uint8_t *tables;
    void *out;  // unit element i goes to element i - out_shift (uint16 BF16 or uint8 FP8)
    int32_t *status;
    uint64_t total_bits;
    uint32_t n_weights;
    uint32_t tile0, n_tiles;  // tiles [tile0, tile0 + n_tiles) of the unit
    uint32_t lds_tables;      // bytes of the table image copied to LDS (all but the root)
    uint32_t ebuf_off;        // dynamic-LDS byte offset of the exponent staging buffer
    uint32_t exp_cap;         // its size in bytes
    uint32_t lut_last;        // highest hierarchical table index held in LDS (>= 1)
    uint32_t out_lo, out_hi, out_shift;
};

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t xcd_grouped(uint32_t b) {
    return (b / kXcdBlock) * kXcdBlock + (b % kXcds) * kXcdRun + (b / kXcds) % kXcdRun;
}

typedef __attribute__((address_space(3))) uint8_t lds8;

// The LDS address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return uint32_t(size_t((const lds8 *)p));
}

// Hierarchical walk for a code longer than the fast tables' index, at the
// head of a left-aligned 32-bit window, in lanes where need is set.  The
// walk starts at level 1: the fast entry names the level-1 table that the
// root would point to, so the root table never needs to be in LDS.
// lut[(k - 1) * 256 + b] is entry b of table k >= 1; last is the highest
// table index present (at least 1), and table indices are clamped to it so
// that every read stays inside the tables.  Levels 2 and 3 (codes over 16
// bits) run only when some lane needs them.  Returns the entry reached: a
// leaf (bit 15 clear: length << 8 | symbol), or a pointer (bit 15 set) when
// no leaf is reached by level 3, which a complete code never leaves.
static_assert(DF11_MAX_LUTS <= 256, "a pointer entry's table index must leave the length field zero");
__device__ __forceinline__ uint32_t walk_tables(const uint16_t *lut, uint32_t last,
                                                uint32_t tbl, uint32_t w32, bool need) {
    const uint16_t *lm = lut - 256;  // table k at lm + 256 k
    uint32_t e = lm[(min(tbl, last) << 8) + __builtin_amdgcn_ubfe(w32, 16, 8)];
    if (ballot(need && (e & 0x8000u) != 0)) {
#pragma unroll
        for (int lvl = 2; lvl < 4; lvl++) {
            const uint32_t next = lm[(min(e & 0x7FFFu, last) << 8) + __builtin_amdgcn_ubfe(w32, 24 - 8 * lvl, 8)];
            e = (e & 0x8000u) ? next : e;
        }
    }
    return e;
}

// A multi-symbol entry (one code) for a window whose first code is longer
// than the index; t is the fast-table entry, which holds the level-1 table
// index.  The symbol goes to byte 0 and the length to bits 29..24, with the
// count 1; a length of 0, or a pointer left by a damaged table, is taken as
// 1 so that the chain still moves.
__device__ __forceinline__ uint32_t long_entry(const uint16_t *lut, uint32_t last, uint32_t t,
                                               uint32_t w32, bool need) {
    const uint32_t le = walk_tables(lut, last, t, w32, need) & 0x3FFFu;
    const uint32_t e = __builtin_amdgcn_perm(0u, le, 0x010C0C00u) | (1u << 30);
    return max(e, (1u << 30) | (1u << 24));
}

// Thread t's C windows: 8*C bytes plus the 4 bytes after them (big-endian
// dwords once swapped), their gap bytes and the tile bounds.
template <int C>
struct TileIn {
    uint32_t d[2 * C + 1];
    uint32_t gaps;  // gap of window c in byte c
    uint32_t bounds;
    // t: the thread's index among the tile's W / C threads
    // (tile is wave-uniform: the tile's base addresses stay scalar)
    template <uint32_t W>
    __device__ __forceinline__ void load(const KArgs &a, uint32_t tile, uint32_t t) {
        const uint64_t win0 = uint64_t(tile) * W;
        const uint8_t *wp = a.stream + win0 * 8 + 8 * C * t;
        const uint8_t *gp = a.gaps + win0 + C * t;
        if constexpr (C == 1) {
            const uint2 v = *reinterpret_cast<const uint2 *>(wp);
            d[0] = v.x;
            d[1] = v.y;
            gaps = *gp;
        } else {
            static_assert(C == 2, "one or two windows per thread");
            const uint4 v = *reinterpret_cast<const uint4 *>(wp);
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
            gaps = *reinterpret_cast<const uint16_t *>(gp);
        }
        d[2 * C] = *reinterpret_cast<const uint32_t *>(wp + 8 * C);
        bounds = (a.bop + tile)[t & 1u];
    }
};

// The 32 stream bits starting p bits into segment s (p % 32) of window c:
// alignbit((hi:lo) >> 1, 31 - p % 32), valid for every p % 32 including 0,
// with a = hi >> 1 and b = alignbit(hi, lo, 1) formed once per tile.  The
// decode loops carry q = ~p, and 31 - p % 32 is q mod 32.
template <int C>
struct Windows {
    uint32_t a[C][2], b[C][2];
    __device__ __forceinline__ void init(const uint32_t (&d)[2 * C + 1]) {
#pragma unroll
        for (int c = 0; c < C; c++)
#pragma unroll
            for (int s = 0; s < 2; s++) {
                a[c][s] = d[2 * c + s] >> 1;
                b[c][s] = __builtin_amdgcn_alignbit(d[2 * c + s], d[2 * c + s + 1], 1);
            }
    }
    __device__ __forceinline__ uint32_t at(int c, int s, uint32_t q) const {
        return __builtin_amdgcn_alignbit(a[c][s], b[c][s], q);
    }
    __device__ __forceinline__ uint32_t at_low(int c, uint32_t p) const {  // any p < 64
        return p < 32 ? at(c, 0, ~p) : at(c, 1, ~p);
    }
};

// Phase 1: cnt[c] = number of codes whose first bit lies in [gap_c, lim_c).
// A step adds every code start that its count-table entry marks in the 12
// bits it looks at; only a chain's last step can reach past lim, so the
// starts at or after lim are taken off once, after the loops, from that
// step's entry (kept in el: finished chains are masked off and keep it).
template <int C>
__device__ __forceinline__ void count_codes(const Windows<C> &W, const uint32_t (&gap)[C],
                                            const uint32_t (&lim)[C], const uint8_t *fast,
                                            const uint16_t *lut, uint32_t last,
                                            uint32_t (&cnt)[C]) {
    uint32_t q[C], bad[C], el[C];
#pragma unroll
    for (int c = 0; c < C; c++) {
        q[c] = ~gap[c];
        cnt[c] = 0;
        bad[c] = 0;
        el[c] = 0;
    }
#pragma unroll
    for (int s = 0; s < 2; s++) {
        uint32_t qend[C];
#pragma unroll
        for (int c = 0; c < C; c++) qend[c] = ~min(32u * (s + 1), lim[c]);  // p < end <=> q > ~end
        // one step of chain c
        auto step = [&](int c) {
            const uint32_t w32 = W.at(c, s, q[c]);
            uint32_t e = *reinterpret_cast<const uint16_t *>(
                fast + kCountOff + ((w32 >> (32 - DF11_COUNT_BITS)) << 1));
            if (__builtin_expect(e < (1u << 12), 0)) {  // rare: a first code longer than the index
                const uint32_t le = walk_tables(lut, last, e, w32, true);
                // one code of that length (as an entry: length << 12, one start
                // at offset 0).  A pointer has a zero length field (table
                // indices are below 64); no leaf, or a zero length, means
                // damaged tables: the window is flagged and its chain ends.
                const uint32_t len12 = (le << 4) & 0x3F000u;
                bad[c] |= len12 ? 0u : kBadCount;
                e = len12 ? len12 | 1u : (64u << 12);
            }
            cnt[c] += uint32_t(__builtin_popcount(e & 0xFFFu));
            q[c] -= e >> 12;
            el[c] = e;
        };
        // divergent loops: a lane leaves (is masked off) when its chains are done
        if constexpr (C == 1) {
            while (q[0] > qend[0]) step(0);
        } else {
            for (;;) {
                bool act[C], any = false;
#pragma unroll
                for (int c = 0; c < C; c++) {
                    act[c] = q[c] > qend[c];
                    any |= act[c];
                }
                if (!any) break;
#pragma unroll
                for (int c = 0; c < C; c++)
                    if (act[c]) step(c);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; c++) {
        // the last step started at p_last = p - advance; starts at offset
        // >= lim - p_last in its mask lie at or beyond lim
        const uint32_t cut = min(lim[c] - (~q[c] - (el[c] >> 12)), uint32_t(DF11_COUNT_BITS));
        cnt[c] -= uint32_t(__builtin_popcount(__builtin_amdgcn_ubfe(el[c], cut, DF11_COUNT_BITS - cut)));
        cnt[c] += bad[c];
    }
}

// One phase-2 step of a chain: the multi-symbol entry at its position (a
// long first code resolved), its three exponent bytes written at dst, dst
// and q advanced.  Returns the entry.  Called in divergent code: only the
// lanes whose chain takes the step run it.
__device__ __forceinline__ uint32_t decode_step(uint32_t w32, const uint8_t *fast,
                                                const uint16_t *lut, uint32_t last,
                                                uint32_t &dst, uint32_t &q) {
    uint32_t e = *reinterpret_cast<const uint32_t *>(
        fast + kMultiOff + ((w32 >> (32 - DF11_MULTI_BITS)) << 2));
    if (__builtin_expect(e < (1u << 30), 0))  // rare: a first code longer than 10 bits
        e = long_entry(lut, last, e, w32, true);
    lds8 *o = (lds8 *)size_t(dst);
    o[0] = uint8_t(e);
    o[1] = uint8_t(e >> 8);
    o[2] = uint8_t(e >> 16);
    dst += e >> 30;
    q -= (e >> 24) & 0x3Fu;
    return e;
}

// Phase 2: exponents of window c's codes to LDS bytes dst[c] .., up to 2
// bytes beyond.  dst are LDS addresses, so the stores need no base added.
// A window's last step may write up to two bytes past its codes, onto the
// next window's first two outputs; f01[c] returns window c's own first two
// exponents (byte 0 and byte 1) for rewriting those afterwards.  The first
// two steps are taken at any position below lim (they can cross into the
// second 32-bit segment); the loops then run segment by segment.  Lanes
// whose chains are done are masked off: they neither write nor move.
template <int C>
__device__ __forceinline__ void decode_codes(const Windows<C> &W, const uint32_t (&gap)[C],
                                             const uint32_t (&lim)[C], const uint8_t *fast,
                                             const uint16_t *lut, uint32_t last,
                                             uint32_t (&dst)[C], uint32_t (&f01)[C]) {
    uint32_t q[C];
#pragma unroll
    for (int c = 0; c < C; c++) {
        q[c] = ~gap[c];
        f01[c] = 0;
        if (q[c] > ~lim[c]) f01[c] = decode_step(W.at_low(c, ~q[c]), fast, lut, last, dst[c], q[c]);
    }
#pragma unroll
    for (int c = 0; c < C; c++) {
        if (q[c] > ~lim[c]) {
            const uint32_t e = decode_step(W.at_low(c, ~q[c]), fast, lut, last, dst[c], q[c]);
            // the second exponent is the first entry's second symbol when it holds two or more
            if ((f01[c] >> 30) < 2) f01[c] = __builtin_amdgcn_perm(e, f01[c], 0x07070400u);
        }
    }
#pragma unroll
    for (int s = 0; s < 2; s++) {
        uint32_t qend[C];
#pragma unroll
        for (int c = 0; c < C; c++) qend[c] = ~min(32u * (s + 1), lim[c]);
        if constexpr (C == 1) {
            while (q[0] > qend[0]) decode_step(W.at(0, s, q[0]), fast, lut, last, dst[0], q[0]);
        } else {
            for (;;) {
                bool act[C], any = false;
#pragma unroll
                for (int c = 0; c < C; c++) {
                    act[c] = q[c] > qend[c];
                    any |= act[c];
                }
                if (!any) break;
#pragma unroll
                for (int c = 0; c < C; c++)
                    if (act[c]) decode_step(W.at(c, s, q[c]), fast, lut, last, dst[c], q[c]);
            }
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Four BF16 outputs from four sm bytes S and four exponent bytes E, as two
// dwords: high byte (sm & 0x80) | (e >> 1), low byte (e & 1) << 7 | (sm & 0x7F).
__device__ __forceinline__ void assemble4(uint32_t S, uint32_t E, uint32_t &lo, uint32_t &hi) {
    const uint32_t H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);
    const uint32_t L = ((E << 7) & 0x80808080u) | (S & 0x7F7F7F7Fu);
    lo = __builtin_amdgcn_perm(H, L, 0x05010400u);
    hi = __builtin_amdgcn_perm(H, L, 0x07030602u);
}

__device__ __forceinline__ uint16_t assemble1(uint32_t s, uint32_t e) {
    return uint16_t(((s & 0x80u) << 8) | (e << 7) | (s & 0x7Fu));
}

// Outputs [gi, gi + 8) from 8 sm bytes and 8 staged exponents, as one 16-byte store.
__device__ __forceinline__ void store8(const KArgs &a, uint32_t gi, uint2 s8, const uint8_t *ex) {
    const uint2 e8 = *reinterpret_cast<const uint2 *>(ex);
    uint4 v;
    assemble4(s8.x, e8.x, v.x, v.y);
    assemble4(s8.y, e8.y, v.z, v.w);
    // plain stores: with non-temporal ones the 128-byte lines that two tiles
    // share were written back twice (write traffic 5% above the output size)
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + (gi - a.out_shift)) = v;
}

// Outputs [gi, gi + 8) of the unit from 8 sm bytes and staged exponents ex[0 .. 8).
__device__ __forceinline__ void emit8(const KArgs &a, uint32_t gi, uint32_t lo, uint32_t hi,
                                      uint2 s8, const uint8_t *ex) {
    if (gi >= lo && gi + 8 <= hi) {
        store8(a, gi, s8, ex);
    } else if (gi + 8 > lo && gi < hi) {
        // a tile's first or last chunk: the sm bytes are already in registers
        // (re-reading them from memory would put serial round trips in front
        // of the next barrier)
#pragma unroll
        for (uint32_t k = 0; k < 8; k++) {
            const uint32_t i = gi + k;
            const uint32_t sk = ((k < 4 ? s8.x : s8.y) >> (8 * (k & 3))) & 0xFFu;
            if (i >= lo && i < hi)
                static_cast<uint16_t *>(a.out)[i - a.out_shift] = assemble1(sk, ex[k]);
        }
    }
}

template <int C, int JP>
__global__ __launch_bounds__(kThreads) void df11_decode(KArgs a) {
    // The fixed-size fast tables are the kernel's only static LDS, at address
    // 0, so their offsets fold into the LDS instructions' immediate offsets.
    // Dynamic LDS: hierarchical tables 1 .. n_luts - 1 (the root is never
    // read: the fast tables point past it), 16 bytes of wave totals, staging.
    __shared__ __align__(16) uint8_t fast[kLutOff];
    extern __shared__ __align__(16) uint8_t dyn[];
    constexpr uint32_t W = kThreads * C;  // windows per tile
    const uint32_t t = threadIdx.x, lane = t & 63u, wid = t >> 6;
    const uint32_t first_tile = xcd_grouped(blockIdx.x);
    if (first_tile >= a.n_tiles) return;

    TileIn<C> cur;
    cur.template load<W>(a, a.tile0 + first_tile, t);
    for (uint32_t i = 16 * t; i < a.lds_tables; i += 16 * kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a.tables + (i < kLutOff ? i : i + 512));
        *reinterpret_cast<uint4 *>(i < kLutOff ? fast + i : dyn + (i - kLutOff)) = v;
    }
    __syncthreads();
    const uint16_t *lut = reinterpret_cast<const uint16_t *>(dyn);
    uint32_t *wave_sum = reinterpret_cast<uint32_t *>(dyn + a.ebuf_off - 16);
    uint8_t *ebuf = dyn + a.ebuf_off;

    for (uint32_t it = first_tile; it < a.n_tiles; it += gridDim.x) {
        const uint32_t tile = a.tile0 + it;
        const uint32_t P0 = __builtin_amdgcn_readlane(cur.bounds, 0);
        const uint32_t P1 = __builtin_amdgcn_readlane(cur.bounds, 1);
        const uint32_t A0 = P0 & ~7u;
        // a tile whose bounds are impossible is rejected before anything is read at them
        const bool sane = P0 <= P1 && P1 <= a.n_weights && P1 - A0 + 16 <= a.exp_cap;
        const uint32_t n8 = sane ? (P1 - A0 + 7) >> 3 : 0;
        uint2 smv[JP];
#pragma unroll
        for (int j = 0; j < JP; j++) {
            const uint32_t c = t + j * kThreads;
            if (c < n8) smv[j] = *reinterpret_cast<const uint2 *>(a.sm + A0 + 8 * c);
        }
        // next tile's inputs, issued before this tile's stores
        TileIn<C> nxt;
        nxt.template load<W>(a, a.tile0 + min(it + gridDim.x, a.n_tiles - 1), t);

        uint32_t d[2 * C + 1];
#pragma unroll
        for (int k = 0; k <= 2 * C; k++) d[k] = __builtin_bswap32(cur.d[k]);
        Windows<C> win;
        win.init(d);
        uint32_t gap[C], lim[C];
#pragma unroll
        for (int c = 0; c < C; c++) {
            gap[c] = (cur.gaps >> (8 * c)) & 0xFFu;
            const uint64_t base = (uint64_t(tile) * W + uint64_t(C) * t + c) * 64;
            lim[c] = a.total_bits > base ? uint32_t(min<uint64_t>(64, a.total_bits - base)) : 0u;
        }

        // phase 1 and the block scan
        uint32_t cnt[C];
        count_codes<C>(win, gap, lim, fast, lut, a.lut_last, cnt);
        uint32_t mine_total = 0;
#pragma unroll
        for (int c = 0; c < C; c++) mine_total += cnt[c];
        const uint32_t incl = wave_inclusive_scan(mine_total);
        if (lane == 63) wave_sum[wid] = incl;
        __syncthreads();
        const uint4 ws = *reinterpret_cast<const uint4 *>(wave_sum);
        const uint32_t total = ws.x + ws.y + ws.z + ws.w;
        const uint32_t before =
            (wid > 0 ? ws.x : 0u) + (wid > 1 ? ws.y : 0u) + (wid > 2 ? ws.z : 0u);
        if (!sane || total != P1 - P0) {  // uniform: every thread skips the tile
            if (t == 0 && a.status) atomicExch(a.status, int32_t(DF11_E_CORRUPT));
            __syncthreads();  // wave_sum is rewritten by the next tile
            cur = nxt;
            continue;
        }

        // phase 2, then repair the two bytes a neighbour's last step may have spilled onto;
        // positions are LDS addresses
        uint32_t first[C], dst[C];
        first[0] = lds_addr(ebuf) + (P0 - A0) + before + incl - mine_total;
#pragma unroll
        for (int c = 1; c < C; c++) first[c] = first[c - 1] + cnt[c - 1];
#pragma unroll
        for (int c = 0; c < C; c++) dst[c] = first[c];
        uint32_t f01[C];
        decode_codes<C>(win, gap, lim, fast, lut, a.lut_last, dst, f01);
        __syncthreads();
#pragma unroll
        for (int c = 0; c < C; c++) {
            lds8 *o = (lds8 *)size_t(first[c]);
            if (cnt[c]) o[0] = uint8_t(f01[c]);
            if (cnt[c] > 1) o[1] = uint8_t(f01[c] >> 8);
        }
        __syncthreads();

        // assemble and store: for each j, the lanes of a wave write 1 KiB contiguously
        const uint32_t lo = max(P0, a.out_lo), hi = min(P1, a.out_hi);
#pragma unroll
        for (int j = 0; j < JP; j++) {
            const uint32_t c = t + j * kThreads;
            if (c < n8) emit8(a, A0 + 8 * c, lo, hi, smv[j], ebuf + 8 * c);
        }
        for (uint32_t c = t + JP * kThreads; c < n8; c += kThreads)
            emit8(a, A0 + 8 * c, lo, hi, *reinterpret_cast<const uint2 *>(a.sm + A0 + 8 * c),
                  ebuf + 8 * c);
        cur = nxt;
    }
}

// Output formats of the wave kernel.  A chunk is the outputs one lane
// stores with one 16-byte write: 8 BF16 values or 16 FP8 values; either way
// it takes 8 bytes of the sign+mantissa array (bytes, or nibbles two per
// byte).  rest_off(g) is the byte offset in that array of weight g's field.
template <int FMT>
struct OutFmt;
template <>
struct OutFmt<DF11_FORMAT_BF16> {
    static constexpr uint32_t kChunk = 8;
    static __device__ __forceinline__ uint32_t rest_off(uint32_t g) { return g; }
    static constexpr uint32_t kElemBytes = 2;
    static __device__ __forceinline__ uint4 chunk(uint2 s8, const uint8_t *ex) {
        const uint2 e8 = *reinterpret_cast<const uint2 *>(ex);
        uint4 v;
        assemble4(s8.x, e8.x, v.x, v.y);
        assemble4(s8.y, e8.y, v.z, v.w);
        return v;
    }
    // chunk c counted from output element base (which may lie before out)
    static __device__ __forceinline__ void store_at(const KArgs &a, int64_t base, uint32_t c,
                                                    uint2 s8, const uint8_t *ex) {
        uint16_t *o = static_cast<uint16_t *>(a.out) + base;
        reinterpret_cast<uint4 *>(o)[c] = chunk(s8, ex);
    }
    // element k (< 8) of a chunk
    static __device__ __forceinline__ uint32_t value1(uint2 s8, uint32_t k, uint32_t e) {
        const uint32_t sk = ((k < 4 ? s8.x : s8.y) >> (8 * (k & 3))) & 0xFFu;
        return assemble1(sk, e);
    }
    static __device__ __forceinline__ void store1(const KArgs &a, uint32_t i, uint2 s8, uint32_t k,
                                                  uint32_t e) {
        static_cast<uint16_t *>(a.out)[i - a.out_shift] = uint16_t(value1(s8, k, e));
    }
    static __device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                         uint32_t v) {
        __builtin_amdgcn_raw_buffer_store_b16(uint16_t(v), r, off, 0, 0);
    }
};
// FP8: byte = sign << 7 | e << M | mantissa, from the nibble (sign << M | mantissa)
template <int M>
struct OutFp8 {
    static constexpr uint32_t kChunk = 16;
    static constexpr uint32_t kSign = 0x80808080u;
    static constexpr uint32_t kKeep = kSign | (0x01010101u * ((1u << M) - 1u));  // sign and mantissa
    static __device__ __forceinline__ uint32_t rest_off(uint32_t g) { return g >> 1; }
    // four outputs from four nibbles (one per byte of D) and four exponents E
    static __device__ __forceinline__ uint32_t assemble(uint32_t D, uint32_t E) {
        constexpr uint32_t mant = 0x01010101u * ((1u << M) - 1u);
        return (D & mant) | ((D << (7 - M)) & kSign) | (E << M);
    }
    // Eight outputs from the 8 nibbles of S and 8 exponents (E0: outputs
    // 0..3, E1: 4..7).  lo holds the even nibbles one per byte and hi the odd
    // ones, each with its sign bit copied to bit 7 (the other bits above the
    // mantissa are cleared by kKeep); byte permutes interleave them into
    // output order.
    static __device__ __forceinline__ void assemble8(uint32_t S, uint32_t E0, uint32_t E1,
                                                     uint32_t &o0, uint32_t &o1) {
        const uint32_t lo = ((S << (7 - M)) & kSign) | (S & ~kSign);
        const uint32_t hi = ((S << (3 - M)) & kSign) | ((S >> 4) & ~kSign);
        o0 = (__builtin_amdgcn_perm(hi, lo, 0x05010400u) & kKeep) | (E0 << M);
        o1 = (__builtin_amdgcn_perm(hi, lo, 0x07030602u) & kKeep) | (E1 << M);
    }
    static __device__ __forceinline__ uint4 chunk(uint2 s8, const uint8_t *ex) {
        const uint4 e16 = *reinterpret_cast<const uint4 *>(ex);
        uint4 v;
        assemble8(s8.x, e16.x, e16.y, v.x, v.y);
        assemble8(s8.y, e16.z, e16.w, v.z, v.w);
        return v;
    }
    static __device__ __forceinline__ void store_at(const KArgs &a, int64_t base, uint32_t c,
                                                    uint2 s8, const uint8_t *ex) {
        uint8_t *o = static_cast<uint8_t *>(a.out) + base;
        reinterpret_cast<uint4 *>(o)[c] = chunk(s8, ex);
    }
    static constexpr uint32_t kElemBytes = 1;
    static __device__ __forceinline__ uint32_t value1(uint2 s8, uint32_t k, uint32_t e) {
        const uint32_t b = ((k < 8 ? s8.x : s8.y) >> (8 * ((k >> 1) & 3))) & 0xFFu;
        const uint32_t nib = (k & 1) ? (b >> 4) : (b & 0xFu);
        return assemble(nib, e) & 0xFFu;
    }
    static __device__ __forceinline__ void store1(const KArgs &a, uint32_t i, uint2 s8, uint32_t k,
                                                  uint32_t e) {
        static_cast<uint8_t *>(a.out)[i - a.out_shift] = uint8_t(value1(s8, k, e));
    }
    static __device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                         uint32_t v) {
        __builtin_amdgcn_raw_buffer_store_b8(uint8_t(v), r, off, 0, 0);
    }
};
template <>
struct OutFmt<DF11_FORMAT_FP8_E4M3> : OutFp8<3> {};
template <>
struct OutFmt<DF11_FORMAT_FP8_E5M2> : OutFp8<2> {};

// The 8 sm bytes of chunk c (wave-uniform, c < n8) of a tile, from the
// registers of the lane that prefetched them, or from memory past the
// prefetched chunks.
template <int JP, int FMT, bool kInSlots = false>
__device__ __forceinline__ uint2 chunk_sm(const KArgs &a, const uint2 (&smv)[JP], uint32_t A0,
                                          uint32_t c) {
    const uint32_t j = c >> 6, l = c & 63u;
    uint2 r = make_uint2(0, 0);
#pragma unroll
    for (int q = 0; q < JP; q++) {
        if (j == uint32_t(q)) {
            r.x = __builtin_amdgcn_readlane(smv[q].x, l);
            r.y = __builtin_amdgcn_readlane(smv[q].y, l);
        }
    }
    // (kInSlots: the caller knows c < 64 JP, so no path loads from memory)
    if (!kInSlots && j >= uint32_t(JP))
        r = *reinterpret_cast<const uint2 *>(a.sm + OutFmt<FMT>::rest_off(A0) + 8 * c);
    return r;
}

// The same two phases with tiles of 64 windows, one per wave: thread lane of
// a wave decodes window lane of the wave's tile.  After the one-time table
// copy there is no workgroup barrier: each wave counts, scans (DPP only),
// decodes, repairs and stores its own tile, and LDS operations of one wave
// take effect in issue order, so its later reads see its earlier writes.
// Each wave has its own staging buffer.  The chunks holding a tile's first
// and last outputs are usually shared with the neighbouring tiles; they are
// written element by element, one lane per element, in one pass.  FMT is the
// weight format (BF16 or FP8): only the final assembly differs.
//
// Epi is what happens to a decoded tile: StoreEpi writes the weights, the
// fused GEMV and GEMM consume them (df11_decompress_gemv, _gemm).  Epi::kSmv
// says whether the tile's sign+mantissa bytes are loaded in lane order
// (chunk lane + 64 j in smv[j]) before the decode; Epi::prefetch may load
// whatever else the epilogue needs at that point; Epi::kAlways says that the
// epilogue also runs on a rejected tile (with an empty range), so that every
// path through the loop issues its memory instructions.  The wave takes
// tiles first + slot, first + slot + n_slots, ... below first + count.
template <int JP, int FMT, class Epi>
__device__ __forceinline__ void wave_tiles(const KArgs &a, Epi &epi, uint32_t first,
                                           uint32_t count, uint32_t slot, uint32_t n_slots) {
    using F = OutFmt<FMT>;
    constexpr uint32_t CH = F::kChunk;
    __shared__ __align__(16) uint8_t fast[kLutOff];
    extern __shared__ __align__(16) uint8_t dyn[];
    constexpr uint32_t W = 64;  // windows per tile
    const uint32_t t = threadIdx.x, lane = t & 63u, wid = t >> 6;

    TileIn<1> cur;
    if (slot < count) cur.load<W>(a, first + slot, lane);
    for (uint32_t i = 16 * t; i < a.lds_tables; i += 16 * kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a.tables + (i < kLutOff ? i : i + 512));
        *reinterpret_cast<uint4 *>(i < kLutOff ? fast + i : dyn + (i - kLutOff)) = v;
    }
    __syncthreads();
    // Let the first tile's loads complete here, so that the wait at the top
    // of the tile loop is set by the loop's own paths.  The immediate is the
    // gfx9 s_waitcnt encoding of vmcnt(0) with expcnt and lgkmcnt left at
    // their maxima (7 in bits 6:4, 15 in bits 11:8).
    if constexpr (Epi::kAlways) __builtin_amdgcn_s_waitcnt(0x0F70);
    const uint16_t *lut = reinterpret_cast<const uint16_t *>(dyn);
    uint8_t *ebuf = dyn + a.ebuf_off + wid * a.exp_cap;
    // The FP8 assembly shifts whole dwords of staged exponents, so a staged
    // byte with bits above the symbol's width would carry into the next
    // output's mantissa.  Every byte this kernel stages is a symbol, but the
    // first chunk's bytes below a tile's first output are never written by
    // that tile and start as whatever LDS held before (another kernel's
    // data); they are cleared once.
    if constexpr (FMT != DF11_FORMAT_BF16)
        if (lane < 4) reinterpret_cast<uint32_t *>(ebuf)[lane] = 0;

    for (uint32_t it = slot; it < count; it += n_slots) {
        const uint32_t tile = first + it;
        const uint32_t P0 = __builtin_amdgcn_readlane(cur.bounds, 0);
        const uint32_t P1 = __builtin_amdgcn_readlane(cur.bounds, 1);
        const uint32_t A0 = P0 & ~(CH - 1);
        const bool sane = P0 <= P1 && P1 <= a.n_weights && P1 - A0 + 16 <= a.exp_cap;
        const uint32_t n8 = sane ? (P1 - A0 + CH - 1) / CH : 0;  // chunks
        const uint8_t *sm0 = a.sm + F::rest_off(A0);
        uint2 smv[JP];
        if constexpr (Epi::kSmv) {
#pragma unroll
            for (int j = 0; j < JP; j++) {
                const uint32_t c = lane + j * 64;
                if (c < n8) smv[j] = reinterpret_cast<const uint2 *>(sm0 + 8 * size_t(lane))[64 * j];
            }
        }
        if (sane) epi.prefetch(a, P0, P1, lane);
        TileIn<1> nxt;
        nxt.load<W>(a, first + min(it + n_slots, count - 1), lane);

        uint32_t d[3];
#pragma unroll
        for (int k = 0; k < 3; k++) d[k] = __builtin_bswap32(cur.d[k]);
        Windows<1> win;
        win.init(d);
        uint32_t gap[1], lim[1];
        gap[0] = cur.gaps & 0xFFu;
        {
            // stream bits of the tile (uniform), then this lane's share of them
            const uint64_t tbase = uint64_t(tile) * W * 64;
            const uint32_t rem = a.total_bits > tbase ? uint32_t(min<uint64_t>(W * 64, a.total_bits - tbase)) : 0u;
            lim[0] = uint32_t(min(max(int32_t(rem) - int32_t(64 * lane), 0), 64));
        }

        uint32_t cnt[1];
        count_codes<1>(win, gap, lim, fast, lut, a.lut_last, cnt);
        const uint32_t incl = wave_inclusive_scan(cnt[0]);
        const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
        const bool ok = sane && total == P1 - P0;  // uniform over the wave
        if (!ok) {
            if (lane == 0 && a.status) atomicExch(a.status, int32_t(DF11_E_CORRUPT));
            // An epilogue with a fixed number of memory instructions runs on a
            // rejected tile too, with an empty range (BufStoreEpi): a path that
            // skipped its stores would make the wait at the top of the loop
            // wait for every store of the tile.
            if constexpr (!Epi::kAlways) {
                cur = nxt;
                continue;
            }
        }

        if (ok) {
            uint32_t beg[1], dst[1];  // LDS addresses of the window's first output
            beg[0] = lds_addr(ebuf) + (P0 - A0) + incl - cnt[0];
            dst[0] = beg[0];
            uint32_t f01[1];
            decode_codes<1>(win, gap, lim, fast, lut, a.lut_last, dst, f01);
            // keep the compiler from moving LDS accesses across the steps below;
            // the hardware keeps one wave's LDS operations in order
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            {
                lds8 *o = (lds8 *)size_t(beg[0]);
                if (cnt[0]) o[0] = uint8_t(f01[0]);
                if (cnt[0] > 1) o[1] = uint8_t(f01[0] >> 8);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }

        epi.template tile<JP, FMT>(a, tile, P0, ok ? P1 : P0, A0, ok ? n8 : 0u, smv, sm0, ebuf, lane);
        cur = nxt;
    }
}

struct StoreEpi {
    static constexpr bool kSmv = true, kAlways = false;
    __device__ __forceinline__ void prefetch(const KArgs &, uint32_t, uint32_t, uint32_t) {}
    template <int JP, int FMT>
    __device__ __forceinline__ void tile(const KArgs &a, uint32_t, uint32_t P0, uint32_t P1,
                                         uint32_t A0, uint32_t n8, const uint2 (&smv)[JP],
                                         const uint8_t *sm0, const uint8_t *ebuf, uint32_t lane) {
        using F = OutFmt<FMT>;
        constexpr uint32_t CH = F::kChunk;
        // whole chunks: the lanes of the wave write 1 KiB contiguously per j.
        // Chunk c is whole and in range when c_lo <= c < c_hi (uniform bounds).
        const uint32_t lo = max(P0, a.out_lo), hi = min(P1, a.out_hi);
        const int32_t c_lo = int32_t((lo - A0 + CH - 1) / CH);
        const int32_t c_hi = hi > A0 ? int32_t((hi - A0) / CH) : 0;
        const int32_t r0 = int32_t(lane) - c_lo, r1 = int32_t(lane) - c_hi;
        const uint8_t *el = ebuf + CH * lane;
        const int64_t base = int64_t(A0) - int64_t(a.out_shift);  // output index of chunk 0
#pragma unroll
        for (int j = 0; j < JP; j++)
            if (r0 >= -64 * j && r1 < -64 * j)
                F::store_at(a, base, lane + 64 * j, smv[j], el + 64 * CH * j);
        for (uint32_t c = lane + JP * 64; c < n8; c += 64) {
            if (int32_t(c) >= c_lo && int32_t(c) < c_hi)
                F::store_at(a, base, c, *reinterpret_cast<const uint2 *>(sm0 + 8 * c), ebuf + CH * c);
        }
        // the chunks holding the first and last output in range, element by
        // element: lanes 0 .. CH-1 and CH .. 2CH-1 (they are whole only when aligned)
        if (lo < hi) {
            const uint32_t ch = (lo - A0) / CH, ct = (hi - 1 - A0) / CH;
            const uint2 sh = chunk_sm<JP, FMT>(a, smv, A0, ch), sl = chunk_sm<JP, FMT>(a, smv, A0, ct);
            if (lane < 2 * CH) {
                const uint32_t c = lane < CH ? ch : ct, k = lane & (CH - 1);
                const uint32_t gi = A0 + CH * c, i = gi + k;
                const bool whole = gi >= lo && gi + CH <= hi;
                if (!whole && i >= lo && i < hi) F::store1(a, i, lane < CH ? sh : sl, k, ebuf[CH * c + k]);
            }
        }
    }
};

// the grid's waves over the tiles tile0 .. tile0 + n_tiles - 1, in the
// XCD-grouped order
template <int JP, int FMT, class Epi>
__device__ __forceinline__ void wave_tiles(const KArgs &a, Epi &epi) {
    const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
    wave_tiles<JP, FMT>(a, epi, a.tile0, a.n_tiles, 4 * xcd_grouped(blockIdx.x) + wid,
                        4 * gridDim.x);
}

template <int JP, int FMT>
__global__ __launch_bounds__(kThreads) void df11_decode_wave(KArgs a) {
    StoreEpi epi;
    wave_tiles<JP, FMT>(a, epi);
}

// The store epilogue for units whose tiles all fit the JP prefetched chunk
// slots (n8 <= 64 JP).  Every lane issues the same JP + 1 stores on every
// tile, through buffer resources whose ranges cover exactly the outputs the
// tile may write; the hardware drops stores outside a resource's range, so
// no lane needs a branch or an exec mask to stay out of its neighbours'
// outputs.  With a fixed count of stores after the next tile's loads, the
// wait for those loads at the top of the next tile need not wait for this
// tile's stores to complete (CDNA counts loads and stores in order with one
// counter; a store count that varied by path forced a wait for all of them).
struct BufStoreEpi {
    static constexpr bool kSmv = true, kAlways = true;
    __device__ __forceinline__ void prefetch(const KArgs &, uint32_t, uint32_t, uint32_t) {}
    template <int JP, int FMT>
    __device__ __forceinline__ void tile(const KArgs &a, uint32_t, uint32_t P0, uint32_t P1,
                                         uint32_t A0, uint32_t n8, const uint2 (&smv)[JP],
                                         const uint8_t *, const uint8_t *ebuf, uint32_t lane) {
        using F = OutFmt<FMT>;
        constexpr uint32_t CH = F::kChunk, ES = F::kElemBytes;
        constexpr uint32_t kDrop = 0x80000000u;  // an offset far outside every range
        const uint32_t lo = max(P0, a.out_lo), hi = min(P1, a.out_hi);
        const bool any = lo < hi;
        // whole chunks c_lo .. c_hi - 1 (uniform)
        const int32_t c_lo = any ? int32_t((lo - A0 + CH - 1) / CH) : 0;
        const int32_t c_hi = any ? max(int32_t((hi - A0) / CH), c_lo) : c_lo;
        char *out0 = static_cast<char *>(a.out) + (int64_t(A0) - int64_t(a.out_shift)) * ES;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            out0 + 16 * int64_t(c_lo), 0, uint32_t(16 * (c_hi - c_lo)), 0x00020000);
        const int32_t r = 16 * (int32_t(lane) - c_lo);
        const uint32_t cmax = n8 ? n8 - 1 : 0;  // staging reads stay inside the tile
#pragma unroll
        for (int j = 0; j < JP; j++) {
            const uint32_t c = min(lane + 64 * j, cmax);
            const uint4 v = F::chunk(smv[j], ebuf + CH * c);
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 w = {v.x, v.y, v.z, v.w};
            // a negative offset (a chunk below c_lo) keeps its sign bit and
            // stays far from wrapping around: outside the range
            __builtin_amdgcn_raw_buffer_store_b128(w, rc, uint32_t(r + 1024 * j) & 0x8FFFFFFFu, 0, 0);
        }
        // the chunks holding the first and last output, element by element:
        // lanes 0 .. CH-1 and CH .. 2CH-1, except where the chunk was whole
        const uint32_t ch = any ? (lo - A0) / CH : 0, ct = any ? (hi - 1 - A0) / CH : 0;
        const uint2 sh = chunk_sm<JP, FMT, true>(a, smv, A0, ch), sl = chunk_sm<JP, FMT, true>(a, smv, A0, ct);
        const uint32_t c = lane < CH ? ch : ct, k = lane & (CH - 1);
        const uint32_t i = A0 + CH * c + k;
        const bool whole = int32_t(c) >= c_lo && int32_t(c) < c_hi;
        const uint32_t v = F::value1(lane < CH ? sh : sl, k, ebuf[CH * c + k]);
        // the range is wave-uniform; built from scalars, so that the compiler
        // does not loop over lanes to find distinct descriptors
        const uint64_t pe = reinterpret_cast<uint64_t>(static_cast<char *>(a.out) +
                                                       (int64_t(lo) - int64_t(a.out_shift)) * ES);
        const uint32_t pe_lo = __builtin_amdgcn_readfirstlane(uint32_t(pe));
        const uint32_t pe_hi = __builtin_amdgcn_readfirstlane(uint32_t(pe >> 32));
        const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char *>((uint64_t(pe_hi) << 32) | pe_lo), 0,
            __builtin_amdgcn_readfirstlane(any ? (hi - lo) * ES : 0u), 0x00020000);
        const bool mine = lane < 2 * CH && !whole && i >= lo;
        F::buffer_store1(re, mine ? (i - lo) * ES : kDrop, v);
    }
};

template <int JP, int FMT>
__global__ __launch_bounds__(kThreads) void df11_decode_wave_fixed(KArgs a) {
    BufStoreEpi epi;
    wave_tiles<JP, FMT>(a, epi);
}

// ------------------------------------------------------------ phase-1 counts
// counts[j] = the codes whose first bit lies in stream window j, from the
// decode kernels' own first phase (count_codes), one window per thread: a
// diagnostic that checks that phase window by window.
__global__ __launch_bounds__(kThreads) void df11_count_windows(KArgs a, uint32_t n_windows,
                                                               uint32_t *counts) {
    __shared__ __align__(16) uint8_t fast[kLutOff];
    extern __shared__ __align__(16) uint8_t dyn[];
    const uint32_t t = threadIdx.x;
    for (uint32_t i = 16 * t; i < a.lds_tables; i += 16 * kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a.tables + (i < kLutOff ? i : i + 512));
        *reinterpret_cast<uint4 *>(i < kLutOff ? fast + i : dyn + (i - kLutOff)) = v;
    }
    __syncthreads();
    const uint16_t *lut = reinterpret_cast<const uint16_t *>(dyn);
    const uint32_t j = blockIdx.x * kThreads + t;
    if (j >= n_windows) return;
    // the window's 8 bytes and the 4 after it (the stream ends in 4 padding bytes)
    const uint32_t *wp = reinterpret_cast<const uint32_t *>(a.stream + 8 * uint64_t(j));
    uint32_t d[3];
#pragma unroll
    for (int k = 0; k < 3; k++) d[k] = __builtin_bswap32(wp[k]);
    Windows<1> win;
    win.init(d);
    const uint64_t base = 64 * uint64_t(j);
    uint32_t gap[1] = {a.gaps[j]}, cnt[1];
    uint32_t lim[1] = {a.total_bits > base ? uint32_t(min<uint64_t>(64, a.total_bits - base)) : 0u};
    count_codes<1>(win, gap, lim, fast, lut, a.lut_last, cnt);
    counts[j] = cnt[0];
}

// ---------------------------------------------------------------- fused GEMV
//
// y = W x for the matrices of a BF16 unit, straight from the compressed
// stream: a decoded tile multiplies its weights by x instead of storing them.
// A tile touches at most kRowsPerTile consecutive rows (the host checks this
// from max_tile_symbols and the narrowest matrix); each lane accumulates its
// chunks' products per row, a butterfly over the wave sums the lanes, and the
// tile's row sums go to a scratch array; a second kernel adds, for every row,
// the sums of the tiles that hold it, in tile order.  Every sum is formed in a
// fixed order, so results are deterministic.

constexpr uint32_t kRowsPerTile = 4;

struct GemvDesc {
    uint32_t n;
    // first element of each matrix in the unit; entries n .. 16 hold N, so
    // that the matrix of element e is the number of entries 1 .. 16 <= e
    uint32_t off[DF11_GEMV_MAX_TENSORS + 1];
    uint32_t row0[DF11_GEMV_MAX_TENSORS + 1];  // first global row of each matrix, then the total
    uint32_t cols[DF11_GEMV_MAX_TENSORS];
    uint32_t inv[DF11_GEMV_MAX_TENSORS];  // ceil(2^32 / cols)
    uint32_t x_off[DF11_GEMV_MAX_TENSORS], y_off[DF11_GEMV_MAX_TENSORS];
};

// matrix holding unit element e (e < N): scalar compares over the whole table
__device__ __forceinline__ uint32_t matrix_of(const GemvDesc &g, uint32_t e) {
    uint32_t k = 0;
#pragma unroll
    for (uint32_t m = 1; m <= DF11_GEMV_MAX_TENSORS; m++) k += uint32_t(e >= g.off[m]);
    return k;
}

// floor(v / d) for d = g.cols[k] >= 8, from inv = ceil(2^32 / d): the product's
// high word is the quotient or one more (v < 2^32), so one correction
__device__ __forceinline__ uint32_t div_cols(const GemvDesc &g, uint32_t k, uint32_t v) {
    uint32_t q = __umulhi(v, g.inv[k]);
    if (uint64_t(q) * g.cols[k] > v) q--;
    return q;
}

// Sum over the 64 lanes of a wave, in a fixed order: rows of 16 lanes by DPP
// (lane pairs, quads, then rotations by 4 and 8), then the four row sums of
// lanes 0, 16, 32 and 48 in order.  The result is uniform.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_f(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);  // row_ror:4
    v += dpp_f<0x128>(v);  // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// fp32 value of a BF16 weight from its sign+mantissa byte and exponent byte
__device__ __forceinline__ float bf16_value(uint32_t sm, uint32_t e) {
    return __uint_as_float(((sm & 0x80u) << 24) | (e << 23) | ((sm & 0x7Fu) << 16));
}

// acc + the dot product of 8 weights (sm bytes S, exponent bytes E, two words
// each) with x[0..7], as a chain of fused multiply-adds.  Byte k of H is
// sm.7 | e.7..1 and of L e.0 | sm.6..0, so one byte permute places the fp32
// bits of weight k, [H_k, L_k, 0, 0].
__device__ __forceinline__ float dot8_bf16(float acc, uint2 S, uint2 E, const float4 &x0,
                                           const float4 &x1) {
    const uint32_t H0 = (S.x & 0x80808080u) | ((E.x >> 1) & 0x7F7F7F7Fu);
    const uint32_t L0 = ((E.x << 7) & 0x80808080u) | (S.x & 0x7F7F7F7Fu);
    const uint32_t H1 = (S.y & 0x80808080u) | ((E.y >> 1) & 0x7F7F7F7Fu);
    const uint32_t L1 = ((E.y << 7) & 0x80808080u) | (S.y & 0x7F7F7F7Fu);
    auto w = [](uint32_t H, uint32_t L, uint32_t k) {
        return __uint_as_float(__builtin_amdgcn_perm(H, L, ((4u + k) << 24) | (k << 16) | 0x0C0Cu));
    };
    acc = fmaf(w(H0, L0, 0), x0.x, acc);
    acc = fmaf(w(H0, L0, 1), x0.y, acc);
    acc = fmaf(w(H0, L0, 2), x0.z, acc);
    acc = fmaf(w(H0, L0, 3), x0.w, acc);
    acc = fmaf(w(H1, L1, 0), x1.x, acc);
    acc = fmaf(w(H1, L1, 1), x1.y, acc);
    acc = fmaf(w(H1, L1, 2), x1.z, acc);
    acc = fmaf(w(H1, L1, 3), x1.w, acc);
    return acc;
}

struct GemvEpi {
    static constexpr bool kSmv = true, kAlways = false;
    __device__ __forceinline__ void prefetch(const KArgs &, uint32_t, uint32_t, uint32_t) {}
    const GemvDesc *g;
    const float *x;
    float *part;     // kRowsPerTile row sums per tile
    uint32_t *row_a;  // first global row of each tile

    template <int JP, int FMT>
    __device__ __forceinline__ void tile(const KArgs &a, uint32_t tile, uint32_t P0, uint32_t P1,
                                         uint32_t A0, uint32_t n8, const uint2 (&smv)[JP],
                                         const uint8_t *sm0, const uint8_t *ebuf, uint32_t lane) {
        const GemvDesc &d = *g;
        float *pt = part + uint64_t(tile) * kRowsPerTile;
        if (P0 == P1) {  // a tile past the last code start holds no weights
            if (lane < kRowsPerTile) pt[lane] = 0.0f;
            if (lane == 0) row_a[tile] = 0;
            return;
        }
        // the tile's first row ra, and the rows it touches (uniform over the wave)
        const uint32_t ka = matrix_of(d, P0), kb = matrix_of(d, P1 - 1);
        const uint32_t qa = div_cols(d, ka, P0 - d.off[ka]);
        const uint32_t ra = d.row0[ka] + qa;
        const uint32_t rb = d.row0[kb] + div_cols(d, kb, P1 - 1 - d.off[kb]);
        const uint32_t nrows = rb - ra + 1;
        if (nrows > kRowsPerTile) {
            // impossible for a valid unit (the host checks the widest tile
            // against the narrowest matrix); a corrupt one is reported
            if (lane < kRowsPerTile) pt[lane] = 0.0f;
            if (lane == 0) {
                row_a[tile] = ra;
                if (a.status) atomicExch(a.status, int32_t(DF11_E_CORRUPT));
            }
            return;
        }
        const uint32_t passes = (n8 + 63) / 64;  // 64-chunk passes over the tile
        float acc[kRowsPerTile] = {};
        if (ka == kb && d.cols[ka] >= 512 * passes) {
            // Rows at least as long as the span of one lane's chunks (so the
            // tile touches at most two rows and each lane crosses at most
            // one row start).  Lane l takes chunks l, l+64, ...: a column that
            // advances by 512 per pass, a running sum for the lane's first row
            // (sa) and one for the next (sb), updated by selects.
            const uint32_t cols = d.cols[ka];
            const uint32_t rs = d.off[ka] + qa * cols;  // start of row ra
            const float *xk = x + d.x_off[ka];
            const uint32_t cw0 = P0 == A0 ? 0u : 1u, cw1 = (P1 - A0) / 8;  // whole chunks
            uint32_t col0 = A0 + 8 * lane - rs;
            const bool first_next = col0 >= cols;  // the lane's first chunk is in row ra+1
            col0 -= first_next ? cols : 0u;
            // pass j: column col0 + 512 j, one row further once that reaches
            // cols (below 2 cols, since 512 passes <= cols: one wrap at most)
            float sa = 0.0f, sb = 0.0f;
            auto pass = [&](uint32_t j, uint2 s8) {
                const uint32_t c = lane + 64 * j;
                const uint32_t v = col0 + 512 * j;
                const bool wrapped = v >= cols;
                const float *xp = xk + (wrapped ? v - cols : v);
                const float4 x0 = *reinterpret_cast<const float4 *>(xp);
                const float4 x1 = *reinterpret_cast<const float4 *>(xp + 4);
                const bool ok = c >= cw0 && c < cw1;
                const uint2 e8 = *reinterpret_cast<const uint2 *>(ebuf + 8 * min(c, n8 - 1));
                const float t = dot8_bf16(wrapped ? sb : sa, s8, e8, x0, x1);
                sa = ok && !wrapped ? t : sa;
                sb = ok && wrapped ? t : sb;
            };
#pragma unroll
            for (int j = 0; j < JP; j++)
                if (j < passes) pass(j, smv[j]);
            for (uint32_t j = JP; j < passes; j++) {
                const uint32_t c = min(lane + 64 * j, n8 - 1);
                pass(j, *reinterpret_cast<const uint2 *>(sm0 + 8 * c));
            }
            // rows relative to ra: sa is row first_next, sb the row after
            acc[0] = first_next ? 0.0f : sa;
            acc[1] = first_next ? sa : sb;
            // the chunks holding P0 and P1-1 when they are not whole, one
            // element per lane (lanes 0-7 and 8-15; once if they coincide)
            const uint32_t ch = 0, ct = n8 - 1;
            const bool edge_h = cw0 > 0 || cw1 == 0, edge_t = ct >= cw1 && ct != ch;
            if (edge_h || edge_t) {
                const uint2 sh = chunk_sm<JP, FMT>(a, smv, A0, ch), sl = chunk_sm<JP, FMT>(a, smv, A0, ct);
                if (lane < 16) {
                    const uint32_t c = lane < 8 ? ch : ct, k = lane & 7u;
                    const uint32_t i = A0 + 8 * c + k;
                    if ((lane < 8 ? edge_h : edge_t) && i >= P0 && i < P1) {
                        const uint2 s8 = lane < 8 ? sh : sl;
                        const uint32_t sb8 = ((k < 4 ? s8.x : s8.y) >> (8 * (k & 3u))) & 0xFFu;
                        const float w = bf16_value(sb8, ebuf[8 * c + k]);
                        const bool next = i - rs >= cols;
                        const float xv = xk[i - rs - (next ? cols : 0u)];
                        if (next) acc[1] = fmaf(w, xv, acc[1]);
                        else acc[0] = fmaf(w, xv, acc[0]);
                    }
                }
            }
        } else {
            // short rows (up to four per tile) or a tile that spans matrices:
            // element by element
            for (uint32_t i = P0 + lane; i < P1; i += 64) {
                const uint32_t k = matrix_of(d, i);
                const uint32_t rel = i - d.off[k];
                const uint32_t q = div_cols(d, k, rel);
                const uint32_t idx = d.row0[k] + q - ra;
                const float w = bf16_value(a.sm[i], ebuf[i - A0]);
                const float xv = x[d.x_off[k] + rel - q * d.cols[k]];
#pragma unroll
                for (uint32_t r = 0; r < kRowsPerTile; r++)
                    if (idx == r) acc[r] = fmaf(w, xv, acc[r]);
            }
        }
        // the row sums of the rows the tile touches; lanes 0..3 store them
        float mine = 0.0f;
#pragma unroll
        for (uint32_t i = 0; i < kRowsPerTile; i++) {
            if (i < nrows) {
                const float s = wave_sum_f(acc[i]);
                if (lane == i) mine = s;
            }
        }
        if (lane < kRowsPerTile) pt[lane] = mine;
        if (lane == 0) row_a[tile] = ra;
    }
};

__global__ __launch_bounds__(kThreads, 8) void df11_decode_gemv(KArgs a, GemvDesc d, const float *x,
                                                             float *part, uint32_t *row_a) {
    GemvEpi epi{&d, x, part, row_a};
    wave_tiles<4, DF11_FORMAT_BF16>(a, epi);
}

// The tile holding unit element e: the largest t with bop[t] <= e, given
// bop[lo] <= e < bop[hi].  Output positions grow almost linearly with the
// tile index within a matrix, so each step probes where e falls by linear
// interpolation, and every other step halves the range (at most twice the
// steps of a plain bisection on any input).
__device__ __forceinline__ uint32_t tile_of(const uint32_t *bop, uint32_t e, uint32_t lo,
                                            uint32_t hi) {
    uint32_t blo = bop[lo], bhi = bop[hi];
    for (uint32_t step = 0; hi - lo > 1; step++) {
        uint32_t mid = lo + (hi - lo) / 2;
        if ((step & 1) == 0 && bhi > blo) {
            const uint64_t f = uint64_t(e - blo) * (hi - lo) / (bhi - blo);
            mid = lo + uint32_t(f);
            mid = mid <= lo ? lo + 1 : mid >= hi ? hi - 1 : mid;
        }
        const uint32_t bm = bop[mid];
        if (bm <= e) {
            lo = mid;
            blo = bm;
        } else {
            hi = mid;
            bhi = bm;
        }
    }
    return lo;
}

// y for every row: the sums of the tiles that hold it, in tile order.
__global__ __launch_bounds__(kThreads) void df11_gemv_rows(GemvDesc d, const uint32_t *bop,
                                                           uint32_t n_tiles, const float *part,
                                                           const uint32_t *row_a, float *y) {
    const uint32_t r = blockIdx.x * kThreads + threadIdx.x;
    if (r >= d.row0[d.n]) return;
    uint32_t k = 0;
    while (k + 1 < d.n && r >= d.row0[k + 1]) k++;
    const uint32_t rs = d.off[k] + (r - d.row0[k]) * d.cols[k], re = rs + d.cols[k] - 1;
    // bop[0] = 0 <= rs and re < N = bop[n_tiles] for a valid unit; a corrupt
    // bop only yields other (wrong) tiles in [0, n_tiles)
    const uint32_t t0 = bop[n_tiles] > rs ? tile_of(bop, rs, 0, n_tiles) : n_tiles - 1;
    // the last tile of the row is a few tiles further: widen by doubling
    uint32_t lo = t0, span = 1;
    while (lo + span < n_tiles && bop[lo + span] <= re) {
        lo += span;
        span *= 2;
    }
    const uint32_t t1 = lo + span < n_tiles ? tile_of(bop, re, lo, lo + span)
                                            : (bop[n_tiles] > re ? tile_of(bop, re, lo, n_tiles)
                                                                 : n_tiles - 1);
    // Tiles after t0 start inside the row (rs < bop[t] <= re), so the row is
    // their first: slot 0, and their loads do not wait for one another.
    // row_a of a tile skipped as corrupt was never written: t0's slot is
    // checked so that such a unit yields wrong sums (and its status), never
    // a read outside part.
    const uint32_t i0 = r - row_a[t0];
    float s = i0 < kRowsPerTile ? part[uint64_t(t0) * kRowsPerTile + i0] : 0.0f;
#pragma unroll 4
    for (uint32_t t = t0 + 1; t <= t1; t++) s += part[uint64_t(t) * kRowsPerTile];
    y[d.y_off[k] + (r - d.row0[k])] = s;
}

// ---------------------------------------------------------------- fused GEMM
//
// Y^T = X^T W^T for the matrices of a BF16 unit and n = 16 NB tokens, straight
// from the compressed stream, on the matrix cores.  The unit holds each
// matrix in GEMM order (df11_gemm_order): 16-row blocks, each as 32-column
// sub-blocks of 16 x 32 weights in the lane order of the A operand of
// v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, columns 8 (l / 16) .. +7), so
// lane l takes the sub-block's 8-weight chunk l and a wave reads a
// sub-block's sign+mantissa bytes and staged exponents contiguously.  The
// activations are first reordered the same way for the B operand (lane l:
// token l % 16 of a 16-token group, columns 8 (l / 16) .. +7 of the
// sub-block): per matrix, [32-column block][quarter][token][8], so 16
// neighbouring lanes read 256 contiguous bytes.  One workgroup owns one
// 16-row block: its four waves
// decode the tiles holding the block (the first and last are shared with
// the neighbouring blocks, and decoded by both), each wave accumulating its
// sub-blocks' products; weights of a chunk outside the tile are zeroed.  The
// four waves' sums are added in a fixed order at the end.

constexpr uint32_t kGemmPre = 4;  // sub-blocks whose sm bytes are loaded before the decode

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

struct GemmDesc {
    uint32_t n;
    uint32_t mb0[DF11_GEMV_MAX_TENSORS + 1];  // first row block of each matrix; n .. 16: the total
    uint32_t off[DF11_GEMV_MAX_TENSORS];      // first element of each matrix in the unit
    uint32_t rows[DF11_GEMV_MAX_TENSORS], cols[DF11_GEMV_MAX_TENSORS];
    uint32_t x_off[DF11_GEMV_MAX_TENSORS], y_off[DF11_GEMV_MAX_TENSORS];
    // reordered activations: 16-byte chunks ch0[k] .. ch0[k+1]-1 of the workspace
    uint32_t ch0[DF11_GEMV_MAX_TENSORS + 1];  // n .. 16: the total
    // K segments: a row block of matrix k is split into seg[k] runs of
    // sbl[k] 32-column sub-blocks (the last may be shorter), one workgroup
    // each, segment-major; with seg[k] > 1 the partial sums go to the
    // workspace at p_off[k] (float index, seg[k] slices of rows x tokens)
    uint32_t seg[DF11_GEMV_MAX_TENSORS], sbl[DF11_GEMV_MAX_TENSORS];
    uint32_t p_off[DF11_GEMV_MAX_TENSORS];
    // float4s of the split matrices' outputs: q0[k] .. q0[k+1]-1; n .. 16: the total
    uint32_t q0[DF11_GEMV_MAX_TENSORS + 1];
};

// The activations in the B operand's order: chunk j of matrix k's slice is
// tokens' columns [32 kb + 8 q, +8) with t = j % T, q = (j / T) % 4,
// kb = j / (4 T), T = 16 NB tokens.  One thread per 16-byte chunk.
__global__ __launch_bounds__(kThreads) void df11_gemm_x_order(GemmDesc g, uint32_t n_tok,
                                                              const uint16_t *x, uint16_t *xs) {
    const uint32_t j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= g.ch0[DF11_GEMV_MAX_TENSORS]) return;
    uint32_t k = 0;
#pragma unroll
    for (uint32_t m = 1; m <= DF11_GEMV_MAX_TENSORS; m++) k += uint32_t(j >= g.ch0[m]);
    const uint32_t r = j - g.ch0[k];
    const uint32_t t = r % n_tok, q = (r / n_tok) % 4, kb = r / (4 * n_tok);
    const uint4 v = *reinterpret_cast<const uint4 *>(x + g.x_off[k] + uint64_t(t) * g.cols[k] +
                                                     32 * kb + 8 * q);
    *reinterpret_cast<uint4 *>(xs + 8 * uint64_t(j)) = v;
}

template <int NB>
struct GemmEpi {
    static constexpr bool kSmv = false, kAlways = false;
    uint32_t e0, e1;    // the row block: unit elements [e0, e1)
    const uint16_t *xk;  // the matrix's reordered activations (chunk j at xk + 8 j)
    uint32_t cols;
    f32x4 acc[NB];
    uint2 pre[kGemmPre];  // sm bytes of the tile's first sub-blocks
    // B operands loaded before A is built (its work covers part of their
    // latency) with one 16-token group; after it with more, which keeps
    // fewer registers live (early: 16 tokens 3% faster, 32 tokens 2% slower)
    static constexpr bool kEarly = NB == 1;

    // the lane's chunk of sub-block sb (relative to the row block)
    __device__ __forceinline__ uint32_t chunk_at(uint32_t sb, uint32_t lane) const {
        return e0 + 512 * sb + 8 * lane;
    }

    __device__ __forceinline__ void prefetch(const KArgs &a, uint32_t P0, uint32_t P1,
                                             uint32_t lane) {
        const uint32_t lo = max(P0, e0), hi = min(P1, e1);
        const uint32_t sb0 = lo < hi ? (lo - e0) / 512 : 0;
#pragma unroll
        for (uint32_t s = 0; s < kGemmPre; s++) {
            // sub-blocks lie wholly inside [e0, e1), so the load stays below e1
            if (lo < hi && e0 + 512 * (sb0 + s) < hi)
                pre[s] = *reinterpret_cast<const uint2 *>(a.sm + chunk_at(sb0 + s, lane));
        }
    }

    // Sub-block sb of the row block from its sign+mantissa bytes S and the
    // staged exponents of weights A0 .. P1-1; weights outside [lo, hi) enter
    // as zeros.
    __device__ __forceinline__ void sub_block(const KArgs &a, uint32_t sb, uint2 S, uint32_t lo,
                                              uint32_t hi, uint32_t A0, const uint8_t *ebuf,
                                              uint32_t lane) {
        const uint32_t g = chunk_at(sb, lane);
        // chunk (4 sb + l / 16) * T + 16 nb + l % 16 of the reordered activations
        const uint16_t *xb = xk + 8 * ((4 * sb + (lane >> 4)) * (16 * NB) + (lane & 15u));
        uint4 bv[NB];
        if constexpr (kEarly) {
#pragma unroll
            for (int nb = 0; nb < NB; nb++) bv[nb] = *reinterpret_cast<const uint4 *>(xb + 8 * 16 * nb);
        }
        const uint32_t base = e0 + 512 * sb;
        uint2 E;
        if (base >= lo && base + 512 <= hi) {  // wave-uniform: the tile holds it all
            E = *reinterpret_cast<const uint2 *>(ebuf + (g - A0));
        } else {
            // held in part: a chunk wholly outside the tile reads a clamped
            // staging address; the sm and exponent bytes of the weights
            // outside [lo, hi) are cleared, which makes those weights zero
            E = *reinterpret_cast<const uint2 *>(ebuf + (g < A0 ? 0u : min(g - A0, a.exp_cap - 8)));
            const uint32_t ua = min(uint32_t(max(int32_t(lo - g), 0)), 8u);
            const uint32_t ub = min(uint32_t(max(int32_t(hi - g), 0)), 8u);
            const uint32_t wd = ub > ua ? ub - ua : 0u;
            const uint64_t m = wd >= 8 ? ~0ull : ((1ull << (8 * wd)) - 1) << ((8 * ua) & 63u);
            S.x &= uint32_t(m);
            S.y &= uint32_t(m >> 32);
            E.x &= uint32_t(m);
            E.y &= uint32_t(m >> 32);
        }
        uint32_t w[4];
        assemble4(S.x, E.x, w[0], w[1]);
        assemble4(S.y, E.y, w[2], w[3]);
        bf16x8 A;
        __builtin_memcpy(&A, w, 16);
        if constexpr (!kEarly) {
#pragma unroll
            for (int nb = 0; nb < NB; nb++) bv[nb] = *reinterpret_cast<const uint4 *>(xb + 8 * 16 * nb);
        }
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            bf16x8 B;
            __builtin_memcpy(&B, &bv[nb], 16);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[nb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x020, NB, 0);  // the NB vector-memory reads,
        __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);  // then the NB products
    }

    template <int JP, int FMT>
    __device__ __forceinline__ void tile(const KArgs &a, uint32_t, uint32_t P0, uint32_t P1,
                                         uint32_t A0, uint32_t, const uint2 (&)[JP],
                                         const uint8_t *, const uint8_t *ebuf, uint32_t lane) {
        const uint32_t lo = max(P0, e0), hi = min(P1, e1);
        if (lo >= hi) return;
        const uint32_t sbA = (lo - e0) / 512, sbB = (hi - 1 - e0) / 512;
        // the first kGemmPre sub-blocks' bytes were prefetched (from sbA)
#pragma unroll
        for (uint32_t s = 0; s < kGemmPre; s++) {
            if (sbA + s > sbB) return;
            sub_block(a, sbA + s, pre[s], lo, hi, A0, ebuf, lane);
        }
        for (uint32_t sb = sbA + kGemmPre; sb <= sbB; sb++)
            sub_block(a, sb, *reinterpret_cast<const uint2 *>(a.sm + chunk_at(sb, lane)), lo, hi, A0,
                      ebuf, lane);
    }
};

// Occupancy is held to that of the accumulators plus the decode's registers
// (8, 8, 7 and 6 waves per SIMD for 1-4 token groups; without the cap the
// compiler spent registers that cost a step in occupancy, 4% at 64 tokens).
// One workgroup per 16-row block and K segment (longest segments first, in
// the XCD-grouped order).  The segment's tiles are found in block_out_pos;
// each wave takes every fourth.  Matrices far wider than the narrowest had
// whole row blocks take up to 3.5 times as long as the rest (the 70B
// down projection), which left a tail of few, long workgroups.
template <int NB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NB <= 2 ? 8 : NB == 3 ? 7 : 6))) void df11_decode_gemm(KArgs a, GemmDesc g, const uint16_t *xs,
                                                             float *y, float *part) {
    const uint32_t mb = xcd_grouped(blockIdx.x);
    if (mb >= g.mb0[DF11_GEMV_MAX_TENSORS]) return;  // uniform: the grid is rounded up
    uint32_t k = 0;
#pragma unroll
    for (uint32_t m = 1; m <= DF11_GEMV_MAX_TENSORS; m++) k += uint32_t(mb >= g.mb0[m]);
    const uint32_t cols = g.cols[k], rows = g.rows[k], w = mb - g.mb0[k];
    const uint32_t sg = w / (rows / 16), rb = w - sg * (rows / 16);
    const uint32_t sbS = sg * g.sbl[k], sbE = min(sbS + g.sbl[k], cols / 32);
    GemmEpi<NB> epi;
    epi.e0 = g.off[k] + rb * 16 * cols + 512 * sbS;
    epi.e1 = g.off[k] + rb * 16 * cols + 512 * sbE;
    epi.xk = xs + 8 * (uint64_t(g.ch0[k]) + uint64_t(sbS) * 64 * NB);
    epi.cols = cols;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) epi.acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // tiles holding e0 and e1 - 1 (bop[0] = 0 <= e0 < e1 <= N = bop[n_tiles]
    // for a valid unit; a corrupt bop only yields other tiles in range)
    const uint32_t *bop = a.bop;
    const uint32_t nt = a.n_tiles;
    const uint32_t t0 = bop[nt] > epi.e0 ? tile_of(bop, epi.e0, 0, nt) : nt - 1;
    const uint32_t t1 = bop[nt] > epi.e1 - 1 && bop[t0] <= epi.e1 - 1
                            ? tile_of(bop, epi.e1 - 1, t0, nt)
                            : nt - 1;
    const uint32_t wid = threadIdx.x >> 6, lane = threadIdx.x & 63u;
    const uint32_t first = min(t0, t1);
    wave_tiles<4, DF11_FORMAT_BF16>(a, epi, first, max(t0, t1) - first + 1, wid, 4);

    // ((w0 + w1) + w2) + w3 through LDS, then y^T[token][row]: lane l holds
    // rows 4 (l / 16) .. +3 of token l % 16 of each 16-token group
    extern __shared__ __align__(16) uint8_t dyn[];
    f32x4 *red = reinterpret_cast<f32x4 *>(dyn);
    __syncthreads();
    if (wid > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) red[((wid - 1) * NB + nb) * 64 + lane] = epi.acc[nb];
    }
    __syncthreads();
    if (wid == 0) {
        float *yk = (g.seg[k] > 1 ? part + g.p_off[k] + uint64_t(sg) * 16 * NB * rows
                                  : y + g.y_off[k]) +
                    16 * rb + 4 * (lane >> 4);
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            f32x4 v = epi.acc[nb];
            v += red[(0 * NB + nb) * 64 + lane];
            v += red[(1 * NB + nb) * 64 + lane];
            v += red[(2 * NB + nb) * 64 + lane];
            *reinterpret_cast<f32x4 *>(yk + uint64_t(16 * nb + (lane & 15u)) * rows) = v;
        }
    }
}

// y of the split matrices: the sum of their K segments' partial sums, in
// segment order.  One thread per float4.
__global__ __launch_bounds__(kThreads) void df11_gemm_reduce(GemmDesc g, uint32_t n_tok,
                                                             const float *part, float *y) {
    const uint32_t j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= g.q0[DF11_GEMV_MAX_TENSORS]) return;
    uint32_t k = 0;
#pragma unroll
    for (uint32_t m = 1; m <= DF11_GEMV_MAX_TENSORS; m++) k += uint32_t(j >= g.q0[m]);
    const uint32_t r = 4 * (j - g.q0[k]);
    const uint64_t slice = uint64_t(n_tok) * g.rows[k];
    const float *p = part + g.p_off[k] + r;
    float4 v = *reinterpret_cast<const float4 *>(p);
    for (uint32_t s = 1; s < g.seg[k]; s++) {
        const float4 u = *reinterpret_cast<const float4 *>(p + s * slice);
        v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    *reinterpret_cast<float4 *>(y + g.y_off[k] + r) = v;
}

template <int NB>
const void *gemm_kernel() {
    return reinterpret_cast<const void *>(&df11_decode_gemm<NB>);
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Whether every tile of a 64-window unit fits JP prefetched chunk slots of
// CH outputs: a tile's chunks span at most max_tile_symbols + CH - 1 outputs.
bool fits_slots(uint32_t max_tile_symbols, uint32_t jp, uint32_t ch) {
    return max_tile_symbols + ch - 1 <= 64u * jp * ch;
}

// FP8 units whose tiles fit two chunk slots take the fixed-store kernel
// (2.7% faster on the 70B block); BF16 units measured 1% slower with it
// than with exec-masked plain stores, and keep those.
template <int FMT>
const void *wave_kernel(uint32_t max_tile_symbols) {
    constexpr int JP = FMT == DF11_FORMAT_BF16 ? 4 : 2;
    if (FMT != DF11_FORMAT_BF16 && fits_slots(max_tile_symbols, JP, OutFmt<FMT>::kChunk))
        return reinterpret_cast<const void *>(&df11_decode_wave_fixed<JP, FMT>);
    return reinterpret_cast<const void *>(&df11_decode_wave<JP, FMT>);
}

const void *kernel_for(uint32_t tile_windows, uint32_t format, uint32_t max_tile_symbols) {
    if (format == DF11_FORMAT_FP8_E4M3) return wave_kernel<DF11_FORMAT_FP8_E4M3>(max_tile_symbols);
    if (format == DF11_FORMAT_FP8_E5M2) return wave_kernel<DF11_FORMAT_FP8_E5M2>(max_tile_symbols);
    if (tile_windows == 64) return wave_kernel<DF11_FORMAT_BF16>(max_tile_symbols);
    return tile_windows == 256 ? reinterpret_cast<const void *>(&df11_decode<1, 4>)
                               : reinterpret_cast<const void *>(&df11_decode<2, 8>);
}

// Outputs per 16-byte store: 8 BF16 or 16 FP8 values.
uint32_t chunk_outputs(uint32_t format) { return format == DF11_FORMAT_BF16 ? 8u : 16u; }

// Checks shared by both entry points; fills the launch-independent fields.
int prepare(const df11_device_stream *s, KArgs &a) {
    if (!s) return DF11_E_INVALID;
    if (s->window_bytes != 8 ||
        (s->tile_windows != 64 && s->tile_windows != 256 && s->tile_windows != 512))
        return DF11_E_INVALID;
    if (s->format > DF11_FORMAT_FP8_E5M2 ||
        (s->format != DF11_FORMAT_BF16 && s->tile_windows != 64))
        return DF11_E_INVALID;
    if (s->n_weights >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    const uint64_t tile_bits = uint64_t(64) * s->tile_windows;
    if (s->n_tiles != (s->total_bits + tile_bits - 1) / tile_bits) return DF11_E_INVALID;
    if (s->n_tiles >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    // an empty unit has no stream; a descriptor that claims tiles or bits for
    // it is inconsistent and must not reach a launch (its pointers may be null)
    if (s->n_weights == 0) return s->n_tiles == 0 && s->total_bits == 0 ? DF11_OK : DF11_E_INVALID;
    // every weight has a code of 1 .. 32 bits
    if (s->total_bits < s->n_weights || s->total_bits > uint64_t(DF11_MAX_CODE_LEN) * s->n_weights)
        return DF11_E_INVALID;
    if (!s->stream || !s->sm || !s->gaps || !s->block_out_pos || !s->tables)
        return DF11_E_INVALID;
    if (!aligned(s->stream, 16) || !aligned(s->sm, 16) || !aligned(s->tables, 16) ||
        !aligned(s->gaps, 2))
        return DF11_E_INVALID;
    if (s->n_luts < 1 || s->n_luts > DF11_MAX_LUTS) return DF11_E_INVALID;
    if (s->max_tile_symbols > 64u * s->tile_windows) return DF11_E_INVALID;
    a.stream = s->stream;
    a.sm = s->sm;
    a.gaps = s->gaps;
    a.bop = s->block_out_pos;
    a.tables = static_cast<const uint8_t *>(s->tables);
    a.total_bits = s->total_bits;
    a.n_weights = uint32_t(s->n_weights);
    // LDS holds tables 1 .. n_luts - 1; room for one is kept when there are
    // none, so that a walk on corrupt input still reads inside the allocation
    a.lut_last = s->n_luts > 1 ? s->n_luts - 1 : 1u;
    a.lds_tables = kLutOff + 512u * (s->n_luts - 1);
    // dynamic LDS: hierarchical tables, 16 bytes of wave totals (workgroup
    // tiles only), staging.  With 64-window tiles a Llama block then needs
    // 20,480 bytes per workgroup in all, so 8 workgroups fit in a CU's 160 KiB
    a.ebuf_off = 512u * a.lut_last + (s->tile_windows == 64 ? 0u : 16u);
    // outputs from P0 rounded down to a chunk to the last chunk, plus the 2 spill bytes
    const uint32_t chunk = chunk_outputs(s->format);
    a.exp_cap = (s->max_tile_symbols + (chunk - 1) + 16 + 15) & ~15u;
    return DF11_OK;
}

int launch(const df11_device_stream *s, KArgs &a, uint32_t n_tiles, hipStream_t st,
           uint32_t cap_per_cu = 0) {
    if (n_tiles == 0) return DF11_OK;
    a.n_tiles = n_tiles;
    // one staging buffer per workgroup, or one per wave for 64-window tiles
    const uint32_t per_wg = s->tile_windows == 64 ? 4u : 1u;
    const size_t lds = size_t(a.ebuf_off) + size_t(a.exp_cap) * per_wg;
    const void *fn = kernel_for(s->tile_windows, s->format, s->max_tile_symbols);
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_INVALID;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess)
        return DF11_E_HIP;
    if (per_cu < 1) return DF11_E_INVALID;
    const uint64_t resident = uint64_t(cus) * per_cu;
    const uint64_t slots = (uint64_t(n_tiles) + per_wg - 1) / per_wg;  // workgroups with a tile
    const uint64_t per = s->format == DF11_FORMAT_BF16 ? kTilesPerWorkgroup : kTilesPerWorkgroupFp8;
    uint64_t want = std::max<uint64_t>(resident, (slots + per - 1) / per);
    if (cap_per_cu) want = std::min<uint64_t>(want, uint64_t(cus) * std::min<uint32_t>(cap_per_cu, per_cu));
    const uint64_t used = std::min<uint64_t>(slots, want);
    const uint32_t grid = uint32_t((used + kXcdBlock - 1) / kXcdBlock * kXcdBlock);
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, st);
    return e == hipSuccess ? DF11_OK : DF11_E_HIP;
}

}  // namespace

int df11_detail::decompress_block_capped(const df11_device_stream *s, void *out,
                                         int32_t *d_status, hipStream_t st,
                                         uint32_t workgroups_per_cu) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK || s->n_weights == 0) return rc;
    if (!out || !aligned(out, 16)) return DF11_E_INVALID;
    a.out = out;
    a.status = d_status;
    a.tile0 = 0;
    a.out_lo = 0;
    a.out_hi = uint32_t(s->n_weights);
    a.out_shift = 0;
    return launch(s, a, uint32_t(s->n_tiles), st, workgroups_per_cu);
}

extern "C" {

int df11_decompress_block(const df11_device_stream *s, void *out, int32_t *d_status,
                          df11_hip_stream st) {
    return df11_detail::decompress_block_capped(s, out, d_status, static_cast<hipStream_t>(st), 0);
}

int df11_window_counts(const df11_device_stream *s, uint32_t *counts, df11_hip_stream st) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK) return rc;
    const uint64_t n = uint64_t(s->n_tiles) * s->tile_windows;
    if (n == 0) return DF11_OK;
    if (!counts || !aligned(counts, 4) || n >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    const void *fn = reinterpret_cast<const void *>(&df11_count_windows);
    const size_t lds = 512u * size_t(a.lut_last);
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_INVALID;
    const uint32_t nw = uint32_t(n);
    void *args[] = {&a, const_cast<uint32_t *>(&nw), &counts};
    return hipLaunchKernel(fn, dim3(uint32_t((n + kThreads - 1) / kThreads)), dim3(kThreads), args,
                           lds, static_cast<hipStream_t>(st)) == hipSuccess
               ? DF11_OK
               : DF11_E_HIP;
}

int df11_decompress_tensor(const df11_device_stream *s, uint32_t k, void *out,
                           int32_t *d_status, df11_hip_stream st) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK) return rc;
    if (k >= s->n_tensors || !s->tensor_offsets || !s->tensor_tiles) return DF11_E_INVALID;
    const uint64_t off = s->tensor_offsets[k], end = s->tensor_offsets[k + 1];
    if (end < off || end > s->n_weights || (off & (chunk_outputs(s->format) - 1)))
        return DF11_E_INVALID;
    if (end == off) return DF11_OK;
    if (!out || !aligned(out, 16)) return DF11_E_INVALID;
    const uint64_t t0 = s->tensor_tiles[2 * k], t1 = s->tensor_tiles[2 * k + 1];
    if (t1 < t0 || t1 > s->n_tiles) return DF11_E_INVALID;
    a.out = out;
    a.status = d_status;
    a.tile0 = uint32_t(t0);
    a.out_lo = uint32_t(off);
    a.out_hi = uint32_t(end);
    a.out_shift = uint32_t(off);
    return launch(s, a, uint32_t(t1 - t0), static_cast<hipStream_t>(st));
}

uint64_t df11_decompress_gemv_scratch_bytes(const df11_device_stream *s) {
    return s ? s->n_tiles * (4u * kRowsPerTile + 4u) + 256u : 0u;
}

}  // extern "C"

namespace {

// df11_decompress_gemv on a given workspace (the caller's, or the library's
// static one for df11_decompress_gemv_noalloc)
int gemv_impl(const df11_device_stream *s, const df11_gemv_tensor *t, uint32_t n_tensors,
              const float *x, float *y, void *scratch, uint64_t scratch_bytes, int32_t *d_status,
              df11_hip_stream st) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK) return rc;
    if (s->format != DF11_FORMAT_BF16 || s->tile_windows != 64 || s->n_weights == 0 || !t ||
        n_tensors == 0 || n_tensors > DF11_GEMV_MAX_TENSORS || !x || !y || !aligned(x, 16) ||
        !scratch || !aligned(scratch, 16) || scratch_bytes < df11_decompress_gemv_scratch_bytes(s))
        return DF11_E_INVALID;
    GemvDesc d{};
    d.n = n_tensors;
    uint64_t off = 0, row = 0;
    uint32_t min_cols = ~0u;
    for (uint32_t k = 0; k < n_tensors; k++) {
        // the matrices must tile the unit in order, with rows of whole 8-element chunks
        if (t[k].w_offset != off || t[k].cols == 0 || t[k].cols % 8 || t[k].x_offset % 4 ||
            t[k].rows == 0)
            return DF11_E_INVALID;
        d.off[k] = uint32_t(off);
        d.row0[k] = uint32_t(row);
        d.cols[k] = t[k].cols;
        d.inv[k] = uint32_t(((uint64_t(1) << 32) + t[k].cols - 1) / t[k].cols);
        d.x_off[k] = uint32_t(t[k].x_offset);
        d.y_off[k] = uint32_t(t[k].y_offset);
        if (t[k].x_offset >= (uint64_t(1) << 32) || t[k].y_offset >= (uint64_t(1) << 32))
            return DF11_E_INVALID;
        off += uint64_t(t[k].rows) * t[k].cols;
        row += t[k].rows;
        min_cols = std::min(min_cols, t[k].cols);
    }
    if (off != s->n_weights || row >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    for (uint32_t k = n_tensors; k <= DF11_GEMV_MAX_TENSORS; k++) d.off[k] = uint32_t(off);
    d.row0[n_tensors] = uint32_t(row);
    // a tile of M outputs touches at most (M - 1) / min_cols + 2 rows
    if (s->max_tile_symbols > 0 && (s->max_tile_symbols - 1) / min_cols + 2 > kRowsPerTile)
        return DF11_E_INVALID;
    float *part = static_cast<float *>(scratch);
    uint32_t *row_a = reinterpret_cast<uint32_t *>(part + s->n_tiles * kRowsPerTile);
    a.status = d_status;
    a.out_lo = 0;
    a.out_hi = uint32_t(s->n_weights);
    a.n_tiles = uint32_t(s->n_tiles);
    hipStream_t hs = static_cast<hipStream_t>(st);
    // the launch shape of the 64-window kernel (see launch())
    const size_t lds = size_t(a.ebuf_off) + size_t(a.exp_cap) * 4;
    const void *fn = reinterpret_cast<const void *>(&df11_decode_gemv);
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_INVALID;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess)
        return DF11_E_HIP;
    if (per_cu < 1) return DF11_E_INVALID;
    const uint64_t slots = (s->n_tiles + 3) / 4;
    const uint64_t want = std::max<uint64_t>(uint64_t(cus) * per_cu,
                                             (slots + kTilesPerWorkgroup - 1) / kTilesPerWorkgroup);
    const uint64_t used = std::min<uint64_t>(slots, want);
    const uint32_t grid = uint32_t((used + kXcdBlock - 1) / kXcdBlock * kXcdBlock);
    const float *xp = x;
    void *args[] = {&a, &d, &xp, &part, &row_a};
    if (hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, hs) != hipSuccess)
        return DF11_E_HIP;
    const uint32_t rows = uint32_t(row);
    return df11_detail::launch(df11_gemv_rows, dim3((rows + kThreads - 1) / kThreads),
                               dim3(kThreads), 0, hs, d, s->block_out_pos,
                               uint32_t(s->n_tiles), part, row_a, y) == hipSuccess
               ? DF11_OK
               : DF11_E_HIP;
}

// The workspace of df11_decompress_gemv_noalloc: per-tile row sums and first
// rows for up to DF11_GEMV_NOALLOC_MAX_TILES tiles.  In host code `scratch`
// names a host-side stand-in; kernels get its device address, looked up once
// per device.
constexpr uint64_t kNoAllocScratchBytes =
    uint64_t(DF11_GEMV_NOALLOC_MAX_TILES) * (4u * kRowsPerTile + 4u) + 256u;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// The device address of `scratch` on the current device.  The first call on
// a device asks the runtime for it (with that device current); later calls
// reuse it.  No memory is allocated: the array is part of the loaded code
// object on every device.
int scratch_on_current_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return DF11_E_INVALID;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DF11_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DF11_OK;
}

}  // namespace

extern "C" {

int df11_decompress_gemv(const df11_device_stream *s, const df11_gemv_tensor *t, uint32_t n_tensors,
                         const float *x, float *y, void *scratch_buf, uint64_t scratch_bytes,
                         int32_t *d_status, df11_hip_stream st) {
    return gemv_impl(s, t, n_tensors, x, y, scratch_buf, scratch_bytes, d_status, st);
}

int df11_decompress_gemv_noalloc(const df11_device_stream *s, const df11_gemv_tensor *t,
                                 uint32_t n_tensors, const float *x, float *y, int32_t *d_status,
                                 df11_hip_stream st) {
    if (s && s->n_tiles > DF11_GEMV_NOALLOC_MAX_TILES) return DF11_E_CAPACITY;
    if (s && s->n_weights && df11_decompress_gemv_scratch_bytes(s) > kNoAllocScratchBytes)
        return DF11_E_CAPACITY;
    // argument errors first, so that a rejected call touches no device state
    KArgs probe{};
    const int rc = prepare(s, probe);
    if (rc != DF11_OK) return rc;
    void *ws = nullptr;
    const int r2 = scratch_on_current_device(&ws);
    if (r2 != DF11_OK) return r2;
    return gemv_impl(s, t, n_tensors, x, y, ws, kNoAllocScratchBytes, d_status, st);
}

}  // extern "C"

namespace {
// K segments of matrix k's row blocks: row blocks of matrices much wider
// than the narrowest (at least 4096 columns) are split so that every
// workgroup decodes about as many weights
uint32_t gemm_segments(const df11_gemv_tensor *t, uint32_t n_tensors, uint32_t k) {
    uint32_t ref = ~0u;
    for (uint32_t i = 0; i < n_tensors; i++) ref = std::min(ref, t[i].cols);
    ref = std::max(ref, 4096u);
    return std::max(1u, (t[k].cols + ref - 1) / ref);
}
}  // namespace

extern "C" {

uint64_t df11_decompress_gemm_scratch_bytes(const df11_gemv_tensor *t, uint32_t n_tensors,
                                            uint32_t n_tokens) {
    if (!t && n_tensors) return 0;
    uint64_t b = 0;
    for (uint32_t k = 0; k < n_tensors; k++) b += 2ull * n_tokens * t[k].cols;
    b = (b + 15) / 16 * 16;
    for (uint32_t k = 0; k < n_tensors; k++) {
        const uint32_t sg = gemm_segments(t, n_tensors, k);
        if (sg > 1) b += 4ull * sg * n_tokens * t[k].rows;
    }
    return b;
}

int df11_decompress_gemm(const df11_device_stream *s, const df11_gemv_tensor *t, uint32_t n_tensors,
                         uint32_t n_tokens, const uint16_t *x, float *y, void *work,
                         uint64_t work_bytes, int32_t *d_status, df11_hip_stream st) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK) return rc;
    const uint32_t nb = n_tokens / 16;
    if (s->format != DF11_FORMAT_BF16 || s->tile_windows != 64 || s->n_weights == 0 || !t ||
        n_tensors == 0 || n_tensors > DF11_GEMV_MAX_TENSORS || n_tokens % 16 || nb < 1 || nb > 4 ||
        !x || !y || !work || !aligned(x, 16) || !aligned(y, 16) || !aligned(work, 16) ||
        work_bytes < df11_decompress_gemm_scratch_bytes(t, n_tensors, n_tokens))
        return DF11_E_INVALID;
    // longest segments first: their workgroups take the longest
    uint32_t order[DF11_GEMV_MAX_TENSORS], sbl[DF11_GEMV_MAX_TENSORS], seg[DF11_GEMV_MAX_TENSORS];
    for (uint32_t k = 0; k < n_tensors; k++) {
        order[k] = k;
        seg[k] = gemm_segments(t, n_tensors, k);
        sbl[k] = (t[k].cols / 32 + seg[k] - 1) / seg[k];
        seg[k] = (t[k].cols / 32 + sbl[k] - 1) / sbl[k];  // no empty segment
    }
    std::stable_sort(order, order + n_tensors,
                     [&sbl](uint32_t i, uint32_t j) { return sbl[i] > sbl[j]; });
    GemmDesc g{};
    g.n = n_tensors;
    uint64_t off = 0, mbs = 0, chunks = 0, pw = 0, q4 = 0;
    for (uint32_t k = 0; k < n_tensors; k++) {
        // in the unit the matrices follow one another in the caller's order
        if (t[k].w_offset != off || t[k].rows == 0 || t[k].rows % 16 || t[k].cols == 0 ||
            t[k].cols % 32 || t[k].x_offset % 8 || t[k].y_offset % 4)
            return DF11_E_INVALID;
        off += uint64_t(t[k].rows) * t[k].cols;
    }
    if (off != s->n_weights) return DF11_E_INVALID;
    for (uint32_t i = 0; i < n_tensors; i++) {
        const df11_gemv_tensor &d = t[order[i]];
        if (d.x_offset >= (uint64_t(1) << 32) || d.y_offset >= (uint64_t(1) << 32))
            return DF11_E_INVALID;
        g.mb0[i] = uint32_t(mbs);
        g.off[i] = uint32_t(d.w_offset);
        g.rows[i] = d.rows;
        g.cols[i] = d.cols;
        g.x_off[i] = uint32_t(d.x_offset);
        g.y_off[i] = uint32_t(d.y_offset);
        g.ch0[i] = uint32_t(chunks);
        g.seg[i] = seg[order[i]];
        g.sbl[i] = sbl[order[i]];
        g.p_off[i] = uint32_t(pw);
        g.q0[i] = uint32_t(q4);
        mbs += uint64_t(d.rows / 16) * g.seg[i];
        chunks += uint64_t(n_tokens) * d.cols / 8;
        if (g.seg[i] > 1) {
            pw += uint64_t(g.seg[i]) * n_tokens * d.rows;
            q4 += uint64_t(n_tokens) * d.rows / 4;
        }
    }
    if (chunks >= (uint64_t(1) << 32) || pw >= (uint64_t(1) << 32) || mbs >= (uint64_t(1) << 31))
        return DF11_E_INVALID;
    for (uint32_t k = n_tensors; k <= DF11_GEMV_MAX_TENSORS; k++) {
        g.mb0[k] = uint32_t(mbs);
        g.ch0[k] = uint32_t(chunks);
        g.q0[k] = uint32_t(q4);
    }
    a.status = d_status;
    a.out_lo = 0;
    a.out_hi = uint32_t(s->n_weights);
    a.n_tiles = uint32_t(s->n_tiles);
    // the tables and four staging buffers, then (reused) three waves' sums
    const size_t lds = std::max<size_t>(size_t(a.ebuf_off) + size_t(a.exp_cap) * 4, 3072u * nb);
    const void *fn = nb == 1 ? gemm_kernel<1>() : nb == 2 ? gemm_kernel<2>()
                   : nb == 3 ? gemm_kernel<3>() : gemm_kernel<4>();
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_INVALID;
    hipStream_t hs = static_cast<hipStream_t>(st);
    uint16_t *xs = static_cast<uint16_t *>(work);
    if (df11_detail::launch(df11_gemm_x_order, dim3(uint32_t((chunks + kThreads - 1) / kThreads)),
                            dim3(kThreads), 0, hs, g, n_tokens, x, xs) != hipSuccess)
        return DF11_E_HIP;
    const uint32_t grid = uint32_t((mbs + kXcdBlock - 1) / kXcdBlock * kXcdBlock);
    const uint16_t *xsp = xs;
    float *part = reinterpret_cast<float *>(static_cast<uint8_t *>(work) +
                                            (2 * chunks * 8 + 15) / 16 * 16);
    void *args[] = {&a, &g, &xsp, &y, &part};
    if (hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, hs) != hipSuccess)
        return DF11_E_HIP;
    if (q4 && df11_detail::launch(df11_gemm_reduce, dim3(uint32_t((q4 + kThreads - 1) / kThreads)),
                                  dim3(kThreads), 0, hs, g, n_tokens,
                                  static_cast<const float *>(part), y) != hipSuccess)
        return DF11_E_HIP;
    return DF11_OK;
}

}  // extern "C"
