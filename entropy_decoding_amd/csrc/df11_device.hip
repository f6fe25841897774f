// Device half of the DFloat11-style codec: the two-phase decode kernel for
// gfx950 and the df11_decompress_* entry points.
//
// What is computed follows "70% Size, 100% Accuracy ... (DFloat11)",
// abstract: lookup tables held in on-chip memory, a two-phase kernel in which
// small auxiliary arrays fix every thread's read and write positions, and
// transformer-block-level launches; the output is bit-identical BF16.  The
// kernel's organisation is this library's own, for CDNA4:
//
// * A persistent grid (as many workgroups as fit on the device at once) walks
//   the tiles; each workgroup copies the tables into LDS once.
// * Per tile of T*B stream bytes, thread t owns window t:
//     - one vector load of its B bytes plus the 4 bytes after them, its gap
//       byte, and (issued early, consumed last) the sign+mantissa bytes of
//       the tile's outputs;
//     - phase 1 counts the codes that start in the window, several per step:
//       a 12-bit index into the count table gives the start offsets of every
//       code wholly inside those 12 bits as a bit mask, so a step adds the
//       popcount of the mask cut at the window's end;
//     - a wave64 inclusive scan in DPP row shifts and row broadcasts, then an
//       LDS pass over the T/64 wave totals, turns counts into offsets; the
//       tile total must equal block_out_pos[t+1] - block_out_pos[t];
//     - phase 2 walks the window again with a 10-bit index into the
//       multi-symbol table (up to 3 exponents per step) and writes exponent
//       bytes into an LDS staging buffer at their offsets; a step writes all 3
//       slots, so the last step may spill up to 2 bytes onto the next
//       thread's first two outputs, which every thread rewrites after a
//       barrier;
//     - the outputs are assembled 16 at a time from 16 sm bytes and 16
//       exponent bytes with byte permutes and written with 16-byte stores.
//   Codes longer than the fast tables' index walk the hierarchical 8-bit
//   tables (up to 4 levels for 32-bit codes).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "df11.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMultiOff = 0;                                        // uint32[1024]
constexpr uint32_t kCountOff = kMultiOff + 4u * (1u << DF11_MULTI_BITS);  // uint16[4096]
constexpr uint32_t kLutOff = kCountOff + 2u * (1u << DF11_COUNT_BITS);    // uint16[n][256]
constexpr uint32_t kBadCount = 1u << 20;  // added to a thread's count when its window is corrupt

struct KArgs {
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *bop;
    const uint8_t *tables;
    uint16_t *out;  // unit element i goes to out[i - out_shift]
    int32_t *status;
    uint64_t total_bits;
    uint32_t n_weights;
    uint32_t tile0, n_tiles;  // tiles [tile0, tile0 + n_tiles) of the unit
    uint32_t table_bytes;
    uint32_t ebuf_off;        // LDS byte offset of the exponent staging buffer
    uint32_t exp_cap;         // its size in bytes
    uint32_t n_luts;
    uint32_t out_lo, out_hi, out_shift;
};

// Hierarchical walk for one code at the head of a left-aligned 32-bit window.
// Returns (length << 8) | symbol, or 0 when no leaf is reached in 4 levels.
__device__ __forceinline__ uint32_t walk_tables(const uint16_t *lut, uint32_t n_luts,
                                                uint32_t w32) {
    uint32_t e = lut[w32 >> 24];
    if (e & 0x8000u) {
#pragma unroll
        for (int lvl = 1; lvl < 4; lvl++) {
            const uint32_t tbl = min(e & 0x7FFFu, n_luts - 1);
            e = lut[(tbl << 8) | ((w32 >> (24 - 8 * lvl)) & 0xFFu)];
            if (!(e & 0x8000u)) break;
        }
        if (e & 0x8000u) e = 0;
    }
    return e & 0x3FFFu;
}

// The 32 stream bits starting p bits into segment s of the window, for
// p % 32 in [0, 32): alignbit((hi:lo) >> 1, 31 - p % 32).  a = hi >> 1 and
// b = alignbit(hi, lo, 1) are formed once per segment.
template <int B>
struct Window {
    uint32_t a[B / 4], b[B / 4];
    __device__ __forceinline__ void init(const uint32_t (&d)[B / 4 + 1]) {
#pragma unroll
        for (int s = 0; s < B / 4; s++) {
            a[s] = d[s] >> 1;
            b[s] = __builtin_amdgcn_alignbit(d[s], d[s + 1], 1);
        }
    }
    // q = ~p: the shift 31 - p % 32 is q mod 32
    __device__ __forceinline__ uint32_t at(int s, uint32_t q) const {
        return __builtin_amdgcn_alignbit(a[s], b[s], q);
    }
    // any p < 64, segment chosen at run time (used for two codes per tile)
    __device__ __forceinline__ uint32_t at_low(uint32_t p) const {
        const uint32_t w0 = __builtin_amdgcn_alignbit(a[0], b[0], ~p);
        const uint32_t w1 = __builtin_amdgcn_alignbit(a[1], b[1], ~p);
        return p < 32 ? w0 : w1;
    }
};

// A multi-symbol step at window bits w32: the table entry, or for a first
// code longer than the index, an entry built from the hierarchical walk.
// Entry: bits 31..30 count, 29..24 total length, 23..0 symbols.
__device__ __forceinline__ uint32_t multi_step(const uint8_t *fast, const uint16_t *lut,
                                               uint32_t n_luts, uint32_t w32) {
    uint32_t e = *reinterpret_cast<const uint32_t *>(
        fast + kMultiOff + ((w32 >> (32 - DF11_MULTI_BITS)) << 2));
    if (e < (1u << 30)) {
        const uint32_t le = walk_tables(lut, n_luts, w32);
        uint32_t len = le >> 8;
        if (len == 0) len = 63;  // unreachable once phase 1 accepted the tile
        e = (1u << 30) | (len << 24) | (le & 0xFFu);
    }
    return e;
}

// Phase 1: number of codes whose first bit lies in [gap, lim) of the window.
// The loop carries q = ~p (alignbit takes 31 - p % 32 = ~p mod 32 directly).
template <int B>
__device__ __forceinline__ uint32_t count_codes(const Window<B> &W, uint32_t gap, uint32_t lim,
                                                const uint8_t *fast, const uint16_t *lut,
                                                uint32_t n_luts) {
    uint32_t q = ~gap, cnt = 0;
    const uint32_t lim1 = lim + 1;  // lim - p == lim1 + q
#pragma unroll
    for (int s = 0; s < B / 4; s++) {
        const uint32_t qend = ~min(32u * (s + 1), lim);  // p < end  <=>  q > ~end
        while (q > qend) {
            const uint32_t w32 = W.at(s, q);
            const uint32_t e = *reinterpret_cast<const uint16_t *>(
                fast + kCountOff + ((w32 >> (32 - DF11_COUNT_BITS)) << 1));
            uint32_t adv = e >> 12;
            uint32_t m = __builtin_amdgcn_ubfe(e, 0, min(lim1 + q, uint32_t(DF11_COUNT_BITS)));
            if (adv == 0) {  // first code longer than the index
                adv = walk_tables(lut, n_luts, w32) >> 8;
                m = 1;
                if (adv == 0) {  // no code here: corrupt stream or tables
                    adv = 8 * B;
                    cnt += kBadCount;
                }
            }
            cnt += __builtin_popcount(m);
            q -= adv;
        }
    }
    return cnt;
}

// Phase 2: exponents of the window's codes to dst[0 ..), up to 2 bytes beyond.
template <int B>
__device__ __forceinline__ void decode_codes(const Window<B> &W, uint32_t gap, uint32_t lim,
                                             const uint8_t *fast, const uint16_t *lut,
                                             uint32_t n_luts, uint8_t *dst) {
    uint32_t q = ~gap;
#pragma unroll
    for (int s = 0; s < B / 4; s++) {
        const uint32_t qend = ~min(32u * (s + 1), lim);
        while (q > qend) {
            const uint32_t e = multi_step(fast, lut, n_luts, W.at(s, q));
            dst[0] = uint8_t(e);
            dst[1] = uint8_t(e >> 8);
            dst[2] = uint8_t(e >> 16);
            dst += e >> 30;
            q -= (e >> 24) & 0x3Fu;
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

// Outputs [gi, gi + 8) of the unit from 8 sm bytes and staged exponents ex[0 .. 8).
__device__ __forceinline__ void emit8(const KArgs &a, uint32_t gi, uint32_t lo, uint32_t hi,
                                      uint2 s8, const uint8_t *ex) {
    if (gi >= lo && gi + 8 <= hi) {
        const uint2 e8 = *reinterpret_cast<const uint2 *>(ex);
        uint4 v;
        assemble4(s8.x, e8.x, v.x, v.y);
        assemble4(s8.y, e8.y, v.z, v.w);
        *reinterpret_cast<uint4 *>(a.out + (gi - a.out_shift)) = v;
    } else if (gi + 8 > lo && gi < hi) {
        for (uint32_t k = 0; k < 8; k++) {
            const uint32_t i = gi + k;
            if (i >= lo && i < hi) a.out[i - a.out_shift] = assemble1(a.sm[i], ex[k]);
        }
    }
}

// Per-tile inputs, loaded one tile ahead.  The tile bounds come through a
// vector load (lane l reads block_out_pos[tile + (l & 1)]): a scalar load
// would share its wait counter with LDS and stall the decode loops.
template <int T, int B>
struct TileIn {
    uint32_t d[B / 4 + 1];
    uint32_t gap, bounds;
    __device__ __forceinline__ void load(const KArgs &a, uint32_t tile, uint32_t t) {
        const uint64_t win = uint64_t(tile) * T + t;
        const uint8_t *wp = a.stream + win * B;
        if constexpr (B == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(wp);
            d[0] = v.x;
            d[1] = v.y;
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(wp);
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
        }
        d[B / 4] = *reinterpret_cast<const uint32_t *>(wp + B);
        gap = a.gaps[win];
        bounds = a.bop[tile + (t & 1u)];
    }
};

template <int T, int B, int JP>
__global__ __launch_bounds__(T) void df11_decode(KArgs a) {
    // The fixed-size fast tables are the kernel's only static LDS, at address
    // 0, so their offsets fold into the LDS instructions' immediate offsets.
    // Dynamic LDS: hierarchical tables, 16 bytes of wave totals, staging.
    __shared__ __align__(16) uint8_t fast[kLutOff];
    extern __shared__ __align__(16) uint8_t dyn[];
    static_assert(T == 256, "the block scan reads the 4 wave totals as one uint4");
    const uint32_t t = threadIdx.x, lane = t & 63u, wid = t >> 6;
    if (blockIdx.x >= a.n_tiles) return;

    TileIn<T, B> cur;
    cur.load(a, a.tile0 + blockIdx.x, t);
    for (uint32_t i = 16 * t; i < a.table_bytes; i += 16 * T) {
        const uint4 v = *reinterpret_cast<const uint4 *>(a.tables + i);
        *reinterpret_cast<uint4 *>(i < kLutOff ? fast + i : dyn + (i - kLutOff)) = v;
    }
    __syncthreads();
    const uint16_t *lut = reinterpret_cast<const uint16_t *>(dyn);
    uint32_t *wave_sum = reinterpret_cast<uint32_t *>(dyn + a.ebuf_off - 16);
    uint8_t *ebuf = dyn + a.ebuf_off;

    for (uint32_t it = blockIdx.x; it < a.n_tiles; it += gridDim.x) {
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
            const uint32_t c = t + j * T;
            if (c < n8) smv[j] = *reinterpret_cast<const uint2 *>(a.sm + A0 + 8 * c);
        }
        // next tile's inputs, issued before this tile's stores so that waiting
        // for them never waits for those stores
        TileIn<T, B> nxt;
        nxt.load(a, a.tile0 + min(it + gridDim.x, a.n_tiles - 1), t);

        uint32_t d[B / 4 + 1];
#pragma unroll
        for (int k = 0; k <= B / 4; k++) d[k] = __builtin_bswap32(cur.d[k]);
        Window<B> W;
        W.init(d);
        const uint32_t gap = cur.gap;
        const uint64_t base = (uint64_t(tile) * T + t) * (8 * B);
        const uint32_t lim =
            a.total_bits > base ? uint32_t(min<uint64_t>(8 * B, a.total_bits - base)) : 0u;

        // phase 1 and the block scan
        const uint32_t cnt = count_codes<B>(W, gap, lim, fast, lut, a.n_luts);
        const uint32_t incl = wave_inclusive_scan(cnt);
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

        // phase 2, then repair the two bytes a neighbour's last step may have spilled onto
        uint8_t *mine = ebuf + (P0 - A0) + before + incl - cnt;
        decode_codes<B>(W, gap, lim, fast, lut, a.n_luts, mine);
        __syncthreads();
        if (cnt) {
            uint32_t e = multi_step(fast, lut, a.n_luts, W.at_low(gap));
            mine[0] = uint8_t(e);
            if (cnt > 1) {
                if ((e >> 30) < 2)
                    e = multi_step(fast, lut, a.n_luts, W.at_low(gap + ((e >> 24) & 0x3Fu)));
                else
                    e >>= 8;
                mine[1] = uint8_t(e);
            }
        }
        __syncthreads();

        // assemble and store: for each j, the lanes of a wave write 1 KiB contiguously
        const uint32_t lo = max(P0, a.out_lo), hi = min(P1, a.out_hi);
#pragma unroll
        for (int j = 0; j < JP; j++) {
            const uint32_t c = t + j * T;
            if (c < n8) emit8(a, A0 + 8 * c, lo, hi, smv[j], ebuf + 8 * c);
        }
        for (uint32_t c = t + JP * T; c < n8; c += T)
            emit8(a, A0 + 8 * c, lo, hi, *reinterpret_cast<const uint2 *>(a.sm + A0 + 8 * c),
                  ebuf + 8 * c);
        cur = nxt;
    }
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

template <int B>
const void *kernel_for() {
    return reinterpret_cast<const void *>(&df11_decode<kThreads, B, (B == 8 ? 4 : 8)>);
}

// Checks shared by both entry points; fills the launch-independent fields.
int prepare(const df11_device_stream *s, KArgs &a) {
    if (!s) return DF11_E_INVALID;
    if (s->threads != kThreads || (s->bytes_per_thread != 8 && s->bytes_per_thread != 16))
        return DF11_E_INVALID;
    if (s->n_weights >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    const uint64_t tile_bits = uint64_t(8) * s->bytes_per_thread * s->threads;
    if (s->n_tiles != (s->total_bits + tile_bits - 1) / tile_bits) return DF11_E_INVALID;
    if (s->n_tiles >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    if (s->n_weights == 0) return DF11_OK;
    if (!s->stream || !s->sm || !s->gaps || !s->block_out_pos || !s->tables)
        return DF11_E_INVALID;
    if (!aligned(s->stream, 16) || !aligned(s->sm, 16) || !aligned(s->tables, 16))
        return DF11_E_INVALID;
    if (s->n_luts < 1 || s->n_luts > DF11_MAX_LUTS) return DF11_E_INVALID;
    if (s->max_tile_symbols > 8u * s->bytes_per_thread * s->threads) return DF11_E_INVALID;
    a.stream = s->stream;
    a.sm = s->sm;
    a.gaps = s->gaps;
    a.bop = s->block_out_pos;
    a.tables = static_cast<const uint8_t *>(s->tables);
    a.total_bits = s->total_bits;
    a.n_weights = uint32_t(s->n_weights);
    a.n_luts = s->n_luts;
    a.table_bytes = kLutOff + 512u * s->n_luts;
    // dynamic LDS: hierarchical tables, 16 bytes of wave totals, then staging
    a.ebuf_off = 512u * s->n_luts + 16;
    // outputs from P0 & ~7 to the last 8-chunk, plus the 2 spill bytes
    a.exp_cap = (s->max_tile_symbols + 7 + 16 + 15) & ~15u;
    return DF11_OK;
}

int launch(const df11_device_stream *s, KArgs &a, uint32_t n_tiles, hipStream_t st) {
    if (n_tiles == 0) return DF11_OK;
    a.n_tiles = n_tiles;
    const size_t lds = size_t(a.ebuf_off) + a.exp_cap;
    const void *fn = s->bytes_per_thread == 8 ? kernel_for<8>() : kernel_for<16>();
    if (lds > 65536 &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_INVALID;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess)
        return DF11_E_HIP;
    if (per_cu < 1) return DF11_E_INVALID;
    const uint32_t grid = uint32_t(std::min<uint64_t>(n_tiles, uint64_t(cus) * per_cu));
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, lds, st);
    return e == hipSuccess ? DF11_OK : DF11_E_HIP;
}

}  // namespace

extern "C" {

int df11_decompress_block(const df11_device_stream *s, uint16_t *out, int32_t *d_status,
                          df11_hip_stream st) {
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
    return launch(s, a, uint32_t(s->n_tiles), static_cast<hipStream_t>(st));
}

int df11_decompress_tensor(const df11_device_stream *s, uint32_t k, uint16_t *out,
                           int32_t *d_status, df11_hip_stream st) {
    KArgs a{};
    int rc = prepare(s, a);
    if (rc != DF11_OK) return rc;
    if (k >= s->n_tensors || !s->tensor_offsets || !s->tensor_tiles) return DF11_E_INVALID;
    const uint64_t off = s->tensor_offsets[k], end = s->tensor_offsets[k + 1];
    if (end < off || end > s->n_weights || (off & 7)) return DF11_E_INVALID;
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

}  // extern "C"
