// Device half of the DFloat11-style codec: the two-phase decode kernel for
// gfx950 and the df11_decompress_* entry points.
//
// What is computed follows "70% Size, 100% Accuracy ... (DFloat11)",
// abstract: hierarchical lookup tables in on-chip memory, a two-phase kernel
// in which auxiliary arrays fix every thread's read and write positions, and
// transformer-block-level launches; output is bit-identical BF16.  The layout
// of the kernel is this library's own.
//
// One workgroup of T threads decodes one tile of T*B stream bytes:
//   1. the lookup tables are copied to LDS;
//   2. thread t loads its B-byte window plus 4 look-ahead bytes (one coalesced
//      vector load) and its gap byte;
//   3. phase 1 walks the codes that start in the window and counts them;
//   4. a wave64 inclusive scan (cross-lane shuffles) plus an LDS pass over the
//      T/64 wave totals turns counts into write offsets; the tile total must
//      equal block_out_pos[t+1] - block_out_pos[t];
//   5. phase 2 walks the window again and writes each exponent byte to an
//      LDS staging buffer at its offset;
//   6. the tile's outputs are assembled 8 at a time from 8 sm bytes (global)
//      and 8 exponent bytes (LDS) and written with 16-byte stores.
#include <hip/hip_runtime.h>

#include "df11.h"

namespace {

constexpr int kThreads = 256;

struct KArgs {
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *bop;
    const uint16_t *lut;
    uint16_t *out;       // unit element i goes to out[i - out_shift]
    int32_t *status;
    uint64_t total_bits;
    uint64_t tile0;
    uint32_t n_luts;
    uint32_t exp_cap;    // bytes of LDS exponent staging
    uint32_t out_lo, out_hi, out_shift;
};

// Resolve the code at the head of a left-aligned 32-bit window.  Returns the
// leaf entry ((len << 8) | sym), or 0 when no leaf is reached in 4 levels.
__device__ __forceinline__ uint32_t lookup(const uint16_t *lut, uint32_t n_luts, uint32_t w32) {
    uint32_t e = lut[w32 >> 24];
    if (__builtin_expect((e & 0x8000u) != 0, 0)) {
#pragma unroll
        for (int lvl = 1; lvl < 4; lvl++) {
            const uint32_t tbl = min(e & 0x7FFFu, n_luts - 1);
            e = lut[(tbl << 8) | ((w32 >> (24 - 8 * lvl)) & 0xFFu)];
            if (!(e & 0x8000u)) break;
        }
        if (e & 0x8000u) e = 0;
    }
    return e;
}

// Walks the codes whose first bit lies in [gap, lim) of the thread's window.
// d[0..B/4] are the window's big-endian dwords plus one look-ahead dword.
// Segment s handles starts in [32s, 32s+32): the 32 bits at position p are
// alignbit((hi:lo) >> 1, 31 - p%32), valid for every p%32 including 0.
template <int B, bool kWrite>
__device__ __forceinline__ uint32_t walk(const uint32_t (&d)[B / 4 + 1], uint32_t gap,
                                         uint32_t lim, const uint16_t *lut, uint32_t n_luts,
                                         uint8_t *dst, bool &bad) {
    uint32_t p = gap, n = 0;
#pragma unroll
    for (int s = 0; s < B / 4; s++) {
        const uint32_t hi = d[s], lo = d[s + 1];
        const uint32_t a = hi >> 1;
        const uint32_t b = __builtin_amdgcn_alignbit(hi, lo, 1);
        const uint32_t end = min(32u * (s + 1), lim);
        while (p < end) {
            const uint32_t w32 = __builtin_amdgcn_alignbit(a, b, ~p);
            const uint32_t e = lookup(lut, n_luts, w32);
            const uint32_t len = (e >> 8) & 0x3Fu;
            if (len == 0) {
                bad = true;
                return n;
            }
            if (kWrite) dst[n] = uint8_t(e);
            n++;
            p += len;
        }
    }
    return n;
}

__device__ __forceinline__ uint32_t bf16_pair_lo(uint32_t S, uint32_t E) {
    // bytes of 4 outputs: high = (sm & 0x80) | (e >> 1), low = (e << 7 & 0x80) | (sm & 0x7F)
    const uint32_t H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);
    const uint32_t L = ((E << 7) & 0x80808080u) | (S & 0x7F7F7F7Fu);
    return __builtin_amdgcn_perm(H, L, 0x05010400u);
}

__device__ __forceinline__ uint32_t bf16_pair_hi(uint32_t S, uint32_t E) {
    const uint32_t H = (S & 0x80808080u) | ((E >> 1) & 0x7F7F7F7Fu);
    const uint32_t L = ((E << 7) & 0x80808080u) | (S & 0x7F7F7F7Fu);
    return __builtin_amdgcn_perm(H, L, 0x07030602u);
}

template <int T, int B>
__global__ __launch_bounds__(T) void df11_decode(KArgs a) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ uint32_t wave_sum[T / 64];
    uint16_t *lut = reinterpret_cast<uint16_t *>(lds);
    uint8_t *ebuf = lds + a.n_luts * 512u;

    const uint32_t t = threadIdx.x;
    const uint64_t tile = a.tile0 + blockIdx.x;
    const uint64_t win = tile * T + t;

    {  // 1. tables -> LDS
        const uint4 *src = reinterpret_cast<const uint4 *>(a.lut);
        uint4 *dst = reinterpret_cast<uint4 *>(lut);
        for (uint32_t i = t; i < a.n_luts * 32u; i += T) dst[i] = src[i];
    }

    // 2. window + look-ahead, byte-swapped so bit 0 of the stream is the MSB
    uint32_t d[B / 4 + 1];
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
#pragma unroll
    for (int k = 0; k <= B / 4; k++) d[k] = __builtin_bswap32(d[k]);
    const uint32_t gap = a.gaps[win];
    const uint64_t base = win * (8 * B);
    const uint32_t lim =
        a.total_bits > base ? uint32_t(min<uint64_t>(8 * B, a.total_bits - base)) : 0u;
    const uint32_t P0 = a.bop[tile], P1 = a.bop[tile + 1];
    __syncthreads();

    // 3. phase 1: count
    bool bad = false;
    const uint32_t cnt = walk<B, false>(d, gap, lim, lut, a.n_luts, nullptr, bad);

    // 4. scan
    const uint32_t lane = t & 63u, wid = t >> 6;
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= uint32_t(o)) incl += y;
    }
    if (lane == 63) wave_sum[wid] = incl;
    const int any_bad = __syncthreads_or(bad ? 1 : 0);
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < T / 64; k++) {
        const uint32_t v = wave_sum[k];
        before += (uint32_t(k) < wid) ? v : 0u;
        total += v;
    }
    const uint32_t head = P0 & 7u;
    if (any_bad || total != P1 - P0 || uint64_t(head) + total + 8 > a.exp_cap) {
        if (t == 0 && a.status) atomicExch(a.status, int32_t(DF11_E_CORRUPT));
        return;
    }

    // 5. phase 2: exponents -> LDS at their tile-relative output positions
    walk<B, true>(d, gap, lim, lut, a.n_luts, ebuf + head + before + incl - cnt, bad);
    __syncthreads();

    // 6. assemble and store, chunks of 8 aligned to the unit's element index
    const uint32_t lo = max(P0, a.out_lo), hi = min(P1, a.out_hi);
    if (lo >= hi) return;
    const uint32_t A0 = P0 & ~7u;
    const uint32_t nchunks = (P1 - A0 + 7) >> 3;
    for (uint32_t c = t; c < nchunks; c += T) {
        const uint32_t gi = A0 + 8 * c;
        if (gi >= lo && gi + 8 <= hi) {
            const uint2 s8 = *reinterpret_cast<const uint2 *>(a.sm + gi);
            const uint2 e8 = *reinterpret_cast<const uint2 *>(ebuf + 8 * c);
            uint4 v;
            v.x = bf16_pair_lo(s8.x, e8.x);
            v.y = bf16_pair_hi(s8.x, e8.x);
            v.z = bf16_pair_lo(s8.y, e8.y);
            v.w = bf16_pair_hi(s8.y, e8.y);
            *reinterpret_cast<uint4 *>(a.out + (gi - a.out_shift)) = v;
        } else {
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint32_t i = gi + k;
                if (i >= lo && i < hi) {
                    const uint32_t s = a.sm[i], e = ebuf[8 * c + k];
                    a.out[i - a.out_shift] = uint16_t(((s & 0x80u) << 8) | (e << 7) | (s & 0x7Fu));
                }
            }
        }
    }
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Checks shared by both entry points.  Fills the launch-independent fields.
int prepare(const df11_device_stream *s, KArgs &a) {
    if (!s) return DF11_E_INVALID;
    if (s->threads != kThreads || (s->bytes_per_thread != 8 && s->bytes_per_thread != 16))
        return DF11_E_INVALID;
    if (s->n_weights >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    const uint64_t tile_bits = uint64_t(8) * s->bytes_per_thread * s->threads;
    if (s->n_tiles != (s->total_bits + tile_bits - 1) / tile_bits) return DF11_E_INVALID;
    if (s->n_weights == 0) return DF11_OK;
    if (!s->stream || !s->sm || !s->gaps || !s->block_out_pos || !s->lut) return DF11_E_INVALID;
    if (!aligned(s->stream, 16) || !aligned(s->sm, 16) || !aligned(s->lut, 16))
        return DF11_E_INVALID;
    if (s->n_luts < 1 || s->n_luts > DF11_MAX_LUTS) return DF11_E_INVALID;
    if (s->max_tile_symbols > 8u * s->bytes_per_thread * s->threads) return DF11_E_INVALID;
    a.stream = s->stream;
    a.sm = s->sm;
    a.gaps = s->gaps;
    a.bop = s->block_out_pos;
    a.lut = s->lut;
    a.total_bits = s->total_bits;
    a.n_luts = s->n_luts;
    a.exp_cap = (s->max_tile_symbols + 7 + 8 + 15) & ~15u;
    return DF11_OK;
}

int launch(const df11_device_stream *s, const KArgs &a, uint64_t n_tiles, hipStream_t st) {
    if (n_tiles == 0) return DF11_OK;
    if (n_tiles > 0xFFFFFFFFull) return DF11_E_INVALID;
    const size_t lds = size_t(a.n_luts) * 512 + a.exp_cap;
    if (lds > 65536) return DF11_E_INVALID;
    const void *fn = s->bytes_per_thread == 8
                         ? reinterpret_cast<const void *>(&df11_decode<kThreads, 8>)
                         : reinterpret_cast<const void *>(&df11_decode<kThreads, 16>);
    void *args[] = {const_cast<KArgs *>(&a)};
    const hipError_t e =
        hipLaunchKernel(fn, dim3(uint32_t(n_tiles)), dim3(kThreads), args, lds, st);
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
    return launch(s, a, s->n_tiles, static_cast<hipStream_t>(st));
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
    a.tile0 = t0;
    a.out_lo = uint32_t(off);
    a.out_hi = uint32_t(end);
    a.out_shift = uint32_t(off);
    return launch(s, a, t1 - t0, static_cast<hipStream_t>(st));
}

}  // extern "C"
