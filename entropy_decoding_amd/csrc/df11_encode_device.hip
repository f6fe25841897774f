// GPU-side encoder for units whose weights are already in device memory.
//
// "70% Size, 100% Accuracy ... (DFloat11)", abstract, and "Compressing LLMs
// without Compromise", "Three ways to spend the savings": the exponents are
// entropy-coded with codes chosen from their frequencies.  The histogram runs
// here, the code construction on the host (df11_build_codebook_from_counts),
// and the stream, sign+mantissa array, gaps and block_out_pos are written
// here with exactly the bytes df11_encode writes.
//
// Work split: a workgroup encodes 4096 consecutive weights (16 per thread).
//   1. bits per workgroup;
//   2. their exclusive scan gives each workgroup's start bit (three launches);
//   3. every workgroup recomputes its threads' start bits (block scan), ORs
//      its codes into a bit buffer in LDS and writes it out: words that only
//      it touches with plain stores, its share of a word it shares with a
//      neighbour (its first or last word, when the group boundary falls
//      inside a word) into a side array; each code start that is the first
//      in its window writes the window's gap, and each code start that is
//      the first in its tile writes that tile's output position.  A thread
//      shifts each half of its 16 codes into a 64-bit register pair (with a
//      second pair marking where each code starts), ORs the half into LDS as
//      three words, and finds the window and tile starts in its half from
//      the marks; halves longer than 64 bits, partial groups and codebooks
//      with codes over 27 bits take the codes one at a time;
//   4. one thread per group boundary inside a word ORs the two shares and
//      writes that word (device-wide atomic ORs on the shared words instead
//      made the encode 35% slower), and the largest tile symbol count.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "df11.h"
#include "df11_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kPerThread = 16;
constexpr uint32_t kPerGroup = kThreads * kPerThread;  // weights per workgroup

struct Codes {
    uint32_t code[256];
    uint8_t len[256];
};

// symbol and sign+mantissa field of element i (FP8 field: a nibble)
template <int FMT>
struct Fields;
template <>
struct Fields<DF11_FORMAT_BF16> {
    using T = uint16_t;
    static __device__ __forceinline__ uint32_t sym(uint32_t x) { return (x >> 7) & 0xFFu; }
    static __device__ __forceinline__ uint32_t rest(uint32_t x) {
        return ((x >> 8) & 0x80u) | (x & 0x7Fu);
    }
};
template <>
struct Fields<DF11_FORMAT_FP8_E4M3> {
    using T = uint8_t;
    static __device__ __forceinline__ uint32_t sym(uint32_t x) { return (x >> 3) & 0xFu; }
    static __device__ __forceinline__ uint32_t rest(uint32_t x) { return ((x >> 4) & 0x8u) | (x & 0x7u); }
};
template <>
struct Fields<DF11_FORMAT_FP8_E5M2> {
    using T = uint8_t;
    static __device__ __forceinline__ uint32_t sym(uint32_t x) { return (x >> 2) & 0x1Fu; }
    static __device__ __forceinline__ uint32_t rest(uint32_t x) { return ((x >> 5) & 0x4u) | (x & 0x3u); }
};

// The thread's 16 elements (zero past n) and their count.
template <int FMT>
__device__ __forceinline__ uint32_t load16(const void *w, uint64_t n, uint64_t i0, uint32_t (&x)[16]) {
    using T = typename Fields<FMT>::T;
    const T *p = static_cast<const T *>(w) + i0;
    const uint32_t valid = i0 >= n ? 0u : uint32_t(min<uint64_t>(16, n - i0));
    if (valid == 16) {
        if constexpr (sizeof(T) == 2) {
            const uint4 a = reinterpret_cast<const uint4 *>(p)[0], b = reinterpret_cast<const uint4 *>(p)[1];
            const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int k = 0; k < 8; k++) {
                x[2 * k] = v[k] & 0xFFFFu;
                x[2 * k + 1] = v[k] >> 16;
            }
        } else {
            const uint4 a = *reinterpret_cast<const uint4 *>(p);
            const uint32_t v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int k = 0; k < 16; k++) x[k] = (v[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; k++) x[k] = uint32_t(k) < valid ? uint32_t(p[k]) : 0u;
    }
    return valid;
}

// The thread's 16 elements as loaded, packed (8 words for BF16, 4 for FP8;
// zero past n), and their count; element k is field k of the words.
template <int FMT>
struct Packed16 {
    using T = typename Fields<FMT>::T;
    static constexpr int kWords = sizeof(T) * 4;
    uint32_t w[kWords];
    __device__ __forceinline__ uint32_t load(const void *src, uint64_t n, uint64_t i0) {
        const T *p = static_cast<const T *>(src) + i0;
        const uint32_t valid = i0 >= n ? 0u : uint32_t(min<uint64_t>(16, n - i0));
        if (valid == 16) {
#pragma unroll
            for (int q = 0; q < kWords / 4; q++) {
                const uint4 v = reinterpret_cast<const uint4 *>(p)[q];
                w[4 * q] = v.x;
                w[4 * q + 1] = v.y;
                w[4 * q + 2] = v.z;
                w[4 * q + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < kWords; q++) w[q] = 0;
#pragma unroll
            for (int k = 0; k < 16; k++)
                if (uint32_t(k) < valid) w[k * sizeof(T) / 4] |= uint32_t(p[k]) << (8 * sizeof(T) * (k % (4 / sizeof(T))));
        }
        return valid;
    }
    __device__ __forceinline__ uint32_t elem(int k) const {
        constexpr int per = 4 / sizeof(T), bits = 8 * sizeof(T);
        return (w[k / per] >> (bits * (k % per))) & ((1u << bits) - 1u);
    }
};

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Exclusive prefix over the workgroup's threads and the workgroup total.
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t *wsum, uint32_t &total) {
    const uint32_t t = threadIdx.x, lane = t & 63u, wid = t >> 6;
    const uint32_t incl = wave_inclusive_scan(v);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (uint32_t k = 0; k < kThreads / 64; k++) {
        before += k < wid ? wsum[k] : 0u;
        total += wsum[k];
    }
    __syncthreads();
    return before + incl - v;
}

// ---------------------------------------------------------------- kernels

// Exponents are concentrated on a few values, so one LDS counter per symbol
// would take most atomics on a handful of addresses: lanes spread over
// kCopies copies of the histogram, laid out with a stride of kCopies + 1
// words per symbol so that the copies of one symbol sit in different banks.
constexpr uint32_t kCopies = 16;

template <int FMT>
__global__ __launch_bounds__(kThreads) void enc_histogram(const void *w, uint64_t n,
                                                          unsigned long long *counts) {
    __shared__ uint32_t h[256 * (kCopies + 1)];
    for (uint32_t s = threadIdx.x; s < 256 * (kCopies + 1); s += kThreads) h[s] = 0;
    __syncthreads();
    const uint32_t copy = threadIdx.x % kCopies;
    for (uint64_t i0 = (uint64_t(blockIdx.x) * kThreads + threadIdx.x) * 16; i0 < n;
         i0 += uint64_t(gridDim.x) * kThreads * 16) {
        uint32_t x[16];
        const uint32_t valid = load16<FMT>(w, n, i0, x);
#pragma unroll
        for (uint32_t k = 0; k < 16; k++)
            if (k < valid) atomicAdd(&h[Fields<FMT>::sym(x[k]) * (kCopies + 1) + copy], 1u);
    }
    __syncthreads();
    for (uint32_t s = threadIdx.x; s < 256; s += kThreads) {
        uint32_t c = 0;
        for (uint32_t k = 0; k < kCopies; k++) c += h[s * (kCopies + 1) + k];
        if (c) atomicAdd(&counts[s], (unsigned long long)c);
    }
}

__global__ __launch_bounds__(kThreads) void enc_fill(uint4 *p, uint64_t n16, uint4 v) {
    for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < n16;
         i += uint64_t(gridDim.x) * kThreads)
        p[i] = v;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void enc_group_bits(const void *w, uint64_t n, Codes cb,
                                                           uint32_t *group_bits) {
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ uint8_t len_s[256];
    for (uint32_t s = threadIdx.x; s < 256; s += kThreads) len_s[s] = cb.len[s];
    uint32_t x[16];
    const uint64_t i0 = uint64_t(blockIdx.x) * kPerGroup + uint64_t(threadIdx.x) * kPerThread;
    const uint32_t valid = load16<FMT>(w, n, i0, x);
    __syncthreads();
    uint32_t bits = 0;
#pragma unroll
    for (uint32_t k = 0; k < 16; k++) bits += k < valid ? len_s[Fields<FMT>::sym(x[k])] : 0u;
    uint32_t total;
    block_exclusive(bits, wsum, total);
    if (threadIdx.x == 0) group_bits[blockIdx.x] = total;
}

// start[g] = sum of group_bits[0 .. g), in three launches: sums of runs of
// 1024 entries, their exclusive scan (one workgroup), then each run's scan.
constexpr uint32_t kScanRun = 1024;

__device__ __forceinline__ uint64_t block_scan_u64(uint64_t v, uint64_t *part, uint64_t &total) {
    const uint32_t t = threadIdx.x;
    part[t] = v;
    __syncthreads();
    for (uint32_t off = 1; off < kScanRun; off <<= 1) {  // Hillis-Steele inclusive scan
        const uint64_t u = t >= off ? part[t - off] : 0ull;
        __syncthreads();
        part[t] += u;
        __syncthreads();
    }
    total = part[kScanRun - 1];
    return part[t] - v;  // exclusive
}

__global__ __launch_bounds__(kScanRun) void enc_run_sums(const uint32_t *group_bits, uint32_t n,
                                                         uint64_t *run_sum) {
    __shared__ uint64_t part[kScanRun];
    const uint32_t g = blockIdx.x * kScanRun + threadIdx.x;
    uint64_t total;
    block_scan_u64(g < n ? group_bits[g] : 0u, part, total);
    if (threadIdx.x == 0) run_sum[blockIdx.x] = total;
}

__global__ __launch_bounds__(kScanRun) void enc_scan_runs(uint64_t *run_sum, uint32_t n_runs) {
    __shared__ uint64_t part[kScanRun];
    uint64_t carry = 0;
    for (uint32_t r0 = 0; r0 < n_runs; r0 += kScanRun) {  // n_runs <= 1024 below 2^32 weights
        const uint32_t r = r0 + threadIdx.x;
        const uint64_t v = r < n_runs ? run_sum[r] : 0ull;
        uint64_t total;
        const uint64_t ex = block_scan_u64(v, part, total);
        if (r < n_runs) run_sum[r] = carry + ex;
        carry += total;
        __syncthreads();
    }
}

__global__ __launch_bounds__(kScanRun) void enc_scan_within(const uint32_t *group_bits, uint32_t n,
                                                            const uint64_t *run_start, uint64_t *start) {
    __shared__ uint64_t part[kScanRun];
    const uint32_t g = blockIdx.x * kScanRun + threadIdx.x;
    uint64_t total;
    const uint64_t ex = block_scan_u64(g < n ? group_bits[g] : 0u, part, total);
    if (g < n) start[g] = run_start[blockIdx.x] + ex;
}

struct EmitArgs {
    const void *w;
    uint64_t n;
    const uint64_t *start;  // per workgroup
    uint8_t *stream;
    uint8_t *sm;
    uint8_t *gaps;
    uint32_t *bop;
    uint64_t total_bits;
    uint64_t sm_bytes;
    uint32_t n_tiles;
    uint64_t n_groups;
    uint32_t *edge;           // per group: its shares of its first and last words
    uint32_t wshift, tshift;  // log2 of window and tile bits
    uint32_t buf_words;       // LDS bit-buffer words per workgroup
    Codes cb;
};

// Codes of at most this length leave the low 5 bits of the code left-aligned
// in 32 bits zero, so a fast-path table entry can hold the shift 32 - length
// there: ent = (code << (32 - length)) | (32 - length).
constexpr uint32_t kPackedMaxLen = 27;

// Bits [j0, j0 + 64) of the bit buffer (MSB first) ORed with the 64-bit
// string {hi, lo} placed at bit offset r: three words.
__device__ __forceinline__ void or_string64(uint32_t *buf, uint32_t r, uint32_t hi, uint32_t lo) {
    const uint32_t s = r & 31u, w = r >> 5;
    atomicOr(&buf[w], hi >> s);
    atomicOr(&buf[w + 1], __builtin_amdgcn_alignbit(hi, lo, s));
    atomicOr(&buf[w + 2], __builtin_amdgcn_alignbit(lo, 0u, s));
}

// Relative start p (from the half's first bit) of the first code that starts
// at or after relative position d (0 < d, and some code starts at or after
// it), from the start marks of a half of B bits (bit j of mark <=> a code
// starts at relative position B - 1 - j).
__device__ __forceinline__ uint32_t first_start_at(uint64_t mark, uint32_t B, uint32_t d) {
    const uint64_t m = mark & ((uint64_t(1) << (B - d)) - 1);  // starts at or after d
    return B - 1 - (63 - uint32_t(__clzll((long long)m)));
}

// Held to 80 VGPRs (6 waves per SIMD): uncapped the fast path took 90 and
// ran slower, and a 64-register cap spilled (70B block: 1.071, 1.041 and
// 1.006 ms for the encode call uncapped, at 64 and at 80).
template <int FMT, bool kPacked>
__global__ __launch_bounds__(kThreads, 6) void enc_emit(EmitArgs a) {
    extern __shared__ uint32_t buf[];  // the workgroup's bits, 32 per word, MSB first
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ uint32_t code_s[256];
    __shared__ uint32_t ent_s[256];
    __shared__ uint8_t len_s[256];
    const uint32_t t = threadIdx.x;
    for (uint32_t s = t; s < 256; s += kThreads) {
        const uint32_t l = a.cb.len[s];
        code_s[s] = a.cb.code[s];
        len_s[s] = uint8_t(l);
        ent_s[s] = (l && l <= kPackedMaxLen) ? (a.cb.code[s] << (32u - l)) | (32u - l) : 0u;
    }
    Packed16<FMT> xw;
    const uint64_t i0 = uint64_t(blockIdx.x) * kPerGroup + uint64_t(t) * kPerThread;
    const uint32_t valid = xw.load(a.w, a.n, i0);
    // sign and mantissa fields (zero past n, like the host encoder's padding),
    // formed now so that the weights need not stay unpacked
    uint32_t smw[4];
    if constexpr (FMT == DF11_FORMAT_BF16) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
            smw[q] = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) smw[q] |= Fields<FMT>::rest(xw.elem(4 * q + k)) << (8 * k);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 2; q++) {
            smw[q] = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) smw[q] |= Fields<FMT>::rest(xw.elem(8 * q + k)) << (4 * k);
        }
        smw[2] = smw[3] = 0;
    }
    __syncthreads();

    // Fast path: each half of 8 codes shifted into {hi, lo} (the string,
    // right-aligned) and {mh, ml} (a mark at each code's first bit) with
    // funnel shifts whose shift amount is the entry's own low 5 bits.  A half
    // fits when all 8 marks survive (it is at most 64 bits long).
    uint32_t hi[2] = {0, 0}, lo[2] = {0, 0}, mh[2] = {0, 0}, ml[2] = {0, 0};
    bool fast = kPacked && valid == 16;
    if (kPacked) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint32_t e = ent_s[Fields<FMT>::sym(xw.elem(8 * h + k))];
                hi[h] = __builtin_amdgcn_alignbit(hi[h], lo[h], e);
                lo[h] = __builtin_amdgcn_alignbit(lo[h], e, e);
                mh[h] = __builtin_amdgcn_alignbit(mh[h], ml[h], e);
                ml[h] = __builtin_amdgcn_alignbit(ml[h], 0x80000000u, e);
            }
            fast = fast && __popc(mh[h]) + __popc(ml[h]) == 8;
        }
    }
    uint32_t B[2] = {0, 0}, last_len[2] = {0, 0};
    uint32_t bits = 0;
    if (fast) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const uint64_t mark = (uint64_t(mh[h]) << 32) | ml[h];
            B[h] = 64u - uint32_t(__clzll((long long)mark));
            last_len[h] = uint32_t(__ffsll((unsigned long long)mark));  // the last code's mark is at bit length - 1
        }
        bits = B[0] + B[1];
    } else {
#pragma unroll
        for (uint32_t k = 0; k < 16; k++) bits += k < valid ? len_s[Fields<FMT>::sym(xw.elem(int(k)))] : 0u;
    }
    uint32_t total;
    const uint32_t before = block_exclusive(bits, wsum, total);
    const uint64_t g0 = a.start[blockIdx.x];   // first bit of the workgroup
    const uint64_t base = g0 & ~uint64_t(31);  // first bit of buf[0]
    const uint32_t nw = uint32_t((g0 + total - base + 31) >> 5);  // words holding its bits
    for (uint32_t i = t; i < nw + 3; i += kThreads) buf[i] = 0;
    __syncthreads();

    // The previous weight's code length decides whether a code is the first
    // to start in its window or tile: with a window (or tile) of W >= 32 bits,
    // the previous code started in an earlier one exactly when the start bit
    // modulo W is below that length.  The unit's first weight has no
    // predecessor; a length of 64 makes both tests true for it.  Positions are
    // kept relative to the workgroup (32 bits); the tests need only the low
    // bits of the absolute position.
    uint32_t prev_len = i0 == 0 ? 64u : 0u;
    if (i0 > 0 && i0 <= a.n) {
        using T = typename Fields<FMT>::T;
        prev_len = len_s[Fields<FMT>::sym(static_cast<const T *>(a.w)[i0 - 1])];
    }
    const uint32_t g0lo = uint32_t(g0), wmask = (1u << a.wshift) - 1, tmask = (1u << a.tshift) - 1;
    uint32_t r = before + (g0lo & 31u);  // start bit of the thread's next code, from base
    uint32_t last = r;                    // start of the thread's last code
    if (fast) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const uint64_t mark = (uint64_t(mh[h]) << 32) | ml[h];
            // the half's string left-aligned, then ORed in at bit r
            const uint64_t acc = ((uint64_t(hi[h]) << 32) | lo[h]) << (64u - B[h]);
            or_string64(buf, r, uint32_t(acc >> 32), uint32_t(acc));
            const uint32_t pl = (g0lo & ~31u) + r;  // low 32 bits of the half's absolute start
            const uint32_t span = B[h] - last_len[h];  // relative start of its last code
            const uint64_t at = base + r;
            // its first code, after the previous weight's code
            if ((pl & wmask) < prev_len) a.gaps[at >> a.wshift] = uint8_t(pl & wmask);
            if ((pl & tmask) < prev_len) a.bop[at >> a.tshift] = uint32_t(i0 + 8 * h);
            // window and tile boundaries after its first code start, up to its last
            const uint32_t nwin = ((pl & wmask) + span) >> a.wshift;
            for (uint32_t i = 1; i <= nwin; i++) {
                const uint32_t d = (i << a.wshift) - (pl & wmask);
                const uint32_t p = first_start_at(mark, B[h], d);
                a.gaps[(at >> a.wshift) + i] = uint8_t(p - d);
            }
            const uint32_t ntile = ((pl & tmask) + span) >> a.tshift;
            for (uint32_t i = 1; i <= ntile; i++) {
                const uint32_t d = (i << a.tshift) - (pl & tmask);
                const uint32_t p = first_start_at(mark, B[h], d);
                // codes of the half that start before p: the marks above p's
                const uint32_t k = uint32_t(__popcll((unsigned long long)(mark >> (B[h] - p))));
                a.bop[(at >> a.tshift) + i] = uint32_t(i0 + 8 * h + k);
            }
            last = r + span;
            prev_len = last_len[h];
            r += B[h];
        }
    } else {
#pragma unroll
        for (uint32_t k = 0; k < 16; k++) {
            if (k < valid) {
                const uint32_t s = Fields<FMT>::sym(xw.elem(int(k)));
                const uint32_t l = len_s[s], c = code_s[s];
                const uint32_t pl = (g0lo & ~31u) + r;  // low 32 bits of the absolute start bit
                if ((pl & wmask) < prev_len) {  // first code start in its window
                    const uint64_t pos = base + r;
                    a.gaps[pos >> a.wshift] = uint8_t(pos & wmask);
                }
                if ((pl & tmask) < prev_len) {  // first code start in its tile
                    const uint64_t pos = base + r;
                    a.bop[pos >> a.tshift] = uint32_t(i0 + k);
                }
                // the code, left-aligned at bit r % 32 of word r / 32, over two words
                const uint64_t v = uint64_t(c) << (64u - (r & 31u) - l);
                atomicOr(&buf[r >> 5], uint32_t(v >> 32));
                atomicOr(&buf[(r >> 5) + 1], uint32_t(v));
                last = r;
                prev_len = l;
                r += l;
            }
        }
    }
    if (valid && i0 + valid == a.n) {  // the last weight: tile boundaries after its start
        for (uint64_t b = ((base + last) >> a.tshift) + 1; b <= a.n_tiles; b++) a.bop[b] = uint32_t(a.n);
    }
    // sm_bytes is a multiple of 64, so a thread's 16 or 8 bytes are all inside or all outside
    if ((FMT == DF11_FORMAT_BF16 ? i0 : i0 / 2) < a.sm_bytes) {
        if constexpr (FMT == DF11_FORMAT_BF16)
            *reinterpret_cast<uint4 *>(a.sm + i0) = make_uint4(smw[0], smw[1], smw[2], smw[3]);
        else
            *reinterpret_cast<uint2 *>(a.sm + i0 / 2) = make_uint2(smw[0], smw[1]);
    }
    __syncthreads();
    // out: words touched only here with plain stores; a word shared with the
    // previous group (the group starts inside it) or the next one (it ends
    // inside it) goes to the side array, for enc_edges
    if (total) {
        const uint64_t grp = blockIdx.x;
        const bool lo_shared = (g0 & 31) != 0;
        const bool hi_shared = ((g0 + total) & 31) != 0 && grp + 1 < a.n_groups;
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.stream + (base >> 3));
        for (uint32_t i = t; i < nw; i += kThreads) {
            const uint32_t v = __builtin_bswap32(buf[i]);
            if (i == 0 && lo_shared)
                a.edge[2 * grp] = v;
            else if (i + 1 == nw && hi_shared)
                a.edge[2 * grp + 1] = v;
            else
                dst[i] = v;
        }
    }
}

// The words where a group boundary falls inside a word: the previous group's
// share (its last word) OR this group's share (its first word).
__global__ __launch_bounds__(kThreads) void enc_edges(const uint64_t *start, const uint32_t *edge,
                                                      uint64_t n_groups, uint8_t *stream) {
    for (uint64_t g = uint64_t(blockIdx.x) * kThreads + threadIdx.x + 1; g < n_groups;
         g += uint64_t(gridDim.x) * kThreads)
        if (start[g] & 31)
            reinterpret_cast<uint32_t *>(stream)[start[g] >> 5] = edge[2 * (g - 1) + 1] | edge[2 * g];
}

__global__ __launch_bounds__(kThreads) void enc_max_tile(const uint32_t *bop, uint32_t n_tiles,
                                                         uint32_t *out) {
    __shared__ uint32_t wmax[kThreads / 64];
    uint32_t m = 0;
    for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < n_tiles; b += gridDim.x * kThreads)
        m = max(m, bop[b + 1] - bop[b]);
    // reduce over the wave, then over the workgroup: one atomic per workgroup
    // (one per wave on a single address serialised: 48 us on the 70B block)
    for (int off = 32; off > 0; off >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), off, 64)));
    if ((threadIdx.x & 63u) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (uint32_t w = 1; w < kThreads / 64; w++) m = max(m, wmax[w]);
        if (m) atomicMax(out, m);
    }
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

int log2u(uint64_t x) {
    int r = 0;
    while ((uint64_t(1) << r) < x) r++;
    return r;
}

uint32_t grid_for(uint64_t items, uint64_t per_group, uint32_t cap) {
    return uint32_t(std::max<uint64_t>(1, std::min<uint64_t>(cap, (items + per_group - 1) / per_group)));
}

int launch_fill(void *p, uint64_t bytes, uint32_t byte_value, hipStream_t st) {
    if (!bytes) return DF11_OK;
    const uint32_t b = byte_value * 0x01010101u;
    const uint64_t n16 = bytes / 16;
    return df11_detail::launch(enc_fill, dim3(grid_for(n16, kThreads, 4096)), dim3(kThreads), 0, st,
                               static_cast<uint4 *>(p), n16, make_uint4(b, b, b, b)) == hipSuccess
               ? DF11_OK
               : DF11_E_HIP;
}

template <int FMT>
int encode_fmt(const df11_codebook *cb, const void *w, uint64_t n, const df11_sizes *sz,
               uint32_t T, uint32_t B, const df11_device_encode *o, hipStream_t st) {
    const uint64_t groups = (n + kPerGroup - 1) / kPerGroup;
    const uint32_t runs = uint32_t((groups + kScanRun - 1) / kScanRun);
    uint32_t *group_bits = static_cast<uint32_t *>(o->scratch);
    uint64_t *start = reinterpret_cast<uint64_t *>(
        static_cast<uint8_t *>(o->scratch) + ((groups * 4 + 255) & ~uint64_t(255)));
    uint64_t *run_sum = start + ((groups + 31) & ~uint64_t(31));
    uint32_t *edge = reinterpret_cast<uint32_t *>(run_sum + ((runs + 31) & ~uint32_t(31)));
    Codes c;
    for (int s = 0; s < 256; s++) {
        c.code[s] = cb->code[s];
        c.len[s] = cb->code_len[s];
    }
    // the stream's zero padding after the last word that holds bits (every
    // word before it is written later; the fill starts at the 16-byte
    // boundary below), gaps 255, the sm tail, the maximum
    const uint64_t pad0 = (sz->total_bits + 31) / 32 * 4 / 16 * 16;
    int rc = launch_fill(o->stream + pad0, sz->stream_bytes - pad0, 0, st);
    if (rc == DF11_OK) rc = launch_fill(o->gaps, sz->n_windows, 255, st);
    const uint64_t sm_done = FMT == DF11_FORMAT_BF16 ? groups * kPerGroup : groups * kPerGroup / 2;
    if (rc == DF11_OK && sz->sm_bytes > sm_done)  // past the last workgroup's weights
        rc = launch_fill(o->sm + sm_done, sz->sm_bytes - sm_done, 0, st);
    if (rc == DF11_OK) rc = launch_fill(o->d_max_tile_symbols, 16, 0, st);
    if (rc != DF11_OK) return rc;
    using df11_detail::launch;
    if (launch(enc_group_bits<FMT>, dim3(uint32_t(groups)), dim3(kThreads), 0, st, w, n, c,
               group_bits) != hipSuccess ||
        launch(enc_run_sums, dim3(runs), dim3(kScanRun), 0, st, group_bits, uint32_t(groups),
               run_sum) != hipSuccess ||
        launch(enc_scan_runs, dim3(1), dim3(kScanRun), 0, st, run_sum, runs) != hipSuccess ||
        launch(enc_scan_within, dim3(runs), dim3(kScanRun), 0, st, group_bits, uint32_t(groups),
               run_sum, start) != hipSuccess)
        return DF11_E_HIP;
    EmitArgs a{};
    a.w = w;
    a.n = n;
    a.start = start;
    a.stream = o->stream;
    a.sm = o->sm;
    a.gaps = o->gaps;
    a.bop = o->block_out_pos;
    a.total_bits = sz->total_bits;
    a.sm_bytes = sz->sm_bytes;
    a.n_tiles = uint32_t(sz->n_tiles);
    a.n_groups = groups;
    a.edge = edge;
    a.wshift = uint32_t(log2u(uint64_t(8) * B));
    a.tshift = a.wshift + uint32_t(log2u(T));
    a.buf_words = (kPerGroup * DF11_MAX_CODE_LEN + 31) / 32 + 4;
    a.cb = c;
    const size_t lds = size_t(a.buf_words) * 4;
    uint32_t max_len = 0;
    for (int s = 0; s < 256; s++) max_len = std::max<uint32_t>(max_len, cb->code_len[s]);
    auto *emit = max_len <= kPackedMaxLen ? enc_emit<FMT, true> : enc_emit<FMT, false>;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(emit),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
        return DF11_E_HIP;
    if (launch(emit, dim3(uint32_t(groups)), dim3(kThreads), lds, st, a) != hipSuccess ||
        (groups > 1 &&
         launch(enc_edges, dim3(grid_for(groups, kThreads, 1024)), dim3(kThreads), 0, st,
                static_cast<const uint64_t *>(start), static_cast<const uint32_t *>(edge), groups,
                o->stream) != hipSuccess) ||
        launch(enc_max_tile, dim3(grid_for(sz->n_tiles, kThreads, 256)), dim3(kThreads), 0, st,
               o->block_out_pos, uint32_t(sz->n_tiles), o->d_max_tile_symbols) != hipSuccess)
        return DF11_E_HIP;
    return DF11_OK;
}

}  // namespace

extern "C" {

int df11_histogram_device(uint32_t format, const void *w, uint64_t n, uint64_t *d_counts,
                          df11_hip_stream stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!d_counts || !aligned(d_counts, 16) || (n && (!w || !aligned(w, 16))) ||
        format > DF11_FORMAT_FP8_E5M2)
        return DF11_E_INVALID;
    int rc = launch_fill(d_counts, 256 * sizeof(uint64_t), 0, st);
    if (rc != DF11_OK || n == 0) return rc;
    const uint32_t grid = grid_for(n, uint64_t(kThreads) * 16 * 8, 4096);
    auto *c = reinterpret_cast<unsigned long long *>(d_counts);
    auto *k = format == DF11_FORMAT_BF16       ? enc_histogram<DF11_FORMAT_BF16>
              : format == DF11_FORMAT_FP8_E4M3 ? enc_histogram<DF11_FORMAT_FP8_E4M3>
                                               : enc_histogram<DF11_FORMAT_FP8_E5M2>;
    return df11_detail::launch(k, dim3(grid), dim3(kThreads), 0, st, w, n, c) == hipSuccess
               ? DF11_OK
               : DF11_E_HIP;
}

uint64_t df11_encode_device_scratch_bytes(uint64_t n_weights) {
    const uint64_t groups = (n_weights + kPerGroup - 1) / kPerGroup;
    const uint64_t runs = (groups + kScanRun - 1) / kScanRun;
    return ((groups * 4 + 255) & ~uint64_t(255)) + ((groups + 31) & ~uint64_t(31)) * 8 +
           ((runs + 31) & ~uint64_t(31)) * 8 + groups * 8 + 256;
}

int df11_encode_device(uint32_t format, const df11_codebook *cb, const void *w, uint64_t n,
                       uint32_t tile_windows, uint32_t window_bytes, const df11_sizes *sz,
                       const df11_device_encode *out, df11_hip_stream stream) {
    if (!cb || !sz || !out || format > DF11_FORMAT_FP8_E5M2) return DF11_E_INVALID;
    if (window_bytes != 8 || (tile_windows != 64 && tile_windows != 256 && tile_windows != 512) ||
        (format != DF11_FORMAT_BF16 && tile_windows != 64))
        return DF11_E_INVALID;
    if (n == 0 || n != sz->n_weights || n >= (uint64_t(1) << 32)) return DF11_E_INVALID;
    const uint64_t tile_bits = uint64_t(64) * tile_windows;
    if (sz->n_tiles != (sz->total_bits + tile_bits - 1) / tile_bits ||
        sz->n_windows != sz->n_tiles * tile_windows ||
        sz->stream_bytes != sz->n_tiles * tile_windows * 8 + DF11_STREAM_PAD)
        return DF11_E_INVALID;
    if (!w || !aligned(w, 16) || !out->stream || !aligned(out->stream, 16) || !out->sm ||
        !aligned(out->sm, 16) || !out->gaps || !aligned(out->gaps, 16) || !out->block_out_pos ||
        !out->d_max_tile_symbols || !aligned(out->d_max_tile_symbols, 16) || !out->scratch ||
        !aligned(out->scratch, 256) || out->scratch_bytes < df11_encode_device_scratch_bytes(n))
        return DF11_E_INVALID;
    if (sz->sm_bytes % 64 || sz->sm_bytes < (format == DF11_FORMAT_BF16 ? n : (n + 1) / 2) + 16)
        return DF11_E_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (format) {
    case DF11_FORMAT_BF16: return encode_fmt<DF11_FORMAT_BF16>(cb, w, n, sz, tile_windows, window_bytes, out, st);
    case DF11_FORMAT_FP8_E4M3: return encode_fmt<DF11_FORMAT_FP8_E4M3>(cb, w, n, sz, tile_windows, window_bytes, out, st);
    default: return encode_fmt<DF11_FORMAT_FP8_E5M2>(cb, w, n, sz, tile_windows, window_bytes, out, st);
    }
}

}  // extern "C"
