// Host half of the DFloat11-style codec: codebook construction and the
// offline encoder ("70% Size, 100% Accuracy ... (DFloat11)", abstract:
// frequency-based dynamic-length codes; "Compressing LLMs without
// Compromise", "Three ways to spend the savings": exponents are
// Huffman-coded offline).  Stream format and ABI: include/df11.h.
#include "df11.h"

#include <algorithm>
#include <functional>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <thread>
#include <vector>

namespace {

constexpr int kSyms = 256;
constexpr uint64_t kChunk = uint64_t(1) << 22;  // weights per encoder work item

unsigned worker_count() {
    if (const char *e = std::getenv("DF11_HOST_THREADS")) {
        int v = std::atoi(e);
        if (v > 0) return unsigned(v);
    }
    unsigned hc = std::thread::hardware_concurrency();
    return std::max(1u, std::min(16u, hc ? hc : 1u));
}

// Runs f(i) for i in [0, n) on up to worker_count() threads.
template <class F>
void parallel_for(size_t n, F &&f) {
    size_t nt = std::min<size_t>(n, worker_count());
    if (nt <= 1) {
        for (size_t i = 0; i < n; i++) f(i);
        return;
    }
    std::atomic<size_t> next{0};
    auto body = [&] {
        for (size_t i; (i = next.fetch_add(1, std::memory_order_relaxed)) < n;) f(i);
    };
    std::vector<std::thread> pool;
    pool.reserve(nt - 1);
    for (size_t t = 0; t + 1 < nt; t++) pool.emplace_back(body);
    body();
    for (auto &th : pool) th.join();
}

// Weight formats.  The coded symbol is the exponent field; the sign and
// mantissa are stored raw: one byte per BF16 weight, one nibble per FP8
// weight (sign just above the mantissa, two per byte, lower index in the low
// nibble).
struct BF16 {
    using T = uint16_t;
    static constexpr bool kNibbles = false;
    static uint32_t sym(T x) { return (x >> 7) & 0xFF; }
    static uint32_t rest(T x) { return ((x >> 8) & 0x80) | (x & 0x7F); }
};
struct E4M3 {
    using T = uint8_t;
    static constexpr bool kNibbles = true;
    static uint32_t sym(T x) { return (x >> 3) & 0xF; }
    static uint32_t rest(T x) { return ((x >> 4) & 0x8) | (x & 0x7); }
};
struct E5M2 {
    using T = uint8_t;
    static constexpr bool kNibbles = true;
    static uint32_t sym(T x) { return (x >> 2) & 0x1F; }
    static uint32_t rest(T x) { return ((x >> 5) & 0x4) | (x & 0x3); }
};

// Calls f with the traits of a format; false for an unknown format.
template <class F>
bool with_format(uint32_t format, F &&f) {
    switch (format) {
    case DF11_FORMAT_BF16: f(BF16{}); return true;
    case DF11_FORMAT_FP8_E4M3: f(E4M3{}); return true;
    case DF11_FORMAT_FP8_E5M2: f(E5M2{}); return true;
    default: return false;
    }
}

uint32_t element_bytes(uint32_t format) { return format == DF11_FORMAT_BF16 ? 2u : 1u; }

struct Piece {
    const void *w;   // first element of the piece
    uint64_t count;
    uint64_t begin;  // global weight index
    uint32_t tensor;
};

std::vector<Piece> split(uint32_t format, const void *const *tensors, const uint64_t *numel,
                         uint32_t n) {
    std::vector<Piece> out;
    const uint32_t eb = element_bytes(format);
    uint64_t g = 0;
    for (uint32_t k = 0; k < n; k++) {
        for (uint64_t o = 0; o < numel[k]; o += kChunk)
            out.push_back({static_cast<const uint8_t *>(tensors[k]) + o * eb,
                           std::min(kChunk, numel[k] - o), g + o, k});
        g += numel[k];
    }
    return out;
}

// Exponent histogram over all pieces, one partial table per piece.
template <class Fm>
void histogram(const std::vector<Piece> &pieces, std::vector<uint64_t> &per_piece,
               uint64_t total[kSyms]) {
    per_piece.assign(pieces.size() * kSyms, 0);
    parallel_for(pieces.size(), [&](size_t p) {
        uint32_t h[4][kSyms] = {};
        const auto *w = static_cast<const typename Fm::T *>(pieces[p].w);
        uint64_t n = pieces[p].count, i = 0;
        for (; i + 4 <= n; i += 4) {
            h[0][Fm::sym(w[i])]++;
            h[1][Fm::sym(w[i + 1])]++;
            h[2][Fm::sym(w[i + 2])]++;
            h[3][Fm::sym(w[i + 3])]++;
        }
        for (; i < n; i++) h[0][Fm::sym(w[i])]++;
        uint64_t *dst = &per_piece[p * kSyms];
        for (int s = 0; s < kSyms; s++) dst[s] = uint64_t(h[0][s]) + h[1][s] + h[2][s] + h[3][s];
    });
    std::fill(total, total + kSyms, 0);
    for (size_t p = 0; p < pieces.size(); p++)
        for (int s = 0; s < kSyms; s++) total[s] += per_piece[p * kSyms + s];
}

void histogram_any(uint32_t format, const std::vector<Piece> &pieces,
                   std::vector<uint64_t> &per_piece, uint64_t total[kSyms]) {
    with_format(format, [&](auto fm) { histogram<decltype(fm)>(pieces, per_piece, total); });
}

// ---------------------------------------------------------------- lengths

// Huffman lengths with a binary min-heap on (weight, tiebreak).
int huffman(const uint64_t counts[kSyms], uint8_t len[kSyms]) {
    struct Key {
        uint64_t w;
        uint32_t tb;
        int node;
    };
    auto greater = [](const Key &a, const Key &b) {
        return a.w != b.w ? a.w > b.w : a.tb > b.tb;
    };
    std::vector<Key> heap;
    int parent[2 * kSyms];
    int leaf_node[kSyms];
    int nodes = 0;
    std::memset(len, 0, kSyms);
    for (int s = 0; s < kSyms; s++) {
        leaf_node[s] = -1;
        if (counts[s]) {
            leaf_node[s] = nodes;
            parent[nodes] = -1;
            heap.push_back({counts[s], uint32_t(s), nodes++});
        }
    }
    const int present = nodes;
    if (present == 0) return 0;
    if (present == 1) {
        int only = 0, dummy = 0;
        while (!counts[only]) only++;
        while (counts[dummy]) dummy++;
        len[only] = len[dummy] = 1;
        return 1;
    }
    std::make_heap(heap.begin(), heap.end(), greater);
    for (int k = 0; k + 1 < present; k++) {
        std::pop_heap(heap.begin(), heap.end(), greater);
        Key a = heap.back();
        heap.pop_back();
        std::pop_heap(heap.begin(), heap.end(), greater);
        Key b = heap.back();
        heap.pop_back();
        parent[a.node] = parent[b.node] = nodes;
        parent[nodes] = -1;
        heap.push_back({a.w + b.w, uint32_t(kSyms + k), nodes++});
        std::push_heap(heap.begin(), heap.end(), greater);
    }
    // depth of node v = depth(parent) + 1; parents are created after children,
    // so walking node ids downward from the root visits parents first
    std::vector<int> depth(nodes, 0);
    for (int v = nodes - 2; v >= 0; v--) depth[v] = depth[parent[v]] + 1;
    int mx = 0;
    for (int s = 0; s < kSyms; s++)
        if (leaf_node[s] >= 0) {
            len[s] = uint8_t(std::min(depth[leaf_node[s]], 255));
            mx = std::max(mx, depth[leaf_node[s]]);
        }
    return mx;
}

// Length-limited optimal lengths by boundary package-merge (Katajainen,
// Moffat and Turpin, "A fast and space-economical algorithm for length-limited
// coding", 1995): package-merge evaluated lazily.  Level 0 is the deepest
// denomination (leaves only); the item lists of level j are never stored,
// only their two newest items ("lookahead chains").  A chain records its
// weight, the number of leaves among the items of its level up to it, and the
// chain of the level below that closes the last package up to it.  Advancing
// the top level 2n - 2 items advances each level below only as far as the
// packages above need; the chains reached from the top level's last item are
// then the ends of the chosen prefixes of every level, and leaf i (in
// ascending weight order) gets one bit per level whose prefix holds more than
// i leaves.  Ties between a leaf and a package take the leaf.
int package_merge(const uint64_t counts[kSyms], int limit, uint8_t len[kSyms]) {
    std::vector<int> sym;
    for (int s = 0; s < kSyms; s++)
        if (counts[s]) sym.push_back(s);
    const uint32_t n = uint32_t(sym.size());
    std::stable_sort(sym.begin(), sym.end(),
                     [&](int a, int b) { return counts[a] < counts[b]; });
    std::memset(len, 0, kSyms);
    if (n < 2) return huffman(counts, len);
    struct Chain {
        uint64_t weight;
        uint32_t leaves;  // leaves among the level's items up to this one
        int below;        // chain of the level below closing the last package (-1: none)
    };
    std::vector<Chain> pool;
    pool.reserve(size_t(limit) * (2 * n + 2));
    auto make = [&](uint64_t w, uint32_t c, int t) {
        pool.push_back({w, c, t});
        return int(pool.size() - 1);
    };
    const auto leaf_w = [&](uint32_t i) { return counts[sym[i]]; };
    // the two newest chains of every level; all levels start with the two
    // lightest leaves
    std::vector<int> older(limit), newer(limit);
    for (int j = 0; j < limit; j++) {
        older[j] = make(leaf_w(0), 1, -1);
        newer[j] = make(leaf_w(1), 2, -1);
    }
    // next item of level j: the next leaf, or the package of the two newest
    // items of level j - 1, whichever is lighter (then level j - 1 moves on
    // by two items)
    std::function<void(int)> advance = [&](int j) {
        const Chain cur = pool[newer[j]];
        if (j == 0) {
            if (cur.leaves >= n) return;
            older[0] = newer[0];
            newer[0] = make(leaf_w(cur.leaves), cur.leaves + 1, -1);
            return;
        }
        const uint64_t pkg = pool[older[j - 1]].weight + pool[newer[j - 1]].weight;
        older[j] = newer[j];
        if (cur.leaves < n && leaf_w(cur.leaves) <= pkg) {
            newer[j] = make(leaf_w(cur.leaves), cur.leaves + 1, cur.below);
        } else {
            newer[j] = make(pkg, cur.leaves, newer[j - 1]);
            advance(j - 1);
            advance(j - 1);
        }
    };
    for (uint32_t k = 2; k < 2 * n - 2; k++) advance(limit - 1);
    int mx = 0;
    for (int c = newer[limit - 1]; c >= 0; c = pool[c].below)
        for (uint32_t i = 0; i < pool[c].leaves; i++) mx = std::max<int>(mx, ++len[sym[i]]);
    return mx;
}

// Canonical codes from lengths: per-length counts give each length's first
// code; symbols of equal length take consecutive codes in value order.
void canonical(const uint8_t len[kSyms], uint32_t code[kSyms]) {
    uint64_t count[DF11_MAX_CODE_LEN + 2] = {}, next[DF11_MAX_CODE_LEN + 2] = {};
    for (int s = 0; s < kSyms; s++)
        if (len[s]) count[len[s]]++;
    for (int l = 2; l <= DF11_MAX_CODE_LEN; l++) next[l] = (next[l - 1] + count[l - 1]) << 1;
    for (int s = 0; s < kSyms; s++) code[s] = len[s] ? uint32_t(next[len[s]]++) : 0;
}

// Hierarchical 8-bit-indexed lookup tables (the compact hierarchical LUTs of
// the DFloat11 abstract).  A code of length l, left-aligned in 32 bits, is
// resolved at level floor((l - 1) / 8); shorter levels hold pointers.
int build_luts(df11_codebook *cb) {
    std::memset(cb->lut, 0, sizeof(cb->lut));
    uint32_t n_luts = 1;
    for (int s = 0; s < kSyms; s++) {
        const int l = cb->code_len[s];
        if (!l) continue;
        const uint32_t v = cb->code[s] << (32 - l);  // l >= 1
        uint32_t table = 0;
        for (int lvl = 0;; lvl++) {
            const uint32_t idx = (v >> (24 - 8 * lvl)) & 0xFF;
            if (l <= 8 * (lvl + 1)) {
                const uint32_t span = 1u << (8 * (lvl + 1) - l);
                for (uint32_t i = 0; i < span; i++)
                    cb->lut[table][idx + i] = uint16_t((l << 8) | s);
                break;
            }
            uint16_t &e = cb->lut[table][idx];
            if (!(e & 0x8000)) {
                if (n_luts >= DF11_MAX_LUTS) return DF11_E_LUT_BUDGET;
                e = uint16_t(0x8000 | n_luts++);
            }
            table = e & 0x7FFF;
        }
    }
    cb->n_luts = n_luts;
    return DF11_OK;
}

// Length and symbol of the code at the head of a 32-bit left-aligned value,
// by walking the hierarchical tables; length 0 if no leaf is reached.
void head_code(const df11_codebook *cb, uint32_t v, uint32_t &len, uint32_t &sym) {
    uint32_t e = cb->lut[0][v >> 24];
    for (int lvl = 1; (e & 0x8000) && lvl < 4; lvl++)
        e = cb->lut[e & 0x7FFF][(v >> (24 - 8 * lvl)) & 0xFF];
    len = (e & 0x8000) ? 0 : (e >> 8) & 0x3F;
    sym = e & 0xFF;
}

// The table a root entry points at, or 0 when the entry is a leaf.
uint32_t level1_table(const df11_codebook *cb, uint32_t top8) {
    const uint32_t e = cb->lut[0][top8];
    return (e & 0x8000) ? (e & 0x7FFF) : 0u;
}

// Multi-code tables for the decoder's fast path.  Bits beyond the index are
// taken as zero: a code that fits in the remaining index bits is decoded the
// same whatever follows, and one that does not fit comes out longer than
// the remaining bits, so it is left out.
void build_multi_tables(df11_codebook *cb) {
    constexpr uint32_t kM = DF11_MULTI_BITS, kC = DF11_COUNT_BITS;
    for (uint32_t x = 0; x < (1u << kM); x++) {
        const uint32_t v = x << (32 - kM);
        uint32_t used = 0, n = 0, syms = 0;
        while (n < 3) {
            uint32_t len, sym;
            head_code(cb, v << used, len, sym);
            if (len == 0 || used + len > kM) break;
            syms |= sym << (8 * n);
            n++;
            used += len;
        }
        // no code fits: the first is longer than 8 bits, so the root entry of
        // the index's top 8 bits points at the level-1 table to walk from
        cb->multi[x] = n ? (n << 30) | (used << 24) | syms : level1_table(cb, x >> (kM - 8));
    }
    for (uint32_t x = 0; x < (1u << kC); x++) {
        const uint32_t v = x << (32 - kC);
        uint32_t used = 0, mask = 0;
        for (;;) {
            uint32_t len, sym;
            head_code(cb, v << used, len, sym);
            if (len == 0 || used + len > kC) break;
            mask |= 1u << used;
            used += len;
        }
        cb->count[x] = uint16_t(used ? (used << 12) | mask : level1_table(cb, x >> (kC - 8)));
    }
}

bool valid_layout(uint32_t T, uint32_t B) { return B == 8 && (T == 64 || T == 256 || T == 512); }

// FP8 units are decoded by the 64-window kernel only.
bool valid_format_layout(uint32_t format, uint32_t T) {
    if (format == DF11_FORMAT_BF16) return true;
    return (format == DF11_FORMAT_FP8_E4M3 || format == DF11_FORMAT_FP8_E5M2) && T == 64;
}

int log2u(uint64_t x) {
    int r = 0;
    while ((uint64_t(1) << r) < x) r++;
    return r;
}

bool valid_codebook(const df11_codebook *cb) {
    if (cb->n_luts < 1 || cb->n_luts > DF11_MAX_LUTS) return false;
    for (int s = 0; s < kSyms; s++)
        if (cb->code_len[s] > DF11_MAX_CODE_LEN) return false;
    return true;
}

int sizes_from_counts(uint32_t format, const df11_codebook *cb, const uint64_t counts[kSyms],
                      uint64_t n, uint32_t T, uint32_t B, df11_sizes *out) {
    uint64_t bits = 0;
    for (int s = 0; s < kSyms; s++) {
        if (counts[s] && !cb->code_len[s]) return DF11_E_SYMBOL;
        bits += counts[s] * cb->code_len[s];
    }
    const uint64_t tile_bits = uint64_t(8) * B * T;
    out->n_weights = n;
    out->total_bits = bits;
    out->n_tiles = (bits + tile_bits - 1) / tile_bits;
    out->n_windows = out->n_tiles * T;
    out->stream_bytes = out->n_tiles * T * B + DF11_STREAM_PAD;
    const uint64_t rest_bytes = format == DF11_FORMAT_BF16 ? n : (n + 1) / 2;
    out->sm_bytes = (rest_bytes + 63) / 64 * 64 + 64;
    out->bop_entries = out->n_tiles + 1;
    return DF11_OK;
}

bool bad_inputs(const void *const *tensors, const uint64_t *numel, uint32_t n) {
    if (n && (!tensors || !numel)) return true;
    for (uint32_t k = 0; k < n; k++)
        if (numel[k] && !tensors[k]) return true;
    return false;
}

// Per-piece encoder results needed to stitch neighbouring pieces together.
struct PieceOut {
    uint64_t first_window = 0, last_window = 0;
    uint32_t first_gap = 0;
};

inline void or_byte(uint8_t *p, uint8_t v) {
    if (v) __atomic_fetch_or(p, v, __ATOMIC_RELAXED);
}

// Encodes one piece whose first code starts at bit `pos`.
template <class Fm>
void encode_piece(const df11_codebook *cb, const Piece &pc, uint64_t pos, uint64_t end_pos,
                  int wshift, int tshift, uint8_t *stream, uint8_t *sm, uint8_t *gaps,
                  uint32_t *bop, PieceOut &po) {
    const uint64_t wmask = (uint64_t(1) << wshift) - 1;
    uint64_t byte = pos >> 3;
    unsigned nacc = unsigned(pos & 7);  // pending bits; the leading ones belong to the previous piece
    uint64_t acc = 0;
    bool shared_head = nacc != 0;

    po.first_window = pos >> wshift;
    po.first_gap = uint32_t(pos & wmask);
    uint64_t next_window = (po.first_window + 1) << wshift;
    uint64_t last_window = po.first_window;
    uint64_t next_tile = ((pos >> tshift) + 1) << tshift;

    const auto *w = static_cast<const typename Fm::T *>(pc.w);
    uint32_t pend = 0;  // FP8: the low nibble waiting for its pair
    for (uint64_t i = 0; i < pc.count; i++) {
        const auto x = w[i];
        const uint32_t e = Fm::sym(x);
        if (pos >= next_window) {  // first code starting in a new window
            last_window = pos >> wshift;
            gaps[last_window] = uint8_t(pos & wmask);
            next_window = (last_window + 1) << wshift;
        }
        if (pos >= next_tile) {  // first code at or after a tile boundary
            bop[next_tile >> tshift] = uint32_t(pc.begin + i);
            next_tile += uint64_t(1) << tshift;
        }
        const unsigned l = cb->code_len[e];
        acc = (acc << l) | cb->code[e];
        nacc += l;
        pos += l;
        if (nacc >= 32) {
            const uint32_t word = uint32_t(acc >> (nacc - 32));
            uint8_t b[4] = {uint8_t(word >> 24), uint8_t(word >> 16), uint8_t(word >> 8),
                            uint8_t(word)};
            if (shared_head) {
                or_byte(stream + byte, b[0]);
                std::memcpy(stream + byte + 1, b + 1, 3);
                shared_head = false;
            } else {
                std::memcpy(stream + byte, b, 4);
            }
            byte += 4;
            nacc -= 32;
            acc &= (uint64_t(1) << nacc) - 1;
        }
        if constexpr (!Fm::kNibbles) {
            sm[pc.begin + i] = uint8_t(Fm::rest(x));
        } else {
            const uint64_t g = pc.begin + i;
            if (g & 1) {
                const uint8_t v = uint8_t(pend | (Fm::rest(x) << 4));
                if (i == 0) or_byte(sm + (g >> 1), v);  // low nibble from the piece before
                else sm[g >> 1] = v;
            } else {
                pend = Fm::rest(x);
            }
        }
    }
    if constexpr (Fm::kNibbles) {
        const uint64_t g = pc.begin + pc.count;  // one past the last weight
        if (pc.count && (g & 1)) or_byte(sm + (g >> 1), uint8_t(pend));  // high nibble from the next
    }
    // tail bytes, the last possibly shared with the next piece
    for (unsigned k = 0; k < nacc; k += 8) {
        const unsigned take = std::min(8u, nacc - k);
        const uint8_t v = uint8_t(((acc >> (nacc - k - take)) & ((1u << take) - 1)) << (8 - take));
        or_byte(stream + byte++, v);
    }
    // tile boundaries after this piece's last code start, up to the next piece's first
    while (next_tile <= end_pos) {
        bop[next_tile >> tshift] = uint32_t(pc.begin + pc.count);
        next_tile += uint64_t(1) << tshift;
    }
    po.last_window = last_window;
}

// Element offsets and tile ranges of the unit's tensors: tensor k holds
// numel[k] weights whose codes take bits[k] bits, and its last weight's symbol
// is last_sym[k].  Its tiles run from the one holding its first code start to
// the one holding its last.
void tensor_ranges(const df11_codebook *cb, const uint64_t *numel, const uint64_t *bits,
                   const uint32_t *last_sym, uint32_t n_tensors, int tshift,
                   uint64_t *tensor_offsets, uint64_t *tensor_tiles) {
    uint64_t g = 0, bit = 0;
    for (uint32_t k = 0; k < n_tensors; k++) {
        tensor_offsets[k] = g;
        tensor_tiles[2 * k] = bit >> tshift;
        if (numel[k]) {
            const uint64_t last_start = bit + bits[k] - cb->code_len[last_sym[k] & 0xFFu];
            tensor_tiles[2 * k + 1] = (last_start >> tshift) + 1;
        } else {
            tensor_tiles[2 * k + 1] = tensor_tiles[2 * k];
        }
        g += numel[k];
        bit += bits[k];
    }
    tensor_offsets[n_tensors] = g;
}

}  // namespace

extern "C" {

const char *df11_status_string(int status) {
    switch (status) {
    case DF11_OK: return "ok";
    case DF11_E_INVALID: return "invalid argument";
    case DF11_E_LUT_BUDGET: return "codebook needs more lookup tables than DF11_MAX_LUTS";
    case DF11_E_SYMBOL: return "input exponent has no code in the codebook";
    case DF11_E_CAPACITY: return "output buffer smaller than df11_encode_size reports";
    case DF11_E_HIP: return "HIP launch error";
    case DF11_E_CORRUPT: return "compressed stream is inconsistent with its auxiliary arrays";
    default: return "unknown status";
    }
}

int df11_build_codebook_fmt(uint32_t format, const void *const *tensors, const uint64_t *numel,
                            uint32_t n_tensors, df11_codebook *cb) {
    try {
        if (!cb || bad_inputs(tensors, numel, n_tensors) || !with_format(format, [](auto) {}))
            return DF11_E_INVALID;
        auto pieces = split(format, tensors, numel, n_tensors);
        std::vector<uint64_t> per;
        uint64_t counts[kSyms];
        histogram_any(format, pieces, per, counts);
        return df11_build_codebook_from_counts(counts, cb);
    } catch (...) {
        return DF11_E_INVALID;
    }
}

int df11_build_codebook_from_counts(const uint64_t *counts, df11_codebook *cb) {
    try {
        if (!counts || !cb) return DF11_E_INVALID;
        uint64_t n = 0;
        for (int s = 0; s < kSyms; s++) n += counts[s];
        if (n == 0) return DF11_E_INVALID;
        std::memset(cb, 0, sizeof(*cb));
        int mx = huffman(counts, cb->code_len);
        if (mx > DF11_MAX_CODE_LEN) mx = package_merge(counts, DF11_MAX_CODE_LEN, cb->code_len);
        cb->max_len = uint32_t(mx);
        canonical(cb->code_len, cb->code);
        int rc = build_luts(cb);
        if (rc != DF11_OK) return rc;
        build_multi_tables(cb);
        return DF11_OK;
    } catch (...) {
        return DF11_E_INVALID;
    }
}

int df11_encode_size_from_counts(uint32_t format, const df11_codebook *cb, const uint64_t *counts,
                                 uint64_t n_weights, uint32_t tile_windows, uint32_t window_bytes,
                                 df11_sizes *out) {
    if (!cb || !counts || !out || !valid_layout(tile_windows, window_bytes) ||
        !valid_codebook(cb) || !valid_format_layout(format, tile_windows))
        return DF11_E_INVALID;
    uint64_t n = 0;
    for (int s = 0; s < kSyms; s++) n += counts[s];
    if (n != n_weights) return DF11_E_INVALID;
    return sizes_from_counts(format, cb, counts, n, tile_windows, window_bytes, out);
}

int df11_tensor_ranges_from_counts(uint32_t format, const df11_codebook *cb,
                                   const uint64_t *counts, const uint32_t *last_weights,
                                   uint32_t n_tensors, uint32_t tile_windows,
                                   uint32_t window_bytes, uint64_t *tensor_offsets,
                                   uint64_t *tensor_tiles) {
    try {
        if (!cb || !valid_codebook(cb) || !valid_layout(tile_windows, window_bytes) ||
            !valid_format_layout(format, tile_windows) || !tensor_offsets ||
            (n_tensors && (!counts || !last_weights || !tensor_tiles)))
            return DF11_E_INVALID;
        std::vector<uint64_t> numel(n_tensors, 0), bits(n_tensors, 0);
        std::vector<uint32_t> last_sym(n_tensors, 0);
        uint64_t n = 0;
        for (uint32_t k = 0; k < n_tensors; k++) {
            const uint64_t *c = counts + uint64_t(k) * kSyms;
            for (int s = 0; s < kSyms; s++) {
                if (c[s] && !cb->code_len[s]) return DF11_E_SYMBOL;
                numel[k] += c[s];
                bits[k] += c[s] * cb->code_len[s];
            }
            n += numel[k];
            if (!numel[k]) continue;
            bool ok = with_format(format, [&](auto fm) {
                using Fm = decltype(fm);
                last_sym[k] = Fm::sym(typename Fm::T(last_weights[k]));
            });
            if (!ok) return DF11_E_INVALID;
            if (!c[last_sym[k]]) return DF11_E_INVALID;  // the last weight is not counted
        }
        if (n >= (uint64_t(1) << 32)) return DF11_E_INVALID;
        const int tshift = log2u(uint64_t(8) * window_bytes) + log2u(tile_windows);
        tensor_ranges(cb, numel.data(), bits.data(), last_sym.data(), n_tensors, tshift,
                      tensor_offsets, tensor_tiles);
        return DF11_OK;
    } catch (...) {
        return DF11_E_INVALID;
    }
}

int df11_build_codebook(const uint16_t *const *tensors, const uint64_t *numel, uint32_t n_tensors,
                        df11_codebook *cb) {
    return df11_build_codebook_fmt(DF11_FORMAT_BF16, reinterpret_cast<const void *const *>(tensors),
                                   numel, n_tensors, cb);
}

int df11_encode_size_fmt(uint32_t format, const df11_codebook *cb, const void *const *tensors,
                         const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                         uint32_t window_bytes, df11_sizes *out) {
    try {
        if (!cb || !out || bad_inputs(tensors, numel, n_tensors) ||
            !valid_layout(tile_windows, window_bytes) || !valid_codebook(cb) ||
            !valid_format_layout(format, tile_windows))
            return DF11_E_INVALID;
        auto pieces = split(format, tensors, numel, n_tensors);
        std::vector<uint64_t> per;
        uint64_t counts[kSyms];
        histogram_any(format, pieces, per, counts);
        uint64_t n = 0;
        for (uint32_t k = 0; k < n_tensors; k++) n += numel[k];
        return sizes_from_counts(format, cb, counts, n, tile_windows, window_bytes, out);
    } catch (...) {
        return DF11_E_INVALID;
    }
}

int df11_encode_size(const df11_codebook *cb, const uint16_t *const *tensors, const uint64_t *numel,
                     uint32_t n_tensors, uint32_t tile_windows, uint32_t window_bytes,
                     df11_sizes *out) {
    return df11_encode_size_fmt(DF11_FORMAT_BF16, cb, reinterpret_cast<const void *const *>(tensors),
                                numel, n_tensors, tile_windows, window_bytes, out);
}

int df11_encode_fmt(uint32_t format, const df11_codebook *cb, const void *const *tensors,
                    const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                    uint32_t window_bytes, df11_host_stream *out) {
    try {
        if (!cb || !out || bad_inputs(tensors, numel, n_tensors) ||
            !valid_layout(tile_windows, window_bytes) || !valid_codebook(cb) ||
            !valid_format_layout(format, tile_windows) || out->n_tensors != n_tensors)
            return DF11_E_INVALID;
        auto pieces = split(format, tensors, numel, n_tensors);
        std::vector<uint64_t> per;
        uint64_t counts[kSyms];
        histogram_any(format, pieces, per, counts);
        uint64_t n = 0;
        for (uint32_t k = 0; k < n_tensors; k++) n += numel[k];
        if (n >= (uint64_t(1) << 32)) return DF11_E_INVALID;
        df11_sizes sz;
        int rc = sizes_from_counts(format, cb, counts, n, tile_windows, window_bytes, &sz);
        if (rc != DF11_OK) return rc;
        if (!out->stream || !out->sm || !out->block_out_pos || !out->tensor_offsets ||
            (n_tensors && !out->tensor_tiles) || (sz.n_windows && !out->gaps))
            return DF11_E_INVALID;
        if (out->stream_capacity < sz.stream_bytes || out->sm_capacity < sz.sm_bytes ||
            out->gaps_capacity < sz.n_windows || out->bop_capacity < sz.bop_entries)
            return DF11_E_CAPACITY;

        // start bit of every piece
        std::vector<uint64_t> start(pieces.size() + 1, 0);
        for (size_t p = 0; p < pieces.size(); p++) {
            uint64_t b = 0;
            for (int s = 0; s < kSyms; s++) b += per[p * kSyms + s] * cb->code_len[s];
            start[p + 1] = start[p] + b;
        }
        const int wshift = log2u(uint64_t(8) * window_bytes);
        const int tshift = wshift + log2u(tile_windows);

        std::memset(out->stream, 0, sz.stream_bytes);
        std::memset(out->gaps, 255, sz.n_windows);
        if (format == DF11_FORMAT_BF16) std::memset(out->sm + n, 0, sz.sm_bytes - n);
        else std::memset(out->sm, 0, sz.sm_bytes);  // nibbles of neighbouring pieces are OR-ed
        out->block_out_pos[0] = 0;
        out->block_out_pos[sz.n_tiles] = uint32_t(n);

        std::vector<PieceOut> po(pieces.size());
        with_format(format, [&](auto fm) {
            parallel_for(pieces.size(), [&](size_t p) {
                encode_piece<decltype(fm)>(cb, pieces[p], start[p], start[p + 1], wshift, tshift,
                                           out->stream, out->sm, out->gaps, out->block_out_pos,
                                           po[p]);
            });
        });
        // a piece's first window may already have a code start from the piece before
        bool have_prev = false;
        uint64_t prev_last = 0;
        for (size_t p = 0; p < pieces.size(); p++) {
            if (!pieces[p].count) continue;
            if (!have_prev || prev_last != po[p].first_window)
                out->gaps[po[p].first_window] = uint8_t(po[p].first_gap);
            have_prev = true;
            prev_last = po[p].last_window;
        }

        // per-tensor element offsets and tile ranges
        std::vector<uint64_t> bits(n_tensors, 0);
        std::vector<uint32_t> last_sym(n_tensors, 0);
        for (size_t p = 0; p < pieces.size(); p++) bits[pieces[p].tensor] += start[p + 1] - start[p];
        for (uint32_t k = 0; k < n_tensors; k++) {
            if (!numel[k]) continue;
            with_format(format, [&](auto fm) {
                using Fm = decltype(fm);
                last_sym[k] = Fm::sym(static_cast<const typename Fm::T *>(tensors[k])[numel[k] - 1]);
            });
        }
        tensor_ranges(cb, numel, bits.data(), last_sym.data(), n_tensors, tshift,
                      out->tensor_offsets, out->tensor_tiles);

        uint32_t mx = 0;
        for (uint64_t t = 0; t < sz.n_tiles; t++)
            mx = std::max(mx, out->block_out_pos[t + 1] - out->block_out_pos[t]);
        out->tile_windows = tile_windows;
        out->window_bytes = window_bytes;
        out->max_tile_symbols = mx;
        out->n_weights = n;
        out->total_bits = sz.total_bits;
        out->n_tiles = sz.n_tiles;
        out->format = format;
        return DF11_OK;
    } catch (...) {
        return DF11_E_INVALID;
    }
}

int df11_encode(const df11_codebook *cb, const uint16_t *const *tensors, const uint64_t *numel,
                uint32_t n_tensors, uint32_t tile_windows, uint32_t window_bytes,
                df11_host_stream *out) {
    return df11_encode_fmt(DF11_FORMAT_BF16, cb, reinterpret_cast<const void *const *>(tensors),
                           numel, n_tensors, tile_windows, window_bytes, out);
}

int df11_gemm_order(const uint16_t *w, uint32_t rows, uint32_t cols, uint16_t *out) {
    if (rows == 0 || cols == 0) return DF11_OK;
    if (!w || !out || w == out || rows % 16 || cols % 32) return DF11_E_INVALID;
    const uint32_t kbs = cols / 32;
    // one 16-row block per task: its sub-blocks (kb) of 16 rows x 32 columns,
    // each as four 8-column quarters q, each as 16 rows of 8 weights
    parallel_for(rows / 16, [&](size_t m) {
        uint16_t *o = out + m * 16 * size_t(cols);
        for (uint32_t kb = 0; kb < kbs; kb++)
            for (uint32_t q = 0; q < 4; q++)
                for (uint32_t i = 0; i < 16; i++) {
                    const uint16_t *src = w + (m * 16 + i) * size_t(cols) + 32 * kb + 8 * q;
                    std::copy(src, src + 8, o + ((size_t(kb) * 4 + q) * 16 + i) * 8);
                }
    });
    return DF11_OK;
}

}  // extern "C"
