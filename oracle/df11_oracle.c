/*
 * df11_oracle.c -- plain, slow, bit-serial CPU oracle for DFloat11-style
 * lossless BF16 compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * What it computes, and from where:
 *  - "70% Size, 100% Accuracy: Lossless LLM Compression for Efficient GPU
 *    Inference via Dynamic-Length Float (DFloat11)", abstract: weights are
 *    entropy-coded with dynamic-length codes chosen by frequency, and the
 *    decompressed model is bit-for-bit identical to the original.
 *  - "Compressing LLMs without Compromise" summary page, sections "Where the
 *    redundancy lives" (a BF16 value is 1 sign, 8 exponent and 7 mantissa
 *    bits; only the exponent is low-entropy) and "Three ways to spend the
 *    savings" (the exponents are Huffman-coded offline).
 *
 * Readings where the pages are silent (each is fixed so two independent
 * implementations can be compared byte for byte):
 *  - symbol e = (w >> 7) & 0xFF; sign+mantissa byte sm = ((w >> 8) & 0x80) | (w & 0x7F);
 *  - Huffman merges the two nodes with the smallest (weight, tiebreak); a leaf's
 *    tiebreak is its symbol, the k-th internal node's is 256 + k;
 *  - a single present symbol gets length 1 together with a dummy: the smallest
 *    absent symbol value, also length 1;
 *  - if a Huffman length exceeds 32 the lengths are recomputed by
 *    package-merge with a 32-bit limit;
 *  - canonical codes: symbols sorted by (length, value) take consecutive codes;
 *  - the bitstream is MSB-first: stream bit j is bit (7 - j % 8) of byte j / 8;
 *  - window j covers stream bits [8B*j, 8B*(j+1)); its gap is the offset of the
 *    first code that starts inside it, or 255 when none does;
 *  - block_out_pos[w] = number of codes that start before bit 8*B*T*w.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NSYM 256
#define MAXLEN 32

/* Histogram of exponent symbols: counts[s] = #{i : ((w_i >> 7) & 0xFF) == s}. */
void oracle_histogram(const uint16_t *w, uint64_t n, uint64_t *counts)
{
    for (int s = 0; s < NSYM; s++)
        counts[s] = 0;
    for (uint64_t i = 0; i < n; i++)
        counts[(w[i] >> 7) & 0xFF] += 1;
}

/*
 * Huffman code lengths (unlimited).  Returns the longest length, 0 when no
 * symbol is present.  Node selection is a linear scan for the smallest
 * (weight, tiebreak) among live nodes: O(n^2), which is nothing for n <= 256.
 */
int oracle_huffman_lengths(const uint64_t *counts, uint8_t *lens)
{
    uint64_t weight[2 * NSYM];
    uint32_t tiebreak[2 * NSYM];
    int parent[2 * NSYM];
    int live[2 * NSYM];
    int nodes = 0, present = 0;
    int leaf_of_sym[NSYM];

    for (int s = 0; s < NSYM; s++) {
        lens[s] = 0;
        leaf_of_sym[s] = -1;
    }
    for (int s = 0; s < NSYM; s++) {
        if (counts[s] == 0)
            continue;
        weight[nodes] = counts[s];
        tiebreak[nodes] = (uint32_t)s;
        parent[nodes] = -1;
        live[nodes] = 1;
        leaf_of_sym[s] = nodes;
        nodes++;
        present++;
    }
    if (present == 0)
        return 0;
    if (present == 1) {
        int only = -1, dummy = -1;
        for (int s = 0; s < NSYM; s++)
            if (counts[s] != 0)
                only = s;
        for (int s = 0; s < NSYM && dummy < 0; s++)
            if (counts[s] == 0)
                dummy = s;
        lens[only] = 1;
        lens[dummy] = 1;
        return 1;
    }
    for (int k = 0; k < present - 1; k++) {
        int pick[2];
        for (int r = 0; r < 2; r++) {
            int best = -1;
            for (int i = 0; i < nodes; i++) {
                if (!live[i])
                    continue;
                if (best < 0 || weight[i] < weight[best] ||
                    (weight[i] == weight[best] && tiebreak[i] < tiebreak[best]))
                    best = i;
            }
            live[best] = 0;
            pick[r] = best;
        }
        weight[nodes] = weight[pick[0]] + weight[pick[1]];
        tiebreak[nodes] = (uint32_t)(NSYM + k);
        parent[nodes] = -1;
        live[nodes] = 1;
        parent[pick[0]] = nodes;
        parent[pick[1]] = nodes;
        nodes++;
    }
    int maxlen = 0;
    for (int s = 0; s < NSYM; s++) {
        if (leaf_of_sym[s] < 0)
            continue;
        int depth = 0;
        for (int v = leaf_of_sym[s]; parent[v] >= 0; v = parent[v])
            depth++;
        lens[s] = (uint8_t)(depth > 255 ? 255 : depth);
        if (depth > maxlen)
            maxlen = depth;
    }
    return maxlen;
}

/*
 * Length-limited optimal code lengths by package-merge (Larmore and
 * Hirschberg, "A fast algorithm for optimal length-limited Huffman codes",
 * JACM 1990), coin-collector form: every present symbol contributes one coin
 * of face value 2^-l and weight counts[s] for each l in 1..limit; the cheapest
 * set of coins of total face value (n - 1) gives l_s = number of coins of s
 * chosen.  Lists are built from denomination 2^-limit up to 2^-1 by pairing
 * neighbours into packages and merging them with the leaves (leaves first on
 * equal weight).  Returns the longest length, or -1 if n > 2^limit.
 */
typedef struct {
    uint64_t w;
    int leaf;     /* symbol, or -1 for a package */
    int a, b;     /* package: indexes into the next-deeper list */
} pm_item;

static void pm_count(pm_item **lists, int level, int idx, int limit, uint8_t *lens)
{
    pm_item it = lists[level][idx];
    if (it.leaf >= 0) {
        lens[it.leaf] += 1;
        return;
    }
    pm_count(lists, level + 1, it.a, limit, lens);
    pm_count(lists, level + 1, it.b, limit, lens);
}

int oracle_limited_lengths(const uint64_t *counts, int limit, uint8_t *lens)
{
    int sym[NSYM];
    int n = 0;
    for (int s = 0; s < NSYM; s++) {
        lens[s] = 0;
        if (counts[s] != 0)
            sym[n++] = s;
    }
    if (n <= 1 || limit < 1)
        return oracle_huffman_lengths(counts, lens);
    if (limit < 31 && ((uint64_t)1 << limit) < (uint64_t)n)
        return -1;

    /* leaves sorted by (weight, symbol): insertion sort */
    for (int i = 1; i < n; i++) {
        int s = sym[i], j = i - 1;
        while (j >= 0 && (counts[sym[j]] > counts[s] ||
                          (counts[sym[j]] == counts[s] && sym[j] > s))) {
            sym[j + 1] = sym[j];
            j--;
        }
        sym[j + 1] = s;
    }

    pm_item **lists = (pm_item **)calloc((size_t)limit + 2, sizeof(pm_item *));
    int *len_of = (int *)calloc((size_t)limit + 2, sizeof(int));
    /* deepest denomination 2^-limit: the leaves alone */
    lists[limit] = (pm_item *)malloc(sizeof(pm_item) * (size_t)n);
    for (int i = 0; i < n; i++) {
        lists[limit][i].w = counts[sym[i]];
        lists[limit][i].leaf = sym[i];
        lists[limit][i].a = lists[limit][i].b = -1;
    }
    len_of[limit] = n;
    for (int level = limit - 1; level >= 1; level--) {
        int npk = len_of[level + 1] / 2;
        pm_item *out = (pm_item *)malloc(sizeof(pm_item) * (size_t)(n + npk));
        int li = 0, pi = 0, o = 0;
        while (li < n || pi < npk) {
            uint64_t pw = 0;
            if (pi < npk)
                pw = lists[level + 1][2 * pi].w + lists[level + 1][2 * pi + 1].w;
            if (li < n && (pi >= npk || counts[sym[li]] <= pw)) {
                out[o].w = counts[sym[li]];
                out[o].leaf = sym[li];
                out[o].a = out[o].b = -1;
                li++;
            } else {
                out[o].w = pw;
                out[o].leaf = -1;
                out[o].a = 2 * pi;
                out[o].b = 2 * pi + 1;
                pi++;
            }
            o++;
        }
        lists[level] = out;
        len_of[level] = o;
    }
    for (int i = 0; i < 2 * n - 2; i++)
        pm_count(lists, 1, i, limit, lens);
    int maxlen = 0;
    for (int s = 0; s < NSYM; s++)
        if (lens[s] > maxlen)
            maxlen = lens[s];
    for (int l = 1; l <= limit; l++)
        free(lists[l]);
    free(lists);
    free(len_of);
    return maxlen;
}

/* Full codebook lengths: Huffman, then package-merge at 32 if Huffman is longer. */
int oracle_code_lengths(const uint64_t *counts, uint8_t *lens)
{
    int m = oracle_huffman_lengths(counts, lens);
    if (m > MAXLEN)
        m = oracle_limited_lengths(counts, MAXLEN, lens);
    return m;
}

/*
 * Canonical codes: present symbols ordered by (length, value) receive
 * consecutive code values; moving to a longer length appends zeros.
 * Codes are right-aligned in codes[s]; absent symbols get 0.
 */
void oracle_canonical_codes(const uint8_t *lens, uint32_t *codes)
{
    int order[NSYM];
    int n = 0;
    for (int s = 0; s < NSYM; s++) {
        codes[s] = 0;
        if (lens[s] != 0)
            order[n++] = s;
    }
    for (int i = 1; i < n; i++) {
        int s = order[i], j = i - 1;
        while (j >= 0 && (lens[order[j]] > lens[s] ||
                          (lens[order[j]] == lens[s] && order[j] > s))) {
            order[j + 1] = order[j];
            j--;
        }
        order[j + 1] = s;
    }
    uint64_t code = 0;
    for (int i = 0; i < n; i++) {
        if (i > 0)
            code = (code + 1) << (lens[order[i]] - lens[order[i - 1]]);
        codes[order[i]] = (uint32_t)code;
    }
}

/*
 * Bit-serial encoder.  For each weight in order: append its exponent's code
 * MSB-first, one bit at a time, and write its sign+mantissa byte.
 * stream must hold stream_bytes zero-initialised bytes (this function clears
 * them first).  Returns 0, or -1 if a symbol has no code, or -2 if the stream
 * buffer is too small.  *total_bits receives the number of bits written.
 */
int oracle_encode(const uint16_t *w, uint64_t n, const uint8_t *lens, const uint32_t *codes,
                  uint8_t *stream, uint64_t stream_bytes, uint8_t *sm, uint64_t *total_bits)
{
    memset(stream, 0, (size_t)stream_bytes);
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        int e = (w[i] >> 7) & 0xFF;
        int l = lens[e];
        if (l == 0)
            return -1;
        if ((pos + (uint64_t)l + 7) / 8 > stream_bytes)
            return -2;
        for (int k = l - 1; k >= 0; k--) {
            if ((codes[e] >> k) & 1u)
                stream[pos / 8] |= (uint8_t)(0x80u >> (pos % 8));
            pos++;
        }
        sm[i] = (uint8_t)(((w[i] >> 8) & 0x80) | (w[i] & 0x7F));
    }
    *total_bits = pos;
    return 0;
}

/*
 * Auxiliary arrays from the definition, computed from code start positions
 * alone (start_0 = 0, start_{i+1} = start_i + len(e_i)); the stream is not
 * consulted.
 *   gaps[j] (j < n_windows): offset of the first code start in window j, else 255
 *   block_out_pos[t] (t <= n_tiles): number of codes with start < 8*B*T*t
 * window_bits = 8*B, tile_windows = T.  Returns 0, or -1 on a bad argument.
 */
int oracle_aux(const uint16_t *w, uint64_t n, const uint8_t *lens,
               uint32_t window_bits, uint32_t tile_windows,
               uint8_t *gaps, uint64_t n_windows, uint32_t *block_out_pos, uint64_t n_tiles)
{
    if (window_bits == 0 || tile_windows == 0 || n_windows != n_tiles * tile_windows)
        return -1;
    for (uint64_t j = 0; j < n_windows; j++)
        gaps[j] = 255;
    for (uint64_t t = 0; t <= n_tiles; t++)
        block_out_pos[t] = 0;
    uint64_t start = 0;
    uint64_t tile_bits = (uint64_t)window_bits * tile_windows;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t j = start / window_bits;
        if (j >= n_windows)
            return -1;
        if (gaps[j] == 255)
            gaps[j] = (uint8_t)(start - j * window_bits);
        /* this code starts before every tile boundary strictly after it */
        for (uint64_t t = start / tile_bits + 1; t <= n_tiles; t++)
            block_out_pos[t] += 1;
        start += lens[(w[i] >> 7) & 0xFF];
    }
    return 0;
}

/*
 * Faster form of the block_out_pos loop above for large inputs: identical
 * definition, counted per tile and then summed.  Kept separate so the plain
 * loop stays as written for small cases.
 */
int oracle_aux_fast(const uint16_t *w, uint64_t n, const uint8_t *lens,
                    uint32_t window_bits, uint32_t tile_windows,
                    uint8_t *gaps, uint64_t n_windows, uint32_t *block_out_pos, uint64_t n_tiles)
{
    if (window_bits == 0 || tile_windows == 0 || n_windows != n_tiles * tile_windows)
        return -1;
    for (uint64_t j = 0; j < n_windows; j++)
        gaps[j] = 255;
    uint64_t *starts_in_tile = (uint64_t *)calloc((size_t)n_tiles + 1, sizeof(uint64_t));
    uint64_t start = 0;
    uint64_t tile_bits = (uint64_t)window_bits * tile_windows;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t j = start / window_bits;
        if (j >= n_windows) {
            free(starts_in_tile);
            return -1;
        }
        if (gaps[j] == 255)
            gaps[j] = (uint8_t)(start - j * window_bits);
        starts_in_tile[start / tile_bits] += 1;
        start += lens[(w[i] >> 7) & 0xFF];
    }
    uint64_t acc = 0;
    for (uint64_t t = 0; t <= n_tiles; t++) {
        block_out_pos[t] = (uint32_t)acc;
        if (t < n_tiles)
            acc += starts_in_tile[t];
    }
    free(starts_in_tile);
    return 0;
}

/*
 * Textbook canonical-Huffman bit-serial decoder.  From the lengths alone it
 * derives, per length l, the first canonical code first[l], the number of codes
 * count[l] and where symbols of that length begin in the (length, value)
 * order.  Bits are read one at a time from start_bit; a code of length l is
 * complete when first[l] <= v < first[l] + count[l].  Rebuilds
 * w = ((sm & 0x80) << 8) | (e << 7) | (sm & 0x7F).  Stops after n symbols.
 * Returns 0, -1 if a code runs past end_bit, -2 if no code matches in 32 bits.
 */
int oracle_decode(const uint8_t *stream, uint64_t start_bit, uint64_t end_bit,
                  const uint8_t *lens, const uint8_t *sm, uint64_t n, uint16_t *out)
{
    uint32_t count[MAXLEN + 1], first[MAXLEN + 1], offset[MAXLEN + 1];
    int sorted[NSYM];
    int nsorted = 0;
    for (int l = 0; l <= MAXLEN; l++)
        count[l] = 0;
    for (int s = 0; s < NSYM; s++)
        if (lens[s] >= 1 && lens[s] <= MAXLEN)
            count[lens[s]] += 1;
    for (int l = 1; l <= MAXLEN; l++)
        for (int s = 0; s < NSYM; s++)
            if (lens[s] == l)
                sorted[nsorted++] = s;
    uint64_t code = 0;
    uint32_t off = 0;
    for (int l = 1; l <= MAXLEN; l++) {
        first[l] = (uint32_t)code;
        offset[l] = off;
        off += count[l];
        code = (code + count[l]) << 1;
    }
    uint64_t pos = start_bit;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t v = 0;
        int l = 0;
        int sym = -1;
        while (sym < 0) {
            if (pos >= end_bit)
                return -1;
            v = (v << 1) | ((stream[pos / 8] >> (7 - pos % 8)) & 1u);
            pos++;
            l++;
            if (l > MAXLEN)
                return -2;
            if (count[l] != 0 && v >= first[l] && v - first[l] < count[l])
                sym = sorted[offset[l] + (uint32_t)(v - first[l])];
        }
        out[i] = (uint16_t)(((sm[i] & 0x80u) << 8) | ((uint32_t)sym << 7) | (sm[i] & 0x7Fu));
    }
    return 0;
}

/* ------------------------------------------------------------------ FP8 weights
 *
 * The same coding applied to 8-bit floating-point weights ("To Compress or
 * Not? ... Exponent Concentration", abstract: the exponents of FP8 weights are
 * concentrated too).  Formats (OCP 8-bit floating point):
 *   fmt 1 = E4M3: bit 7 sign, bits 6..3 exponent, bits 2..0 mantissa;
 *   fmt 2 = E5M2: bit 7 sign, bits 6..2 exponent, bits 1..0 mantissa.
 * Readings (the pages give no layout): the symbol is the exponent field; the
 * sign and mantissa form one 4-bit value, sign just above the mantissa
 * (E4M3: s<<3 | m; E5M2: s<<2 | m), stored two per byte with the
 * lower-indexed weight in the low nibble.
 */

static int fp8_fields(int fmt, int *ebits, int *mbits)
{
    if (fmt == 1) { *ebits = 4; *mbits = 3; return 0; }
    if (fmt == 2) { *ebits = 5; *mbits = 2; return 0; }
    return -1;
}

/* sym[i] = exponent field of b[i]; smpack nibble i = sign and mantissa of b[i]. */
int oracle_fp8_split(const uint8_t *b, uint64_t n, int fmt, uint8_t *sym, uint8_t *smpack)
{
    int eb, mb;
    if (fp8_fields(fmt, &eb, &mb))
        return -1;
    memset(smpack, 0, (size_t)((n + 1) / 2));
    for (uint64_t i = 0; i < n; i++) {
        unsigned s = b[i] >> 7;
        unsigned e = (b[i] >> mb) & ((1u << eb) - 1u);
        unsigned m = b[i] & ((1u << mb) - 1u);
        unsigned nib = (s << mb) | m;
        sym[i] = (uint8_t)e;
        smpack[i / 2] |= (uint8_t)(nib << (4 * (i % 2)));
    }
    return 0;
}

/* The inverse: out[i] = s << 7 | e << mbits | m. */
int oracle_fp8_merge(const uint8_t *sym, const uint8_t *smpack, uint64_t n, int fmt, uint8_t *out)
{
    int eb, mb;
    if (fp8_fields(fmt, &eb, &mb))
        return -1;
    for (uint64_t i = 0; i < n; i++) {
        unsigned nib = (smpack[i / 2] >> (4 * (i % 2))) & 0xFu;
        unsigned s = (nib >> mb) & 1u;
        unsigned m = nib & ((1u << mb) - 1u);
        out[i] = (uint8_t)((s << 7) | ((unsigned)sym[i] << mb) | m);
    }
    return 0;
}

void oracle_histogram_symbols(const uint8_t *sym, uint64_t n, uint64_t *counts)
{
    for (int s = 0; s < NSYM; s++)
        counts[s] = 0;
    for (uint64_t i = 0; i < n; i++)
        counts[sym[i]] += 1;
}

/* The bit-serial encoder of oracle_encode for a symbol sequence (no sm bytes). */
int oracle_encode_symbols(const uint8_t *sym, uint64_t n, const uint8_t *lens,
                          const uint32_t *codes, uint8_t *stream, uint64_t stream_bytes,
                          uint64_t *total_bits)
{
    memset(stream, 0, (size_t)stream_bytes);
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n; i++) {
        int e = sym[i];
        int l = lens[e];
        if (l == 0)
            return -1;
        if ((pos + (uint64_t)l + 7) / 8 > stream_bytes)
            return -2;
        for (int k = l - 1; k >= 0; k--) {
            if ((codes[e] >> k) & 1u)
                stream[pos / 8] |= (uint8_t)(0x80u >> (pos % 8));
            pos++;
        }
    }
    *total_bits = pos;
    return 0;
}

/* oracle_aux_fast for a symbol sequence: same definitions of gaps and block_out_pos. */
int oracle_aux_symbols(const uint8_t *sym, uint64_t n, const uint8_t *lens,
                       uint32_t window_bits, uint32_t tile_windows,
                       uint8_t *gaps, uint64_t n_windows, uint32_t *block_out_pos, uint64_t n_tiles)
{
    if (window_bits == 0 || tile_windows == 0 || n_windows != n_tiles * tile_windows)
        return -1;
    for (uint64_t j = 0; j < n_windows; j++)
        gaps[j] = 255;
    uint64_t *starts_in_tile = (uint64_t *)calloc((size_t)n_tiles + 1, sizeof(uint64_t));
    uint64_t start = 0;
    uint64_t tile_bits = (uint64_t)window_bits * tile_windows;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t j = start / window_bits;
        if (j >= n_windows) {
            free(starts_in_tile);
            return -1;
        }
        if (gaps[j] == 255)
            gaps[j] = (uint8_t)(start - j * window_bits);
        starts_in_tile[start / tile_bits] += 1;
        start += lens[sym[i]];
    }
    uint64_t acc = 0;
    for (uint64_t t = 0; t <= n_tiles; t++) {
        block_out_pos[t] = (uint32_t)acc;
        if (t < n_tiles)
            acc += starts_in_tile[t];
    }
    free(starts_in_tile);
    return 0;
}

/* The textbook decoder of oracle_decode, returning the symbols themselves. */
int oracle_decode_symbols(const uint8_t *stream, uint64_t start_bit, uint64_t end_bit,
                          const uint8_t *lens, uint64_t n, uint8_t *sym_out)
{
    uint32_t count[MAXLEN + 1], first[MAXLEN + 1], offset[MAXLEN + 1];
    int sorted[NSYM];
    int nsorted = 0;
    for (int l = 0; l <= MAXLEN; l++)
        count[l] = 0;
    for (int s = 0; s < NSYM; s++)
        if (lens[s] >= 1 && lens[s] <= MAXLEN)
            count[lens[s]] += 1;
    for (int l = 1; l <= MAXLEN; l++)
        for (int s = 0; s < NSYM; s++)
            if (lens[s] == l)
                sorted[nsorted++] = s;
    uint64_t code = 0;
    uint32_t off = 0;
    for (int l = 1; l <= MAXLEN; l++) {
        first[l] = (uint32_t)code;
        offset[l] = off;
        off += count[l];
        code = (code + count[l]) << 1;
    }
    uint64_t pos = start_bit;
    for (uint64_t i = 0; i < n; i++) {
        uint64_t v = 0;
        int l = 0;
        int sym = -1;
        while (sym < 0) {
            if (pos >= end_bit)
                return -1;
            v = (v << 1) | ((stream[pos / 8] >> (7 - pos % 8)) & 1u);
            pos++;
            l++;
            if (l > MAXLEN)
                return -2;
            if (count[l] != 0 && v >= first[l] && v - first[l] < count[l])
                sym = sorted[offset[l] + (uint32_t)(v - first[l])];
        }
        sym_out[i] = (uint8_t)sym;
    }
    return 0;
}
