/*
 * Host codec and oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Test infrastructure: built by tests/test_sanitize.py with gcc/g++ and
 * -fsanitize=address,undefined, linking the library's host codec
 * (df11_host.cpp, through include/df11.h) and the oracle (oracle/df11_oracle.c).
 * It runs the codec and the oracle on seeded units of many shapes and checks
 * that they agree byte for byte, that the oracle's own pins hold (Kraft sum,
 * brute-force optimal costs, the 32-bit limit, round trips), and that every
 * entry point rejects bad arguments; any memory error or undefined behaviour
 * in either aborts the run.  Prints "sanitize ok" at the end.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "df11.h"

/* the oracle's C entry points (oracle/df11_oracle.c) */
void oracle_histogram(const uint16_t *w, uint64_t n, uint64_t *counts);
int oracle_huffman_lengths(const uint64_t *counts, uint8_t *lens);
int oracle_limited_lengths(const uint64_t *counts, int limit, uint8_t *lens);
int oracle_code_lengths(const uint64_t *counts, uint8_t *lens);
void oracle_canonical_codes(const uint8_t *lens, uint32_t *codes);
int oracle_encode(const uint16_t *w, uint64_t n, const uint8_t *lens, const uint32_t *codes,
                  uint8_t *stream, uint64_t stream_bytes, uint8_t *sm, uint64_t *total_bits);
int oracle_aux(const uint16_t *w, uint64_t n, const uint8_t *lens, uint32_t window_bits,
               uint32_t tile_windows, uint8_t *gaps, uint64_t n_windows, uint32_t *block_out_pos,
               uint64_t n_tiles);
int oracle_aux_fast(const uint16_t *w, uint64_t n, const uint8_t *lens, uint32_t window_bits,
                    uint32_t tile_windows, uint8_t *gaps, uint64_t n_windows,
                    uint32_t *block_out_pos, uint64_t n_tiles);
int oracle_decode(const uint8_t *stream, uint64_t start_bit, uint64_t end_bit,
                  const uint8_t *lens, const uint8_t *sm, uint64_t n, uint16_t *out);
int oracle_fp8_split(const uint8_t *b, uint64_t n, int fmt, uint8_t *sym, uint8_t *smpack);
int oracle_fp8_merge(const uint8_t *sym, const uint8_t *smpack, uint64_t n, int fmt, uint8_t *out);
void oracle_histogram_symbols(const uint8_t *sym, uint64_t n, uint64_t *counts);
int oracle_encode_symbols(const uint8_t *sym, uint64_t n, const uint8_t *lens,
                          const uint32_t *codes, uint8_t *stream, uint64_t stream_bytes,
                          uint64_t *total_bits);
int oracle_aux_symbols(const uint8_t *sym, uint64_t n, const uint8_t *lens, uint32_t window_bits,
                       uint32_t tile_windows, uint8_t *gaps, uint64_t n_windows,
                       uint32_t *block_out_pos, uint64_t n_tiles);
int oracle_decode_symbols(const uint8_t *stream, uint64_t start_bit, uint64_t end_bit,
                          const uint8_t *lens, uint64_t n, uint8_t *out);

static int failures = 0;
#define CHECK(c)                                                                         \
    do {                                                                                 \
        if (!(c)) {                                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);        \
            failures++;                                                                  \
        }                                                                                \
    } while (0)

/* splitmix64: a counter-based generator of its published definition */
static uint64_t rng_state;
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* A BF16 pattern of kind k: 0 narrow (a bell-shaped exponent spread around
 * 121, from the sum of uniforms), 1 raw 16-bit patterns, 2 three exponents,
 * 3 one exponent. */
static uint16_t weight(int kind) {
    const uint64_t r = next_u64();
    const uint16_t sm = (uint16_t)(((r >> 8) & 0x80) << 8 | (r & 0x7F));
    switch (kind) {
    case 0: {
        int e = 121;
        for (int k = 0; k < 6; k++) e += (int)((r >> (16 + 4 * k)) & 3) - 1;  /* -6 .. +12 spread */
        if (((r >> 50) & 16383) == 0) e = 100 + (int)((r >> 40) & 31);      /* rare outliers */
        return (uint16_t)(sm | (uint16_t)(e << 7));
    }
    case 1: return (uint16_t)r;
    case 2: return (uint16_t)(sm | (uint16_t)((120 + (r >> 30) % 3) << 7));
    default: return (uint16_t)(sm | (uint16_t)(121 << 7));
    }
}

static uint64_t cost(const uint64_t *c, const uint8_t *l) {
    uint64_t s = 0;
    for (int i = 0; i < 256; i++) s += c[i] * l[i];
    return s;
}

static int kraft_is_one(const uint8_t *l) {
    uint64_t s = 0;
    int n = 0;
    for (int i = 0; i < 256; i++)
        if (l[i]) {
            s += (uint64_t)1 << (32 - l[i]);
            n++;
        }
    return n == 0 || s == ((uint64_t)1 << 32);
}

/* One BF16 unit of n_t tensors through the codec and the oracle. */
static void check_bf16_unit(uint16_t **t, const uint64_t *numel, uint32_t n_t, uint32_t tw) {
    uint64_t n = 0;
    for (uint32_t k = 0; k < n_t; k++) n += numel[k];
    if (n == 0) return;
    uint16_t *all = malloc(n * 2);
    for (uint32_t k = 0, g = 0; k < n_t; g += (uint32_t)numel[k], k++) memcpy(all + g, t[k], numel[k] * 2);

    df11_codebook *cb = malloc(sizeof(df11_codebook));
    const int rc = df11_build_codebook((const uint16_t *const *)t, numel, n_t, cb);
    if (rc != DF11_OK) {
        fprintf(stderr, "df11_build_codebook: %d (%s) for n=%llu tensors=%u\n", rc,
                df11_status_string(rc), (unsigned long long)n, n_t);
        failures++;
        free(cb);
        free(all);
        return;
    }
    uint64_t counts[256];
    uint8_t olens[256];
    uint32_t ocodes[256];
    oracle_histogram(all, n, counts);
    oracle_code_lengths(counts, olens);
    CHECK(kraft_is_one(cb->code_len) && cb->max_len <= 32);
    CHECK(cost(counts, cb->code_len) == cost(counts, olens));
    /* the stream comparison takes the library's lengths (several optimal
     * codes exist only when the 32-bit limit binds) with the oracle's own
     * canonical codes for them */
    oracle_canonical_codes(cb->code_len, ocodes);
    for (int s = 0; s < 256; s++) CHECK(!cb->code_len[s] || cb->code[s] == ocodes[s]);

    df11_sizes sz;
    CHECK(df11_encode_size(cb, (const uint16_t *const *)t, numel, n_t, tw, 8, &sz) == DF11_OK);
    df11_host_stream hs;
    memset(&hs, 0, sizeof hs);
    hs.stream = malloc(sz.stream_bytes);
    hs.sm = malloc(sz.sm_bytes);
    hs.gaps = malloc(sz.n_windows ? sz.n_windows : 1);
    hs.block_out_pos = malloc(sz.bop_entries * 4);
    hs.tensor_offsets = malloc((n_t + 1) * 8);
    hs.tensor_tiles = malloc(2 * n_t * 8 + 8);
    hs.stream_capacity = sz.stream_bytes;
    hs.sm_capacity = sz.sm_bytes;
    hs.gaps_capacity = sz.n_windows;
    hs.bop_capacity = sz.bop_entries;
    hs.n_tensors = n_t;
    CHECK(df11_encode(cb, (const uint16_t *const *)t, numel, n_t, tw, 8, &hs) == DF11_OK);
    hs.stream_capacity -= 1; /* one byte short is refused */
    CHECK(df11_encode(cb, (const uint16_t *const *)t, numel, n_t, tw, 8, &hs) == DF11_E_CAPACITY);

    const uint64_t ob = (sz.total_bits + 7) / 8 + 8;
    uint8_t *ostream = calloc(ob, 1), *osm = malloc(n);
    uint64_t total = 0;
    CHECK(oracle_encode(all, n, cb->code_len, ocodes, ostream, ob, osm, &total) == 0);
    CHECK(total == sz.total_bits && total == hs.total_bits);
    CHECK(memcmp(hs.stream, ostream, (total + 7) / 8) == 0);
    for (uint64_t i = (total + 7) / 8; i < sz.stream_bytes; i++) CHECK(hs.stream[i] == 0);
    CHECK(memcmp(hs.sm, osm, n) == 0);
    uint8_t *ogaps = malloc(sz.n_windows ? sz.n_windows : 1);
    uint32_t *obop = malloc(sz.bop_entries * 4);
    CHECK(oracle_aux_fast(all, n, cb->code_len, 64, tw, ogaps, sz.n_windows, obop, sz.n_tiles) == 0);
    CHECK(memcmp(hs.gaps, ogaps, sz.n_windows) == 0);
    CHECK(memcmp(hs.block_out_pos, obop, sz.bop_entries * 4) == 0);
    if (n < 200000) {
        CHECK(oracle_aux(all, n, cb->code_len, 64, tw, ogaps, sz.n_windows, obop, sz.n_tiles) == 0);
        CHECK(memcmp(hs.block_out_pos, obop, sz.bop_entries * 4) == 0);
    }
    uint16_t *dec = malloc(n * 2);
    CHECK(oracle_decode(hs.stream, 0, total, cb->code_len, hs.sm, n, dec) == 0);
    CHECK(memcmp(dec, all, n * 2) == 0);

    /* tensor ranges from per-tensor histograms equal the encoder's */
    uint64_t *pc = calloc((size_t)n_t * 256, 8);
    uint32_t *last = calloc(n_t, 4);
    for (uint32_t k = 0; k < n_t; k++) {
        oracle_histogram(t[k], numel[k], pc + (size_t)k * 256);
        last[k] = numel[k] ? t[k][numel[k] - 1] : 0;
    }
    uint64_t *offs = malloc((n_t + 1) * 8), *tiles = malloc(2 * n_t * 8 + 8);
    CHECK(df11_tensor_ranges_from_counts(0, cb, pc, last, n_t, tw, 8, offs, tiles) == DF11_OK);
    CHECK(memcmp(offs, hs.tensor_offsets, (n_t + 1) * 8) == 0);
    CHECK(memcmp(tiles, hs.tensor_tiles, 2 * n_t * 8) == 0);

    free(pc); free(last); free(offs); free(tiles);
    free(dec); free(ogaps); free(obop); free(ostream); free(osm);
    free(hs.stream); free(hs.sm); free(hs.gaps); free(hs.block_out_pos);
    free(hs.tensor_offsets); free(hs.tensor_tiles);
    free(cb); free(all);
}

/* One FP8 unit (fmt 1 = E4M3, 2 = E5M2) through the codec and the oracle. */
static void check_fp8_unit(const uint8_t *b, uint64_t n, int fmt) {
    const void *tp[2] = {b, b + n / 3};
    uint64_t numel[2] = {n / 3, n - n / 3};
    df11_codebook *cb = malloc(sizeof(df11_codebook));
    CHECK(df11_build_codebook_fmt((uint32_t)fmt, tp, numel, 2, cb) == DF11_OK);
    df11_sizes sz;
    CHECK(df11_encode_size_fmt((uint32_t)fmt, cb, tp, numel, 2, 64, 8, &sz) == DF11_OK);
    df11_host_stream hs;
    memset(&hs, 0, sizeof hs);
    hs.stream = malloc(sz.stream_bytes);
    hs.sm = malloc(sz.sm_bytes);
    hs.gaps = malloc(sz.n_windows ? sz.n_windows : 1);
    hs.block_out_pos = malloc(sz.bop_entries * 4);
    hs.tensor_offsets = malloc(3 * 8);
    hs.tensor_tiles = malloc(4 * 8);
    hs.stream_capacity = sz.stream_bytes;
    hs.sm_capacity = sz.sm_bytes;
    hs.gaps_capacity = sz.n_windows;
    hs.bop_capacity = sz.bop_entries;
    hs.n_tensors = 2;
    CHECK(df11_encode_fmt((uint32_t)fmt, cb, tp, numel, 2, 64, 8, &hs) == DF11_OK);
    uint8_t *sym = malloc(n), *smp = malloc((n + 1) / 2);
    CHECK(oracle_fp8_split(b, n, fmt, sym, smp) == 0);
    uint64_t counts[256];
    uint8_t olens[256];
    uint32_t ocodes[256];
    oracle_histogram_symbols(sym, n, counts);
    oracle_code_lengths(counts, olens);
    CHECK(memcmp(olens, cb->code_len, 256) == 0);
    oracle_canonical_codes(olens, ocodes);
    const uint64_t ob = (sz.total_bits + 7) / 8 + 8;
    uint8_t *ostream = calloc(ob, 1);
    uint64_t total = 0;
    CHECK(oracle_encode_symbols(sym, n, olens, ocodes, ostream, ob, &total) == 0);
    CHECK(total == hs.total_bits && memcmp(ostream, hs.stream, (total + 7) / 8) == 0);
    CHECK(memcmp(smp, hs.sm, (n + 1) / 2) == 0);
    uint8_t *ogaps = malloc(sz.n_windows ? sz.n_windows : 1);
    uint32_t *obop = malloc(sz.bop_entries * 4);
    CHECK(oracle_aux_symbols(sym, n, olens, 64, 64, ogaps, sz.n_windows, obop, sz.n_tiles) == 0);
    CHECK(memcmp(ogaps, hs.gaps, sz.n_windows) == 0);
    CHECK(memcmp(obop, hs.block_out_pos, sz.bop_entries * 4) == 0);
    uint8_t *dsym = malloc(n), *back = malloc(n);
    CHECK(oracle_decode_symbols(hs.stream, 0, total, olens, n, dsym) == 0);
    CHECK(oracle_fp8_merge(dsym, hs.sm, n, fmt, back) == 0);
    CHECK(memcmp(back, b, n) == 0);
    free(dsym); free(back); free(ogaps); free(obop); free(ostream); free(sym); free(smp);
    free(hs.stream); free(hs.sm); free(hs.gaps); free(hs.block_out_pos);
    free(hs.tensor_offsets); free(hs.tensor_tiles); free(cb);
}

/* Brute-force optimal cost over lengths 1..maxl of n symbols (Kraft <= 1). */
static uint64_t brute(const uint64_t *w, int n, int maxl, int i, uint64_t kraft, uint64_t acc) {
    if (kraft > ((uint64_t)1 << 20)) return UINT64_MAX;
    if (i == n) return acc;
    uint64_t best = UINT64_MAX;
    for (int l = 1; l <= maxl; l++) {
        const uint64_t c = brute(w, n, maxl, i + 1, kraft + ((uint64_t)1 << (20 - l)), acc + w[i] * l);
        if (c < best) best = c;
    }
    return best;
}

static void oracle_pins(void) {
    for (int rep = 0; rep < 30; rep++) {
        uint64_t c[256] = {0};
        const int n = 2 + (int)(next_u64() % 5);
        uint64_t w[8];
        for (int i = 0; i < n; i++) c[10 + 3 * i] = w[i] = 1 + next_u64() % 50;
        uint8_t l[256];
        oracle_huffman_lengths(c, l);
        CHECK(kraft_is_one(l));
        CHECK(cost(c, l) == brute(w, n, n - 1, 0, 0, 0));
        const int lim = 3;
        if (n <= (1 << lim)) {
            CHECK(oracle_limited_lengths(c, lim, l) >= 0);
            CHECK(cost(c, l) == brute(w, n, lim, 0, 0, 0));
        }
    }
    /* Fibonacci counts force depth 39 > 32 */
    uint64_t c[256] = {0}, a = 1, b = 1;
    for (int i = 0; i < 40; i++) {
        c[i] = a;
        const uint64_t t = a + b;
        a = b;
        b = t;
    }
    uint8_t l[256], h[256];
    oracle_huffman_lengths(c, h);
    oracle_code_lengths(c, l);
    int mx = 0, mh = 0;
    for (int s = 0; s < 256; s++) {
        if (l[s] > mx) mx = l[s];
        if (h[s] > mh) mh = h[s];
    }
    CHECK(mh > 32 && mx == 32 && kraft_is_one(l) && cost(c, l) >= cost(c, h));
    /* dyadic counts: exact lengths */
    uint64_t d[256] = {0};
    d[0] = 8; d[1] = 4; d[2] = 2; d[3] = 1; d[4] = 1;
    oracle_code_lengths(d, l);
    CHECK(l[0] == 1 && l[1] == 2 && l[2] == 3 && l[3] == 4 && l[4] == 4);
}

static void argument_errors(void) {
    df11_codebook *cb = malloc(sizeof(df11_codebook));
    uint16_t w[4] = {0x3F80, 0x4000, 0x3F80, 0xBF80};
    const uint16_t *t[1] = {w};
    uint64_t numel[1] = {4};
    CHECK(df11_build_codebook(NULL, numel, 1, cb) == DF11_E_INVALID);
    CHECK(df11_build_codebook(t, numel, 1, NULL) == DF11_E_INVALID);
    CHECK(df11_build_codebook(t, numel, 1, cb) == DF11_OK);
    df11_sizes sz;
    CHECK(df11_encode_size(cb, t, numel, 1, 100, 8, &sz) == DF11_E_INVALID);
    CHECK(df11_encode_size(cb, t, numel, 1, 64, 8, &sz) == DF11_OK);
    uint64_t cnt[256] = {0};
    CHECK(df11_build_codebook_from_counts(cnt, cb) == DF11_E_INVALID);
    CHECK(df11_tensor_ranges_from_counts(0, cb, NULL, NULL, 1, 64, 8, NULL, NULL) == DF11_E_INVALID);
    uint16_t out[32];
    CHECK(df11_gemm_order(w, 3, 32, out) == DF11_E_INVALID);
    free(cb);
}

int main(void) {
    rng_state = 12345;
    oracle_pins();
    argument_errors();
    static const uint64_t sizes[] = {1, 7, 64, 4095, 4096, 4097, 100003, 2500001};
    static const uint32_t layouts[] = {64, 256, 512};
    for (int kind = 0; kind < 4; kind++)
        for (int si = 0; si < 8; si++) {
            const uint64_t n = sizes[si];
            if (kind != 0 && n > 200000) continue;
            uint16_t *a = malloc(n * 2);
            for (uint64_t i = 0; i < n; i++) a[i] = weight(kind);
            /* one tensor, then three (one of them empty) */
            uint16_t *t1[1] = {a};
            uint64_t n1[1] = {n};
            check_bf16_unit(t1, n1, 1, layouts[(kind + si) % 3]);
            uint16_t *t3[3] = {a, a + n / 2, a + n / 2};
            uint64_t n3[3] = {n / 2, 0, n - n / 2};
            check_bf16_unit(t3, n3, 3, 64);
            free(a);
        }
    /* 32-bit codes: 34 exponents with Fibonacci counts (Huffman depth 33,
     * so package-merge limits the code to 32 bits), in a shuffled order */
    {
        uint64_t f[34], tot = 0;
        f[0] = f[1] = 1;
        for (int i = 2; i < 34; i++) f[i] = f[i - 1] + f[i - 2];
        for (int i = 0; i < 34; i++) tot += f[i];
        uint16_t *a = malloc(tot * 2);
        uint64_t g = 0;
        for (int i = 0; i < 34; i++)
            for (uint64_t k = 0; k < f[i]; k++) a[g++] = (uint16_t)(((90 + i) << 7) | (k & 0x807F));
        for (uint64_t i = tot - 1; i > 0; i--) {
            const uint64_t j = next_u64() % (i + 1);
            const uint16_t x = a[i];
            a[i] = a[j];
            a[j] = x;
        }
        uint64_t c[256] = {0};
        uint8_t h[256];
        oracle_histogram(a, tot, c);
        oracle_huffman_lengths(c, h);
        int mh = 0;
        for (int s = 0; s < 256; s++) mh = h[s] > mh ? h[s] : mh;
        CHECK(mh == 33);
        uint16_t *t1[1] = {a};
        check_bf16_unit(t1, &tot, 1, 64);
        free(a);
    }
    for (int fmt = 1; fmt <= 2; fmt++) {
        const uint64_t n = 150001;
        uint8_t *b = malloc(n);
        for (uint64_t i = 0; i < n; i++) {
            const uint64_t r = next_u64();
            b[i] = (uint8_t)((r & 0x83) | ((fmt == 1 ? (5 + (r >> 20) % 4) << 3 : (12 + (r >> 20) % 5) << 2)));
            if ((r >> 40) % 97 == 0) b[i] = (uint8_t)(r >> 8);
        }
        check_fp8_unit(b, n, fmt);
        free(b);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("sanitize ok\n");
    return 0;
}
