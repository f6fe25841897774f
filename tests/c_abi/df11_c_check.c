/*
 * A C99 user of include/df11.h: encodes a two-tensor BF16 unit with the host
 * calls and checks the results' invariants; built with -DDF11_C_CHECK_GPU it
 * also uploads the unit, decompresses it with df11_decompress_block and
 * df11_decompress_tensor and compares every output with the input bits.
 * Exit status 0 on success; prints the first failed check otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "df11.h"

#ifdef DF11_C_CHECK_GPU
#include <hip/hip_runtime_api.h>
#endif

#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                    \
        }                                                                \
    } while (0)

/* BF16 bits of a roughly Gaussian value (sum of four uniforms), scaled */
static uint16_t next_weight(uint64_t *s) {
    float acc = 0.0f;
    for (int i = 0; i < 4; i++) {
        *s = *s * 6364136223846793005ull + 1442695040888963407ull;
        acc += (float)((*s >> 40) & 0xFFFFFF) / 16777216.0f - 0.5f;
    }
    acc *= 0.04f;
    uint32_t u;
    memcpy(&u, &acc, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

int main(void) {
    const uint64_t numel[2] = {70001, 12288};
    uint16_t *w[2];
    uint64_t seed = 7;
    for (int k = 0; k < 2; k++) {
        w[k] = (uint16_t *)malloc(numel[k] * 2);
        CHECK(w[k] != NULL);
        for (uint64_t i = 0; i < numel[k]; i++) w[k][i] = next_weight(&seed);
    }
    const uint16_t *const tensors[2] = {w[0], w[1]};

    df11_codebook cb;
    CHECK(df11_build_codebook(tensors, numel, 2, &cb) == DF11_OK);
    CHECK(cb.n_luts >= 1 && cb.max_len >= 1 && cb.max_len <= DF11_MAX_CODE_LEN);
    CHECK(df11_build_codebook(tensors, numel, 0, &cb) == DF11_E_INVALID);  /* no weights */
    CHECK(df11_build_codebook(tensors, numel, 2, &cb) == DF11_OK);

    df11_sizes sz;
    CHECK(df11_encode_size(&cb, tensors, numel, 2, 64, 8, &sz) == DF11_OK);
    CHECK(sz.n_weights == numel[0] + numel[1]);
    CHECK(sz.n_windows == sz.n_tiles * 64 && sz.bop_entries == sz.n_tiles + 1);

    df11_host_stream hs;
    memset(&hs, 0, sizeof hs);
    hs.stream = (uint8_t *)malloc(sz.stream_bytes);
    hs.sm = (uint8_t *)malloc(sz.sm_bytes);
    hs.gaps = (uint8_t *)malloc(sz.n_windows);
    hs.block_out_pos = (uint32_t *)malloc(4 * sz.bop_entries);
    hs.tensor_offsets = (uint64_t *)malloc(8 * 3);
    hs.tensor_tiles = (uint64_t *)malloc(8 * 4);
    hs.stream_capacity = sz.stream_bytes;
    hs.sm_capacity = sz.sm_bytes;
    hs.gaps_capacity = sz.n_windows;
    hs.bop_capacity = sz.bop_entries;
    hs.n_tensors = 2;
    CHECK(hs.stream && hs.sm && hs.gaps && hs.block_out_pos && hs.tensor_offsets && hs.tensor_tiles);
    hs.sm_capacity = sz.sm_bytes - 1;  /* too small: refused */
    CHECK(df11_encode(&cb, tensors, numel, 2, 64, 8, &hs) == DF11_E_CAPACITY);
    hs.sm_capacity = sz.sm_bytes;
    CHECK(df11_encode(&cb, tensors, numel, 2, 64, 8, &hs) == DF11_OK);
    CHECK(hs.n_weights == sz.n_weights && hs.total_bits == sz.total_bits && hs.n_tiles == sz.n_tiles);
    CHECK(hs.tensor_offsets[0] == 0 && hs.tensor_offsets[1] == numel[0] &&
          hs.tensor_offsets[2] == sz.n_weights);
    CHECK(hs.block_out_pos[0] == 0 && hs.block_out_pos[hs.n_tiles] == sz.n_weights);
    for (uint64_t t = 0; t < hs.n_tiles; t++) {
        CHECK(hs.block_out_pos[t] <= hs.block_out_pos[t + 1]);
        CHECK(hs.block_out_pos[t + 1] - hs.block_out_pos[t] <= hs.max_tile_symbols);
    }
    for (uint64_t i = 0; i < sz.n_weights; i++) {  /* sign and mantissa bytes, raw */
        const uint16_t x = i < numel[0] ? w[0][i] : w[1][i - numel[0]];
        CHECK(hs.sm[i] == (uint8_t)(((x >> 8) & 0x80) | (x & 0x7F)));
    }
    CHECK(strlen(df11_status_string(DF11_E_CORRUPT)) > 0);
    printf("host: %llu weights, %llu tiles, %.3f payload bits/weight\n",
           (unsigned long long)sz.n_weights, (unsigned long long)hs.n_tiles,
           8.0 + (double)hs.total_bits / (double)sz.n_weights);

#ifdef DF11_C_CHECK_GPU
    df11_device_stream ds;
    memset(&ds, 0, sizeof ds);
    void *d[5];
    const size_t bytes[5] = {sz.stream_bytes, sz.sm_bytes, sz.n_windows, 4 * sz.bop_entries,
                             df11_table_bytes(&cb)};
    const void *src[5] = {hs.stream, hs.sm, hs.gaps, hs.block_out_pos, &cb.multi[0]};
    for (int i = 0; i < 5; i++) {
        CHECK(hipMalloc(&d[i], bytes[i]) == hipSuccess);
        CHECK(hipMemcpy(d[i], src[i], bytes[i], hipMemcpyHostToDevice) == hipSuccess);
    }
    ds.stream = (const uint8_t *)d[0];
    ds.sm = (const uint8_t *)d[1];
    ds.gaps = (const uint8_t *)d[2];
    ds.block_out_pos = (const uint32_t *)d[3];
    ds.tables = d[4];
    ds.tensor_offsets = hs.tensor_offsets;
    ds.tensor_tiles = hs.tensor_tiles;
    ds.n_tensors = 2;
    ds.tile_windows = hs.tile_windows;
    ds.window_bytes = hs.window_bytes;
    ds.max_tile_symbols = hs.max_tile_symbols;
    ds.n_weights = hs.n_weights;
    ds.total_bits = hs.total_bits;
    ds.n_tiles = hs.n_tiles;
    ds.n_luts = cb.n_luts;
    ds.format = hs.format;
    uint16_t *d_out;
    int32_t *d_status;
    CHECK(hipMalloc((void **)&d_out, 2 * sz.n_weights) == hipSuccess);
    CHECK(hipMalloc((void **)&d_status, 4) == hipSuccess);
    CHECK(hipMemset(d_status, 0, 4) == hipSuccess);
    CHECK(hipMemset(d_out, 0xFF, 2 * sz.n_weights) == hipSuccess);
    CHECK(df11_decompress_block(&ds, d_out, d_status, NULL) == DF11_OK);
    uint16_t *out = (uint16_t *)malloc(2 * sz.n_weights);
    int32_t status = -1;
    CHECK(hipMemcpy(out, d_out, 2 * sz.n_weights, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(status == DF11_OK);
    CHECK(memcmp(out, w[0], numel[0] * 2) == 0 && memcmp(out + numel[0], w[1], numel[1] * 2) == 0);
    /* the second tensor alone (its offset, 70001, is not a multiple of 8: refused) */
    CHECK(df11_decompress_tensor(&ds, 1, d_out, d_status, NULL) == DF11_E_INVALID);
    CHECK(hipMemset(d_out, 0xFF, 2 * sz.n_weights) == hipSuccess);
    CHECK(df11_decompress_tensor(&ds, 0, d_out, d_status, NULL) == DF11_OK);
    CHECK(hipMemcpy(out, d_out, 2 * numel[0], hipMemcpyDeviceToHost) == hipSuccess);
    CHECK(memcmp(out, w[0], numel[0] * 2) == 0);
    /* the first decode phase alone: each tile's window counts add up to its
       block_out_pos difference */
    uint32_t *d_counts;
    CHECK(hipMalloc((void **)&d_counts, 4 * sz.n_windows) == hipSuccess);
    CHECK(df11_window_counts(&ds, d_counts, NULL) == DF11_OK);
    uint32_t *counts = (uint32_t *)malloc(4 * sz.n_windows);
    CHECK(hipMemcpy(counts, d_counts, 4 * sz.n_windows, hipMemcpyDeviceToHost) == hipSuccess);
    for (uint64_t t = 0; t < sz.n_tiles; t++) {
        uint64_t c = 0;
        for (uint64_t j = 64 * t; j < 64 * (t + 1); j++) c += counts[j];
        CHECK(c == (uint64_t)hs.block_out_pos[t + 1] - hs.block_out_pos[t]);
    }
    printf("gpu: decompress_block and decompress_tensor bit-exact; window counts consistent\n");
#endif
    return 0;
}
