/*
 * df11.h -- C ABI of an MI355X (gfx950) library for DFloat11-style lossless
 * BF16 weight compression.
 *
 * Method: "70% Size, 100% Accuracy: Lossless LLM Compression for Efficient GPU
 * Inference via Dynamic-Length Float (DFloat11)", abstract.  Each BF16 weight
 * keeps its sign and 7 mantissa bits verbatim in one byte; its 8-bit exponent
 * is replaced by a variable-length code chosen from exponent frequencies; a GPU
 * kernel restores bit-identical BF16 values using compact hierarchical lookup
 * tables held in on-chip memory, a two-phase scheme whose small auxiliary
 * arrays tell each thread where to read and where to write, and one launch
 * per transformer block.  The BF16 field split (1 sign, 8 exponent, 7
 * mantissa bits; only the exponent carries low entropy) and offline Huffman
 * coding of the exponents are from "Compressing LLMs without Compromise",
 * sections "Where the redundancy lives" and "Three ways to spend the savings".
 *
 * Terms used below:
 *   weight w      uint16 BF16 bit pattern
 *   exponent e    (w >> 7) & 0xFF, the coded symbol (all 256 values allowed,
 *                 including those of Inf/NaN and zero/subnormals)
 *   sm byte       ((w >> 8) & 0x80) | (w & 0x7F), stored raw
 *   unit          the tensors compressed together under one codebook and
 *                 decompressed by one launch (a tensor, or all weight tensors
 *                 of one transformer block, concatenated in order)
 *   window        B = 8 consecutive stream bytes, decoded serially from its gap
 *   tile          T consecutive windows whose outputs are placed by one
 *                 block_out_pos entry: T = 64 is one wave64 per tile (the
 *                 default), T = 256 one workgroup of 256 threads, T = 512 one
 *                 workgroup with two adjacent windows per thread
 *
 * Stream format.  Codes are canonical (symbols ordered by (length, value)
 * take consecutive codes), at most 32 bits long, and written MSB-first: bit j
 * of the stream is bit 7 - (j % 8) of byte j / 8.  gaps[j] is the offset, in
 * bits, of the first code that starts in window j (always < 32), or 255 when
 * no code starts there.  block_out_pos[t] is the number of codes that start
 * before tile t, so tile t writes outputs [block_out_pos[t], block_out_pos[t+1]).
 *
 * Conventions.  Every call returns a df11_status.  No call allocates device
 * memory, frees caller memory or synchronises a stream; host calls may use
 * worker threads internally and are thread-safe.  The only global state is
 * the per-device address of df11_decompress_gemv_noalloc's static workspace,
 * set once under a lock.
 */
#ifndef DF11_H
#define DF11_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DF11_MAX_CODE_LEN 32   /* longest code; 4 levels of 8-bit-indexed tables */
#define DF11_MAX_LUTS 64       /* table budget: 64 x 256 x 2 B = 32 KiB of LDS */
#define DF11_STREAM_PAD 16     /* zero bytes after the last window (look-ahead) */

typedef enum df11_status {
    DF11_OK = 0,
    DF11_E_INVALID = 1,     /* bad argument: null pointer, size, layout, alignment */
    DF11_E_LUT_BUDGET = 2,  /* codebook needs more than DF11_MAX_LUTS tables */
    DF11_E_SYMBOL = 3,      /* an input exponent has no code in the codebook */
    DF11_E_CAPACITY = 4,    /* a caller buffer is smaller than df11_encode_size says */
    DF11_E_HIP = 5,         /* the HIP runtime rejected the launch */
    DF11_E_CORRUPT = 6      /* written to *d_status by the kernel: inconsistent stream */
} df11_status;

/* An opaque hipStream_t (0 = the null stream). */
typedef void *df11_hip_stream;

/*
 * Weight formats.  The coded symbol is always the exponent field; the sign
 * and mantissa bits are stored raw.  FP8 follows "To Compress or Not? ...
 * Exponent Concentration", abstract (FP8 weight exponents are concentrated
 * too); the pages give no layout, so these are readings of the OCP 8-bit
 * formats:
 *   DF11_FORMAT_BF16      16-bit weights: symbol (w >> 7) & 0xFF, one sm byte
 *                         ((w >> 8) & 0x80) | (w & 0x7F) per weight
 *   DF11_FORMAT_FP8_E4M3  8-bit weights: symbol (b >> 3) & 0xF, one nibble
 *                         (sign << 3) | (b & 7) per weight
 *   DF11_FORMAT_FP8_E5M2  8-bit weights: symbol (b >> 2) & 0x1F, one nibble
 *                         (sign << 2) | (b & 3) per weight
 * Nibbles are stored two per byte, the lower-indexed weight in the low
 * nibble.  FP8 units use 64-window tiles (T = 64).
 */
typedef enum df11_format {
    DF11_FORMAT_BF16 = 0,
    DF11_FORMAT_FP8_E4M3 = 1,
    DF11_FORMAT_FP8_E5M2 = 2
} df11_format;

#define DF11_MULTI_BITS 10      /* index width of the multi-symbol decode table */
#define DF11_COUNT_BITS 12      /* index width of the code-start (count) table */

/*
 * Codebook (caller-owned POD, about 46 KiB).  code_len[s] == 0 means symbol s
 * has no code.  Three kinds of 8-bit-or-wider-indexed tables are derived from
 * the codes ("compact, hierarchical lookup tables", DFloat11 abstract); each is
 * indexed by the leading bits of the stream at a code boundary, MSB-first:
 *
 *   lut[k][256]  hierarchical single-code tables.  Table 0 is indexed by the
 *                top 8 bits of a 32-bit left-aligned window, a level-k table
 *                by the next 8 bits.  Entries:
 *                  leaf     bit 15 = 0, bits 13..8 = code length (1..32), bits 7..0 = symbol
 *                  pointer  bit 15 = 1, bits 14..0 = index of the next-level table
 *   multi[1024]  10-bit index; the first up-to-3 codes that lie wholly inside
 *                the 10 bits: bits 31..30 = how many, bits 29..24 = their
 *                total length, bits 7..0, 15..8, 23..16 = their symbols in
 *                order (unused slots 0).  When the first code is longer than
 *                10 bits, bits 31..30 are 0 and the entry is the index of the
 *                level-1 table that lut[0] points at for the index's top 8 bits.
 *   count[4096]  12-bit index; every code that lies wholly inside the 12 bits:
 *                bits 15..12 = their total length, bit j (j < 12) set iff one
 *                of them starts j bits after the index's first bit.  When the
 *                first code is longer than 12 bits, bits 15..12 are 0 and bits
 *                11..0 hold that level-1 table index.
 *
 * The decoder reads lut[0] only through these level-1 indices, so it keeps
 * lut[1 ..] in on-chip memory and not the root.
 *
 * multi, count and lut[0 .. n_luts) are contiguous: the device copy of the
 * tables is the df11_table_bytes(cb) bytes starting at &cb->multi[0].
 */
typedef struct df11_codebook {
    uint8_t code_len[256];
    uint32_t code[256];
    uint32_t n_luts;
    uint32_t max_len;
    uint32_t multi[1u << DF11_MULTI_BITS];
    uint16_t count[1u << DF11_COUNT_BITS];
    uint16_t lut[DF11_MAX_LUTS][256];
} df11_codebook;

/* Bytes of the device table image of cb (multi, count, then n_luts hierarchical tables). */
static inline size_t df11_table_bytes(const df11_codebook *cb) {
    return sizeof(cb->multi) + sizeof(cb->count) + (size_t)cb->n_luts * 256 * sizeof(uint16_t);
}

/* Exact sizes of everything df11_encode writes, for caller allocation. */
typedef struct df11_sizes {
    uint64_t n_weights;      /* N: weights in the unit */
    uint64_t total_bits;     /* exponent code bits, sum over weights of code_len[e] */
    uint64_t n_tiles;        /* ceil(total_bits / (8 * B * T)) */
    uint64_t n_windows;      /* n_tiles * T: bytes of gaps */
    uint64_t stream_bytes;   /* n_tiles * T * B + DF11_STREAM_PAD */
    uint64_t sm_bytes;       /* N (BF16) or ceil(N / 2) (FP8) rounded up to 64, plus 64 bytes */
    uint64_t bop_entries;    /* n_tiles + 1 entries of block_out_pos */
} df11_sizes;

/*
 * A compressed unit in caller-owned HOST memory, filled by df11_encode.
 * The caller sets the pointers (and their capacities, from df11_sizes) and
 * n_tensors; df11_encode fills the arrays and the scalar results.
 */
typedef struct df11_host_stream {
    uint8_t *stream;            /* [stream_bytes] */
    uint8_t *sm;                /* [sm_bytes]; bytes past N are zero */
    uint8_t *gaps;              /* [n_windows] */
    uint32_t *block_out_pos;    /* [n_tiles + 1] */
    uint64_t *tensor_offsets;   /* [n_tensors + 1] element offset of each tensor, then N */
    uint64_t *tensor_tiles;     /* [2 * n_tensors] first tile and one-past-last tile per tensor */
    uint64_t stream_capacity, sm_capacity, gaps_capacity, bop_capacity;
    uint32_t n_tensors;
    /* results */
    uint32_t tile_windows;      /* T */
    uint32_t window_bytes;      /* B */
    uint32_t max_tile_symbols;  /* max over tiles of block_out_pos[t+1] - block_out_pos[t] */
    uint64_t n_weights;
    uint64_t total_bits;
    uint64_t n_tiles;
    uint32_t format;            /* df11_format of the weights */
} df11_host_stream;

/*
 * A compressed unit in DEVICE memory, as df11_decompress_* read it.  Device
 * pointers: stream, sm and tables (16-byte aligned), gaps, block_out_pos;
 * tables holds the df11_table_bytes(cb) bytes starting at &cb->multi[0].  Host
 * pointers: tensor_offsets and tensor_tiles (read synchronously by
 * df11_decompress_tensor only; may be null for df11_decompress_block).
 * Scalars are copied from the df11_host_stream and df11_codebook they came from.
 */
typedef struct df11_device_stream {
    const uint8_t *stream;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *block_out_pos;
    const void *tables;
    const uint64_t *tensor_offsets;
    const uint64_t *tensor_tiles;
    uint64_t n_weights;
    uint64_t total_bits;
    uint64_t n_tiles;
    uint32_t n_luts;
    uint32_t tile_windows;
    uint32_t window_bytes;
    uint32_t max_tile_symbols;
    uint32_t n_tensors;
    uint32_t format;            /* df11_format; 0 (BF16) when zero-initialised */
} df11_device_stream;

/*
 * df11_build_codebook -- host, offline.
 * Entropy coding by frequency ("DFloat11" abstract; offline Huffman coding of
 * exponents, "Three ways to spend the savings").  Counts exponents over all
 * n_tensors arrays (tensors[k] holds numel[k] weights), builds Huffman code
 * lengths (ties: smallest (count, tiebreak), leaf tiebreak = symbol value,
 * k-th merged node = 256 + k; one present symbol is paired with a dummy, the
 * smallest absent value, both of length 1), limits them to 32 bits by
 * package-merge when needed, assigns canonical codes, and fills the
 * hierarchical lookup tables ("compact, hierarchical lookup tables", DFloat11
 * abstract).  Errors: DF11_E_INVALID (null pointers, no weights at all),
 * DF11_E_LUT_BUDGET.  *cb is fully overwritten on success.
 */
int df11_build_codebook(const uint16_t *const *tensors, const uint64_t *numel,
                        uint32_t n_tensors, df11_codebook *cb);

/* The same for any df11_format: tensors[k] points to numel[k] weights of
 * that format (uint16_t for BF16, uint8_t for FP8).  DF11_E_INVALID for an
 * unknown format. */
int df11_build_codebook_fmt(uint32_t format, const void *const *tensors, const uint64_t *numel,
                            uint32_t n_tensors, df11_codebook *cb);

/*
 * df11_encode_size -- host.  Sizes of all arrays df11_encode will write for
 * these tensors under layout (tile_windows T, window_bytes B).  Supported
 * layouts: B = 8 with T = 64, 256 or 512.  Errors: DF11_E_INVALID, DF11_E_SYMBOL.
 */
int df11_encode_size(const df11_codebook *cb, const uint16_t *const *tensors,
                     const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                     uint32_t window_bytes, df11_sizes *out);

/* df11_encode_size for any df11_format (FP8 requires T = 64). */
int df11_encode_size_fmt(uint32_t format, const df11_codebook *cb, const void *const *tensors,
                         const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                         uint32_t window_bytes, df11_sizes *out);

/*
 * df11_encode -- host, offline.  Writes the concatenated exponent code stream,
 * the sm bytes and the auxiliary arrays (gaps, block_out_pos: the "lightweight
 * auxiliary variables" that coordinate thread read and write positions,
 * DFloat11 abstract) into the caller's buffers in *out, plus tensor_offsets
 * and tensor_tiles.  out->n_tensors must equal n_tensors.  Errors:
 * DF11_E_INVALID, DF11_E_SYMBOL, DF11_E_CAPACITY (a capacity field below the
 * df11_encode_size figure), DF11_E_INVALID when N >= 2^32.
 */
int df11_encode(const df11_codebook *cb, const uint16_t *const *tensors,
                const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                uint32_t window_bytes, df11_host_stream *out);

/* The codebook of df11_build_codebook from an exponent histogram counts[256]
 * (e.g. from df11_histogram_device).  Errors: DF11_E_INVALID (null, all zero),
 * DF11_E_LUT_BUDGET. */
int df11_build_codebook_from_counts(const uint64_t *counts, df11_codebook *cb);

/* df11_encode_size from a histogram of n_weights weights (the counts must sum
 * to n_weights).  Errors: DF11_E_INVALID, DF11_E_SYMBOL. */
int df11_encode_size_from_counts(uint32_t format, const df11_codebook *cb, const uint64_t *counts,
                                 uint64_t n_weights, uint32_t tile_windows, uint32_t window_bytes,
                                 df11_sizes *out);

/*
 * df11_tensor_ranges_from_counts -- host.  The tensor_offsets and
 * tensor_tiles arrays that df11_encode writes (see df11_host_stream), from
 * per-tensor exponent histograms instead of the weights, for a unit encoded
 * elsewhere (df11_encode_device): counts holds n_tensors rows of 256 uint64,
 * row k the histogram of tensor k (its sum is the tensor's weight count);
 * last_weights[k] is the bit pattern of tensor k's last weight (ignored for
 * an empty tensor), whose symbol's code is the tensor's last.  Writes
 * tensor_offsets[0 .. n_tensors] and tensor_tiles[0 .. 2 n_tensors).
 * Errors: DF11_E_INVALID (null pointers, layout, a last weight whose symbol
 * the row does not count, N >= 2^32), DF11_E_SYMBOL (a counted symbol without
 * a code).
 */
int df11_tensor_ranges_from_counts(uint32_t format, const df11_codebook *cb,
                                   const uint64_t *counts, const uint32_t *last_weights,
                                   uint32_t n_tensors, uint32_t tile_windows,
                                   uint32_t window_bytes, uint64_t *tensor_offsets,
                                   uint64_t *tensor_tiles);

/* df11_encode for any df11_format (FP8 requires T = 64); out->format is set. */
int df11_encode_fmt(uint32_t format, const df11_codebook *cb, const void *const *tensors,
                    const uint64_t *numel, uint32_t n_tensors, uint32_t tile_windows,
                    uint32_t window_bytes, df11_host_stream *out);

/*
 * df11_decompress_block -- device.  Transformer-block-level decompression
 * (DFloat11 abstract): the whole unit in exactly one kernel launch, on stream
 * st, into out[0 .. n_weights) (device memory, 16-byte aligned, caller-owned,
 * uint16_t elements for BF16 and uint8_t for FP8 units; tensor k is
 * out[tensor_offsets[k] .. tensor_offsets[k+1])).  Every output equals the
 * original bit pattern.  Asynchronous: returns after the
 * launch.  Synchronous errors: DF11_E_INVALID (null or misaligned pointers,
 * unsupported layout, sizes inconsistent with each other), DF11_E_HIP.  The
 * kernel checks each tile's decoded symbol count against block_out_pos and,
 * on a mismatch, writes DF11_E_CORRUPT to *d_status (device int32, may be
 * null) and leaves that tile's outputs unwritten.  N == 0 launches nothing.
 */
int df11_decompress_block(const df11_device_stream *s, void *out, int32_t *d_status,
                          df11_hip_stream st);

/*
 * df11_decompress_tensor -- device.  Decompresses only tensor k of the unit
 * into out[0 .. numel_k) (device, 16-byte aligned) with one launch over the
 * tiles that hold its codes; same kernel, checks and errors as
 * df11_decompress_block.  The tensor's element offset in the unit must be a
 * multiple of 8 for BF16 and of 16 for FP8 units (DF11_E_INVALID otherwise;
 * decompress the block instead).
 */
int df11_decompress_tensor(const df11_device_stream *s, uint32_t k, void *out,
                           int32_t *d_status, df11_hip_stream st);

/*
 * df11_window_counts -- device, diagnostic.  The first phase of the
 * two-phase decode (DFloat11 abstract: each thread counts the codes of its
 * own window before the outputs are placed) run on its own, one window per
 * thread, with the same device code the decompress kernels use:
 * counts[j] = the number of codes whose first bit lies in stream bits
 * [64 j, 64 j + 64), for every window j < n_tiles * tile_windows.  counts:
 * device, caller-owned, 4-byte aligned, n_tiles * tile_windows uint32
 * entries.  The prefix sums at tile boundaries are block_out_pos; a window
 * whose bits are no valid code gets 2^20 added.  One launch on st,
 * asynchronous.  DF11_E_INVALID for a bad descriptor or a null counts.
 */
int df11_window_counts(const df11_device_stream *s, uint32_t *counts, df11_hip_stream st);

/* Static description of a status code. */
const char *df11_status_string(int status);

/*
 * GPU-side encoder -- for weights already in device memory (a fine-tuned or
 * freshly quantized model): the histogram runs on the device, the codebook is
 * built on the host from it (df11_build_codebook_from_counts), and the
 * encoding runs on the device and writes exactly the bytes df11_encode would
 * (frequency-chosen codes for the exponents, DFloat11 abstract).  One unit is
 * one contiguous device array of n weights (concatenate a block's tensors
 * first); per-tensor offsets and tile ranges follow from per-tensor
 * histograms as in df11_encode.
 */

/* counts[s] = number of weights with exponent symbol s, into d_counts
 * (device, 256 uint64, 16-byte aligned; cleared by the call).  w: device,
 * 16-byte aligned.  Asynchronous on stream st. */
int df11_histogram_device(uint32_t format, const void *w, uint64_t n, uint64_t *d_counts,
                          df11_hip_stream st);

/* Device scratch df11_encode_device needs for n weights (per-4096-weight bit
 * totals, start bits, and the two boundary-word shares of each 4096-weight
 * group). */
uint64_t df11_encode_device_scratch_bytes(uint64_t n_weights);

/* Device buffers of df11_encode_device (all device memory, 16-byte aligned;
 * scratch 256-byte aligned).  Sizes: those of df11_sizes for the stream, sm,
 * gaps and block_out_pos arrays; d_max_tile_symbols: 16 bytes, of which the
 * first uint32 receives max_tile_symbols. */
typedef struct df11_device_encode {
    uint8_t *stream;
    uint8_t *sm;
    uint8_t *gaps;
    uint32_t *block_out_pos;
    uint32_t *d_max_tile_symbols;
    void *scratch;
    uint64_t scratch_bytes;
} df11_device_encode;

/* Encodes the n weights at w (device) with codebook cb under layout (T, B)
 * into out; sz must be df11_encode_size_from_counts's result for the same
 * weights.  Asynchronous on stream st (the buffers are complete when the
 * stream reaches that point).  Errors: DF11_E_INVALID (null, misaligned or
 * inconsistent arguments, n == 0), DF11_E_HIP. */
int df11_encode_device(uint32_t format, const df11_codebook *cb, const void *w, uint64_t n,
                       uint32_t tile_windows, uint32_t window_bytes, const df11_sizes *sz,
                       const df11_device_encode *out, df11_hip_stream st);

/*
 * Overlapped block pipeline -- device orchestration.  Decompression is done
 * per transformer block so that the next block's weights can be prepared
 * while the model consumes the current one ("transformer-block-level
 * decompression", DFloat11 abstract).  A df11_pipeline owns no device memory:
 * it keeps, for each of n_slots caller-owned output buffers, one event that
 * marks "decompressed into this slot" and one that marks "the consumer has
 * finished reading it", and orders a decode stream against consumer streams
 * with them.  Typical use with two slots:
 *
 *   decompress(slot 0, block 0)
 *   for i: decompress(slot (i+1)%2, block i+1)   -- decode stream, waits for the
 *                                                   release of that slot
 *          acquire(slot i%2, compute stream)     -- compute waits for block i
 *          ... consumer kernels on compute reading slot i%2 ...
 *          release(slot i%2, compute stream)
 *
 * All calls only enqueue work or waits and return at once.  A pipeline is
 * used from one host thread at a time; its streams must outlive it.
 */
#define DF11_PIPELINE_MAX_SLOTS 4
typedef struct df11_pipeline df11_pipeline;  /* opaque */

/* Creates a pipeline over n_slots (1..DF11_PIPELINE_MAX_SLOTS) buffers whose
 * decompressions run on decode_stream (2 * n_slots HIP events are created).
 * Errors: DF11_E_INVALID, DF11_E_HIP.  *out is null on error. */
int df11_pipeline_create(df11_hip_stream decode_stream, uint32_t n_slots, df11_pipeline **out);

/* Destroys the events and the object; null is allowed.  Work already enqueued
 * is not waited for. */
int df11_pipeline_destroy(df11_pipeline *p);

/* Enqueues on the decode stream: a wait for the slot's last release (if it
 * was ever released), df11_decompress_block(s, out, d_status), and the slot's
 * ready event.  Same argument errors as df11_decompress_block.  A slot that a
 * consumer has read must be released before it is refilled. */
int df11_pipeline_decompress(df11_pipeline *p, uint32_t slot, const df11_device_stream *s,
                             void *out, int32_t *d_status);

/* How much of the GPU the pipeline's decompressions take: at most
 * workgroups_per_cu resident workgroups per compute unit (a persistent grid
 * of that many workgroups per compute unit of the device, whose waves loop
 * over the tiles), leaving the rest of every compute unit
 * to the consumer's kernels, which then run beside the decode instead of
 * waiting for its workgroups to drain.  0 (the default) launches the full
 * grid of df11_decompress_block.  Applies to later df11_pipeline_decompress
 * calls.  DF11_E_INVALID for a null pipeline or a value above 64. */
int df11_pipeline_set_decode_share(df11_pipeline *p, uint32_t workgroups_per_cu);

/* Makes the consumer stream wait until the slot's latest decompression is
 * done.  DF11_E_INVALID if the slot was never filled. */
int df11_pipeline_acquire(df11_pipeline *p, uint32_t slot, df11_hip_stream consumer);

/* Records, on the consumer stream, that the work enqueued there so far is all
 * that reads the slot; the next decompression into it waits for that work. */
int df11_pipeline_release(df11_pipeline *p, uint32_t slot, df11_hip_stream consumer);

/*
 * df11_gemv_bf16 -- device, a consumer of decompressed blocks: for each of
 * n_tensors (<= DF11_GEMV_MAX_TENSORS) row-major BF16 matrices
 * W_k = w[w_offset_k ..] of rows_k x cols_k, y[y_offset_k + r] = sum over c of
 * W_k[r][c] * x[x_offset_k + c], in float32 (products and sums are fused
 * multiply-adds in a fixed order: 8-column groups per lane in column order,
 * then a butterfly over the 64 lanes, so results are deterministic).  One
 * launch on stream st.  Requirements: w and x 16-byte aligned, cols_k and
 * w_offset_k multiples of 8, x_offset_k a multiple of 4 (DF11_E_INVALID).
 * Offsets are in elements.
 */
#define DF11_GEMV_MAX_TENSORS 16
typedef struct df11_gemv_tensor {
    uint64_t w_offset;
    uint64_t x_offset;
    uint64_t y_offset;
    uint32_t rows;
    uint32_t cols;
} df11_gemv_tensor;

int df11_gemv_bf16(const uint16_t *w, const df11_gemv_tensor *tensors, uint32_t n_tensors,
                   const float *x, float *y, df11_hip_stream st);

/*
 * df11_decompress_gemv -- device, decode fused into its consumer: the same
 * products as df11_gemv_bf16 (y[y_offset_k + r] = sum over c of W_k[r][c] *
 * x[x_offset_k + c], float32), computed straight from the compressed unit s
 * without writing its BF16 weights, so HBM carries only the compressed bytes.
 * A step toward decoding into the consumer's tiles (DFloat11 decompresses
 * "online" right before use, abstract).  Requirements (DF11_E_INVALID
 * otherwise): a BF16 unit with 64-window tiles; the tensors tile the unit in
 * order (w_offset_k = sum of the previous rows * cols), cols_k multiples of 8,
 * x 16-byte aligned with x_offset_k multiples of 4; no tile may touch more
 * than 4 rows, i.e. (max_tile_symbols - 1) / min_k cols_k + 2 <= 4; x, y and
 * scratch must not overlap.  Each
 * output is a sum formed in a fixed order: per weight chunk of 8 a chain of
 * fused multiply-adds, per lane the chunks in order, a butterfly over the
 * wave, then per row the tiles in order (deterministic; it differs from
 * df11_gemv_bf16's order).  scratch: device, 16-byte aligned, at least
 * df11_decompress_gemv_scratch_bytes(s) bytes.  Two launches on st; corrupt
 * tiles are reported in *d_status as by df11_decompress_block.
 */
uint64_t df11_decompress_gemv_scratch_bytes(const df11_device_stream *s);
int df11_decompress_gemv(const df11_device_stream *s, const df11_gemv_tensor *tensors,
                         uint32_t n_tensors, const float *x, float *y, void *scratch,
                         uint64_t scratch_bytes, int32_t *d_status, df11_hip_stream st);

/*
 * df11_decompress_gemv_noalloc -- device.  For callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): df11_decompress_gemv with the library's own
 * workspace instead of a caller's.  That workspace is one static device array
 * per GPU of DF11_GEMV_NOALLOC_MAX_TILES * 20 + 256 bytes (15 MiB), held from
 * the library's load until the process ends; the call itself allocates
 * nothing.  Same arguments (minus the workspace), products, summation order
 * and errors as df11_decompress_gemv, plus DF11_E_CAPACITY, returned before
 * anything is launched, for a unit of more than DF11_GEMV_NOALLOC_MAX_TILES
 * tiles (a Llama-3-70B-shaped block has about 558,000).  Every call on a GPU
 * shares that GPU's workspace: calls that may overlap on one GPU (different
 * streams, or different host threads) race and must be ordered by the
 * caller.  Nothing in the workspace needs clearing between calls (every tile
 * of a valid unit writes its entries before the second launch reads them).
 * The first call on a device looks the workspace's address up on that
 * device (it must be the current device) and keeps it.
 */
#define DF11_GEMV_NOALLOC_MAX_TILES 786432u
int df11_decompress_gemv_noalloc(const df11_device_stream *s, const df11_gemv_tensor *tensors,
                                 uint32_t n_tensors, const float *x, float *y,
                                 int32_t *d_status, df11_hip_stream st);

/*
 * df11_gemm_order -- host, the weight order that df11_decompress_gemm reads:
 * matrix w (rows x cols, row-major BF16; rows a multiple of 16, cols of 32)
 * as 16-row blocks m in order, each as its 32-column sub-blocks kb in order,
 * each as four 8-column quarters q, each as 16 rows i of 8 weights:
 *   out[(((m * cols/32 + kb) * 4 + q) * 16 + i) * 8 + e] = w[(16 m + i) * cols + 32 kb + 8 q + e].
 * A sub-block is then the A operand of one 16x16x32 matrix-core product in
 * its lane order (lane 16 q + i holds row i, columns 8 q .. 8 q + 7), so
 * the lanes of a wave read it contiguously.  A permutation applied before
 * df11_build_codebook / df11_encode.  out must not overlap w.  Returns
 * DF11_E_INVALID for other shapes or pointers.
 */
int df11_gemm_order(const uint16_t *w, uint32_t rows, uint32_t cols, uint16_t *out);

/*
 * df11_decompress_gemm -- device, decode fused into a matrix product on the
 * matrix cores (the GEMM half of decoding straight into the consumer's tiles;
 * DFloat11 decompresses right before use, abstract): for n_tokens = 16,
 * 32, 48 or 64 tokens and each matrix k of the unit,
 *   y[y_offset_k + t * rows_k + r] = sum over c of W_k[r][c] * x[x_offset_k + t * cols_k + c]
 * (x: BF16 activations, token-major; y: float32, token-major), where the
 * unit s holds every W_k in df11_gemm_order order (BF16, 64-window tiles)
 * and tensors[k].w_offset is its offset in the unit (the matrices follow one
 * another).  rows_k multiples of 16, cols_k of 32; x, y and scratch 16-byte
 * aligned and not overlapping, x_offset_k multiples of 8, y_offset_k of 4.  scratch: at least
 * df11_decompress_gemm_scratch_bytes(tensors, n_tensors, n_tokens) bytes
 * (each matrix's activations reordered for the matrix cores, 2 * n_tokens *
 * cols_k bytes, then float32 partial sums of the split matrices); no
 * initialisation needed.  Products are exact; sums are float32 in the
 * matrix cores, per 16-row block and K segment each of four waves adding its
 * 32-column sub-blocks in order, then the four waves in order, then the
 * segments in order (deterministic).  A matrix with cols_k above
 * R = max(4096, min_j cols_j) has its row blocks split into at
 * most ceil(cols_k / R) K segments of whole sub-blocks, so that every
 * workgroup decodes about as many weights.  Weights
 * outside a decoded tile enter as zeros, so x must be finite.  Two launches
 * on st (three when a matrix is split), no allocation; calls sharing a
 * scratch buffer must not overlap.  Corrupt tiles are reported in *d_status as by
 * df11_decompress_block (the rows they hold get wrong values).
 * DF11_E_INVALID for other shapes, formats or layouts.
 */
uint64_t df11_decompress_gemm_scratch_bytes(const df11_gemv_tensor *tensors, uint32_t n_tensors,
                                            uint32_t n_tokens);
int df11_decompress_gemm(const df11_device_stream *s, const df11_gemv_tensor *tensors,
                         uint32_t n_tensors, uint32_t n_tokens, const uint16_t *x, float *y,
                         void *scratch, uint64_t scratch_bytes, int32_t *d_status,
                         df11_hip_stream st);

#ifdef __cplusplus
}
#endif

#endif /* DF11_H */
