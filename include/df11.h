/*
 * df11.h -- C ABI of libdf11.so, an MI355X (gfx950) implementation of the
 * DFloat11 (Dynamic-length Float) codec for BF16 weights.
 *
 * What the codec computes (sources cited by page title and section):
 *   [P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案"
 *        (jsqmd.com) 2.1: a BF16 word is 1 sign bit, 8 exponent bits and
 *        7 mantissa bits.  2.2 item 1: the exponents' frequencies are counted
 *        and a Huffman code gives frequent exponents short codes.  2.2 item 2:
 *        sign and mantissa are kept unchanged next to the variable-length
 *        exponent code, packed into aligned blocks (about 11 bits per weight).
 *        2.2 item 3: the compressed weights stay in GPU memory and a GPU
 *        kernel restores BF16 right before the matmul that uses them.
 *   [P2] "DFloat11：用于高效 GPU 推理的 LLM 和扩散模型无损压缩"
 *        (gittoolsai.com), "工作原理": Huffman-coded BF16 exponents, decoded
 *        on the GPU before each matrix product, output bit-for-bit identical.
 *   [P3] "DFloat11重新定义LLM无损压缩的技术边界" (ocdem.com) 2.2: compact
 *        hierarchical lookup tables, a locate phase and a reconstruct phase,
 *        and a parallel prefix sum for output positions; 4.2: each thread
 *        takes a fixed run of encoded bytes; 5.2: 256-byte aligned data.
 *
 * Conventions
 *   - Every function returns DF11_OK (0) or a negative DF11_E_* status, and
 *     never throws.  df11_last_error() gives the calling thread's detail text
 *     for the most recent failure.
 *   - BF16 tensors are passed as their uint16 bit patterns.
 *   - "host" pointers are CPU memory; "device" pointers are GPU memory of the
 *     current HIP device.  Device work is asynchronous on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream).  The decode,
 *     row-gather and fused-product calls allocate no device memory and keep
 *     no per-call state; only df11_encode_device allocates, the device arrays
 *     it returns (freed with df11_device_encoded_free).
 *
 * Stream format (what df11_encode writes and the kernels read)
 *   exp_words  The exponent codes of all elements in stream order, each code
 *              most significant bit first, laid end to end.  Stream bit j is
 *              bit (31 - j % 32) of 32-bit word j / 32.  Zero bits pad the
 *              stream; when layout.align_elems > 0 zero bits also pad each
 *              block of align_elems elements up to a segment boundary.
 *   sm         One byte per element: sign in bit 7, mantissa in bits 6..0.
 *   segments   The stream is cut into segments of seg_lanes * chunk_bytes
 *              bytes; a segment is decoded by one 64-lane wavefront, each lane
 *              taking one chunk of chunk_bytes bytes.
 *   gaps       One byte per chunk: the distance in bits from the chunk start
 *              to the first code that starts at or after it (0..31), or 0 for
 *              a chunk at or past its segment's last code.
 *   counts     One byte per chunk: the number of codes whose first bit lies
 *              in the chunk (0 for chunks past the segment's last code).  The
 *              decoder's output positions are a prefix sum of these counts.
 *              Optional in a view (n_counts = 0): the decoder then finds each
 *              lane's count itself by walking its chunk (the locate pass).
 *              Encoders always write them; a layout whose chunk could hold
 *              more than 255 codes (chunk bits / shortest code) is refused.
 *   segs       n_segments + 1 records: elem_off = number of codes that start
 *              before the segment (the last record's elem_off = n); nbits =
 *              bits from the segment start to the end of the last code that
 *              starts in it, at most the segment size.
 *   chain      The hierarchical lookup tables: n_tables tables of 256 uint16
 *              entries.  Table 0 is indexed by the next 8 stream bits, each
 *              later table by the 8 bits after its parent's.  Entry bit 15
 *              clear: a code ends here -- exponent in bits 0..7, total code
 *              length in bits 8..13.  Bit 15 set: bits 0..14 name the next
 *              table.
 *   fast       2^fast_bits pairs of uint32 {syms, meta} indexed by the next
 *              fast_bits stream bits: the up to 4 whole codes that fit, first
 *              code in the lowest byte, each byte the exponent rotated right
 *              by one bit; meta = (count << 16) - bits consumed, modulo 2^32;
 *              meta = 0 when the first code is longer than fast_bits.
 *   block_seg  When align_elems > 0: for every block of align_elems elements the
 *              index of the segment its first code starts in, followed by
 *              n_segments (ceil(n / align_elems) + 1 entries); else empty.
 *   Element order is row-major, or, when tile_rows > 0, tile order: the
 *   [rows, cols] matrix is cut into tile_rows x tile_cols tiles taken row
 *   block by row block, row-major inside each tile, or, when tile_kchunk > 0,
 *   in column groups of tile_kchunk columns: group after group, each group
 *   row after row (the order matrix-core operands read).
 */
#ifndef DF11_H
#define DF11_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DF11_OK 0
#define DF11_E_ARG (-1)       /* null/misaligned pointer, size or layout out of range */
#define DF11_E_UNCODED (-2)   /* an input exponent has no code in the codebook */
#define DF11_E_CODE_LEN (-3)  /* max_len outside 1..32, or more than DF11_MAX_TABLES tables */
#define DF11_E_FORMAT (-4)    /* df11_validate found an inconsistent stream or codebook */
#define DF11_E_DEVICE (-5)    /* a HIP call failed; detail in df11_last_error() */
#define DF11_E_ALLOC (-6)     /* an allocation failed */
#define DF11_E_UNSUPPORTED (-7) /* a valid request this build does not handle */

#define DF11_MAX_LEN 32
#define DF11_MAX_TABLES 64
#define DF11_FAST_BITS_MIN 8
#define DF11_FAST_BITS_MAX 12
#define DF11_FAST_BITS_DEFAULT 11
#define DF11_SEG_LANES 64

/* A codebook: code lengths, canonical codes and the lookup tables derived
 * from them.  Plain data; the caller owns the struct. */
typedef struct df11_codebook {
    uint32_t max_len;     /* longest code length (0 when no symbol occurs) */
    uint32_t min_len;     /* shortest code length */
    uint32_t n_symbols;   /* exponents with a code */
    uint32_t n_tables;    /* hierarchical 256-entry tables used in chain[] */
    uint32_t fast_bits;   /* index width of fast[] */
    uint32_t reserved[3];
    uint8_t len[256];     /* code length per exponent, 0 = no code */
    uint32_t code[256];   /* canonical code per exponent, right-aligned */
    uint16_t chain[DF11_MAX_TABLES * 256];
    uint32_t fast[2u << DF11_FAST_BITS_MAX];
} df11_codebook;

/* How the stream is laid out.  Zero-initialise and set what you need:
 * chunk_bytes 0 means 16; seg_lanes 0 means 64. */
typedef struct df11_layout {
    uint32_t chunk_bytes;   /* stream bytes per lane: 16, or 8 (twice the segments, for
                               small tensors that would leave most of the GPU idle) */
    uint32_t seg_lanes;     /* lanes per segment: must be 64 */
    uint64_t align_elems;   /* 0, or begin a new segment every align_elems elements */
    uint64_t rows, cols;    /* matrix shape; cols = 0 means a flat tensor of rows = n */
    uint32_t tile_rows, tile_cols;  /* 0, 0: row-major; else tile order (see above) */
    uint32_t tile_kchunk;           /* 0: row-major inside a tile; else column groups (see above) */
    uint32_t reserved;
} df11_layout;

typedef struct df11_segment {
    uint64_t elem_off;
    uint32_t nbits;
    uint32_t reserved;
} df11_segment;

/* Pointers and sizes of one encoded tensor.  The pointers are all host or all
 * device memory; the caller fills a device view by copying every array of a
 * host view to the GPU and keeping the scalars. */
typedef struct df11_view {
    uint64_t n;             /* elements */
    uint64_t total_bits;    /* end of the last code in the stream */
    uint64_t n_segments;
    uint32_t chunk_bytes, seg_lanes;
    uint64_t rows, cols;
    uint32_t tile_rows, tile_cols;
    uint32_t tile_kchunk;
    int32_t row_win_lo;         /* row window (see below) */
    uint64_t align_elems;
    uint32_t min_len, max_len, n_tables, fast_bits;
    uint32_t max_seg_elems;     /* most codes starting in any one segment */
    uint32_t row_win_span;      /* row window: 0 = none.  For a row-major view with rows and
                                   cols set, both encoders record the window that holds every
                                   segment overlapping any row r: with g(r) = floor(r * cols *
                                   (n_segments / n)), the segment indices in IEEE double
                                   arithmetic (the quotient first), row r's segments lie in
                                   [g(r) + row_win_lo, g(r) + row_win_lo + row_win_span).
                                   df11_decode_rows relies on it as written by the encoder. */
    const uint32_t *exp_words;  uint64_t n_exp_words;  /* n_segments*seg_words + 2 */
    const uint8_t *sm;          uint64_t n_sm;         /* n rounded up to 16 */
    const uint8_t *gaps;        uint64_t n_gaps;       /* n_segments * seg_lanes */
    const df11_segment *segs;   uint64_t n_segs;       /* n_segments + 1 */
    const uint16_t *chain;      uint64_t n_chain;      /* n_tables * 256 */
    const uint32_t *fast;       uint64_t n_fast;       /* 2 << fast_bits */
    const uint64_t *block_seg;  uint64_t n_block_seg;  /* align_elems > 0: first segment of
                                                          every aligned block, then n_segments */
    const uint8_t *counts;      uint64_t n_counts;     /* n_segments * seg_lanes, or 0 */
} df11_view;

typedef struct df11_encoded df11_encoded;   /* opaque, library-owned host arrays */

/* ---------------------------------------------------------------- host side */

/* hist[e] += number of elements of bf16_bits[0..n) whose exponent is e
 * ([P1] 2.2 item 1).  Accumulates, so several tensors can share one codebook.
 * bf16_bits and hist are host pointers; n = 0 is a no-op.  Errors: E_ARG for
 * a null pointer with n > 0. */
int df11_hist_accumulate(const uint16_t *bf16_bits, uint64_t n, uint64_t hist[256]);

/* Build a codebook from an exponent histogram ([P1] 2.2 item 1; [P2]
 * "工作原理"): Huffman code lengths, replaced by the optimal code limited to
 * max_len bits (package-merge) when Huffman is longer; canonical codes in
 * (length, exponent) order; the hierarchical tables ([P3] 2.2) and the
 * fast_bits-wide multi-code table.  max_len in 1..32, fast_bits in 8..12.
 * Errors: E_ARG (null), E_CODE_LEN (max_len out of range or too small for
 * the number of symbols, or more than DF11_MAX_TABLES tables). */
int df11_codebook_build(const uint64_t hist[256], uint32_t max_len, uint32_t fast_bits,
                        df11_codebook *cb);

/* Encode n BF16 words (host) with codebook cb into a new library-owned
 * encoding ([P1] 2.2 item 2; [P3] 4.2): exponent stream, sign+mantissa
 * bytes, per-lane gaps and per-segment records, laid out by `layout` (NULL
 * = defaults).  *out receives the encoding; free it with df11_encoded_free.
 * Every layout it accepts is one the decode calls read.
 * Errors: E_ARG (null pointers, chunk_bytes other than 8 or 16, layout out
 * of range, rows*cols != n, tile shape not dividing the matrix or tile_cols
 * not a multiple of 16), E_UNCODED (an exponent without a code), E_ALLOC. */
int df11_encode(const uint16_t *bf16_bits, uint64_t n, const df11_codebook *cb,
                const df11_layout *layout, df11_encoded **out);

void df11_encoded_free(df11_encoded *enc);

/* Fill *v with host pointers into enc (valid until df11_encoded_free). */
int df11_encoded_view(const df11_encoded *enc, df11_view *v);

/* The layout df11_decode_gemm needs for an [rows, cols] weight: tile order
 * with tiles of df11_gemm_tile_rows() x df11_gemm_tile_cols() elements in
 * 8-column groups, each tile beginning a segment.  Errors: E_ARG when the
 * shape does not divide. */
int df11_gemm_layout(uint64_t rows, uint64_t cols, df11_layout *layout);
uint32_t df11_gemm_tile_rows(void);
uint32_t df11_gemm_tile_cols(void);

/* O(n) CPU check of a host view against its codebook: array sizes, table
 * consistency, gaps and segment records recomputed by walking the stream.
 * Returns DF11_OK or E_FORMAT / E_ARG with the first problem in
 * df11_last_error().  Detection path for corrupt data; the kernels do not
 * check streams. */
int df11_validate(const df11_view *host_view, const df11_codebook *cb);

/* ---------------------------------------------------------- device encoder */

/* A tensor encoded on the GPU: every array in device memory owned by the
 * library (including a copy of the codebook's tables). */
typedef struct df11_device_encoded df11_device_encoded;

/* Exponent histogram of n BF16 words in device memory, added into hist
 * (host) ([P1] 2.2 item 1).  Synchronises `stream`.  Errors: E_ARG (null),
 * E_DEVICE. */
int df11_hist_device(const uint16_t *device_bits, uint64_t n, uint64_t hist[256], void *stream);

/* Encode n BF16 words in device memory on the GPU ([P1] 2.2 items 1-2;
 * [P3] 4.1 on the cost of offline compression): the same stream, sign and
 * mantissa bytes, gaps, segment records and block index, byte for byte, as
 * df11_encode with the same codebook and layout.  The library allocates the
 * device arrays; free them with df11_device_encoded_free.  Synchronises
 * `stream` (twice: the stream length decides the output sizes).  Errors:
 * E_ARG (null, layout), E_UNCODED (an exponent without a code), E_ALLOC,
 * E_DEVICE. */
int df11_encode_device(const uint16_t *device_bits, uint64_t n, const df11_codebook *cb,
                       const df11_layout *layout, void *stream, df11_device_encoded **out);
void df11_device_encoded_free(df11_device_encoded *enc);

/* Fill *v with the device pointers of enc (valid until
 * df11_device_encoded_free): a device view for df11_decode and friends. */
int df11_device_encoded_view(const df11_device_encoded *enc, df11_view *v);

/* Copy a device encoding into a new host encoding (free with
 * df11_encoded_free), e.g. to store it or to check it with df11_validate.
 * Errors: E_ARG, E_ALLOC, E_DEVICE. */
int df11_device_encoded_to_host(const df11_device_encoded *enc, df11_encoded **out);

/* -------------------------------------------------------------- device side */

/* Decode a device view into out[0..n) BF16 bits in row-major order
 * ([P1] 2.2 item 3; [P3] 2.2 locate/reconstruct with a prefix sum).
 * out: device, 16-byte aligned, n elements.  Bit-exact: every input pattern,
 * including zeros, subnormals, Inf and NaN payloads, comes back unchanged.
 * Writes stay inside out[0..n) even for a corrupt stream (the exponent
 * words, gaps or counts; then the values are unspecified): every write
 * address comes from the segment records, which are checked against n.
 * The view's max_seg_elems (set by the encoders) sizes the staging: a
 * hand-built view that understates it leaves the larger segments' outputs
 * unwritten.  n = 0 is a no-op.  Errors: E_ARG (null, misaligned, view
 * inconsistent, max_seg_elems 0 or above segment bits / shortest code),
 * E_UNSUPPORTED (tables too large for the kernel), E_DEVICE. */
int df11_decode(const df11_view *device_view, uint16_t *out, void *stream);

/* Decode several device views in one launch: view i into outs[i] (device,
 * 16-byte aligned, views[i].n elements), for example the seven matrices of a
 * decoder layer.  views is a host array of `count` device views that share
 * their device tables (the same chain and fast pointers, i.e. one codebook
 * uploaded once).  Same guarantees and errors as df11_decode, plus E_ARG when
 * the views do not share their tables.  More than 16 views are decoded in
 * launches of 16. */
int df11_decode_batch(const df11_view *device_views, uint16_t *const *outs, uint32_t count,
                      void *stream);

/* Explicit launch choices of a decode, for measurements and tests.  A zeroed
 * struct, or NULL, is the library's own choice. */
#define DF11_STORES_AUTO 0       /* streaming when the launch writes more than the 256 MB last-level cache */
#define DF11_STORES_CACHED 1     /* normal loads and stores: the output stays cache-resident for its consumer */
#define DF11_STORES_STREAMING 2  /* nontemporal BF16 stores */
typedef struct df11_decode_tuning {
    uint32_t waves;        /* waves per workgroup: 0 = from occupancy and size, else 4, 6, ..., 16 */
    uint32_t stores;       /* DF11_STORES_* */
    uint32_t groups;       /* workgroups per launch: 0 = as many as are resident at once (each wave
                              then walks several segments), else that many, at most 2^31 - 1 */
    uint32_t reserved[5];  /* zero */
} df11_decode_tuning;

/* df11_decode_batch with explicit launch choices ([P3] 5.2: occupancy is
 * the tuning lever).  The output is the same for every choice.  Errors: as
 * df11_decode_batch, and E_ARG for a choice out of range or a wave count
 * whose staging and tables do not fit in LDS. */
int df11_decode_batch_tuned(const df11_view *device_views, uint16_t *const *outs, uint32_t count,
                            const df11_decode_tuning *tuning, void *stream);

/* Row gather: decode rows rows[0..n_rows) of a row-major [rows, cols] view
 * into out[i][0..cols) (device, 16-byte aligned, n_rows x cols BF16), for
 * an embedding lookup that restores only the rows a batch uses ([P1] 2.2
 * item 3: weights are restored right before use).  rows: device int64 ids,
 * 8-byte aligned.  For a few rows whose view records a row window of at
 * most 16 segments (row_win_span), each row gets a workgroup in which every
 * segment of the window has its own wave, so no search precedes the segment
 * loads, and the row's sign+mantissa bytes are copied into LDS beside them;
 * otherwise the segments that
 * overlap each requested row are found from an interpolated guess, checked
 * against the 64 segment records around it, else by a 64-way search (up to
 * eight waves per row, one segment each).  Segments are decoded whole
 * (8-byte chunks halve the segments and with them the latency of a lookup);
 * only the row's elements are written.  An id outside
 * [0, rows) leaves its output row unwritten.  Bit-exact like df11_decode.  Errors: E_ARG (null, misaligned,
 * tile-ordered view, cols not a multiple of 8), E_UNSUPPORTED, E_DEVICE. */
int df11_decode_rows(const df11_view *device_view, const int64_t *rows, uint64_t n_rows, uint16_t *out,
                     void *stream);

/* Fused decode + matrix product ([P1] 2.2 item 3: decoded weights feed the
 * matmul and are discarded): y[b][j] = sum_k x[b][k] * W[j][k] for W the
 * [rows = N, cols = K] weight of `w` (encoded with df11_gemm_layout), x a
 * device [B, K] BF16 row-major matrix, y a device [B, N] float32 matrix.
 * Products of BF16 values are exact in float32 and accumulate in float32.
 * w_debug: NULL, or a device [N, K] buffer that also receives the decoded
 * BF16 weights.  B in 1..256.  x, y and w_debug 16-byte aligned.  y is
 * overwritten.  When the weight has too few 32-row blocks to fill the
 * device, a row block's work is split across workgroups (along K, or into
 * runs of its segments) and the partial sums are added into y (cleared
 * first, on the same stream) with float atomics, so the order of those few
 * additions, and with it the last bits of y, can differ from run to run.
 * The kernel is chosen by B: up to 64 rows (128 with the workspace of
 * df11_decode_gemm_ex) one whose decoder waves hand tiles of exponents to
 * matrix-core waves through a ring in LDS, above that (with the workspace)
 * one whose ring holds whole BF16 tiles, else one that merges each decoded
 * tile once into a BF16 tile in LDS shared by all batch tiles (two row
 * blocks per workgroup above 112 rows); w_debug calls take a
 * tile-synchronous kernel up to 32 rows and the shared-tile one above.  A
 * kernel that forms the products on the vector ALU (one or two rows) and a
 * segment-parallel one (up to 64 rows) are explicit choices
 * (df11_decode_gemm_ex makes every choice explicit).
 * Non-finite x: a row of x holding Inf or NaN gives a non-finite row of y;
 * where a plain product would give +-Inf, the segment-parallel and vector
 * kernels may give NaN instead (they multiply the weights of a
 * neighbouring segment, masked to +0, by the same x).  Rows of x without
 * them are unaffected.
 * Errors: E_ARG (null, misaligned, layout not from df11_gemm_layout, B out
 * of range), E_UNSUPPORTED, E_DEVICE. */
int df11_decode_gemm(const df11_view *device_view, const uint16_t *x, uint32_t B,
                     float *y, uint16_t *w_debug, void *stream);

/* Output types of df11_decode_gemm_out. */
#define DF11_Y_F32 0
#define DF11_Y_BF16 1

/* df11_decode_gemm with the type of y chosen by y_dtype: DF11_Y_F32 is
 * df11_decode_gemm itself; DF11_Y_BF16 makes y a device [B, N] BF16 matrix,
 * each element the float32 sum rounded once to the nearest BF16 (ties to
 * even; NaN stays NaN).  A BF16 y is written by exactly one workgroup per
 * element (the K range is not split), so it is the same on every run.
 * Errors: as df11_decode_gemm, and E_ARG for an unknown y_dtype. */
int df11_decode_gemm_out(const df11_view *device_view, const uint16_t *x, uint32_t B,
                         void *y, int y_dtype, uint16_t *w_debug, void *stream);

/* Explicit kernel choices of a fused product, for measurements and tests.
 * A zeroed struct, or NULL, is the library's own choice. */
#define DF11_GEMM_AUTO 0
#define DF11_GEMM_SEGMENT 1   /* segment-parallel: up to 64 rows of x, no w_debug */
#define DF11_GEMM_WIDE 2      /* one BF16 tile in LDS shared by the batch tiles: 33 rows of x or more */
#define DF11_GEMM_TILED 3     /* tile-synchronous, any rows of x */
#define DF11_GEMM_VECTOR 4    /* dot products on the vector ALU: one or two rows of x, no w_debug */
#define DF11_GEMM_PIPE 5      /* decoder and matrix-core waves on a ring of BF16 tiles in LDS: any rows of x */
#define DF11_GEMM_RING 6      /* as DF11_GEMM_PIPE with exponent-only planes, two workgroups per CU: up to 128 rows of x
                                 (two matrix-core waves per batch tile, k_slices, up to 64) */
typedef struct df11_gemm_tuning {
    uint32_t kernel;       /* DF11_GEMM_* */
    uint32_t row_blocks;   /* wide kernel: 0 = by B, else 1 or 2 row blocks per workgroup */
    uint32_t parts;        /* segment-parallel and vector kernels: 0 = enough runs of a row block's
                              segments to fill the device, else that many (float32 y) */
    uint32_t split;        /* wide, tile-synchronous, pipelined and exponent-ring kernels (named in
                              `kernel`): 0 = by occupancy, else that many K ranges per row block
                              (float32 y) */
    uint32_t one_writer;   /* nonzero: every element of y is summed by one workgroup in a fixed
                              order (no K ranges, no segment runs: parts and split 1), so a
                              float32 y is the same on every run; slower for weights with too few
                              row blocks to fill the device */
    uint32_t tiles_per_wave; /* pipelined kernel: 0 = by B, else 1 or 2 batch tiles of 32 rows of x
                              per matrix-core wave */
    uint32_t k_slices;     /* exponent-ring kernel: 0 = by B, else 1 or 2 matrix-core waves per batch
                              tile of x, each taking that share of a tile's k-steps (2: up to 64 rows) */
    uint32_t reserved[1];  /* zero */
} df11_gemm_tuning;

/* Bytes of the workspace df11_decode_gemm_ex can use for B rows of x with
 * this weight: x repacked in the matrix cores' operand order (16 bytes per
 * lane and k-step, one contiguous kilobyte per wavefront load, rows past B
 * zero): 32 T rows of x, (K / 16) * T * 1024 bytes, for T = 2, 4 or 8
 * batch tiles of 32 rows (B up to 64, 128, 256).  0 when B <= 32, where x
 * is read in place, and for a view not in the fused layout. */
uint64_t df11_decode_gemm_workspace_bytes(const df11_view *device_view, uint32_t B);

/* df11_decode_gemm_out with explicit kernel choices and a workspace
 * ([P1] 2.2 item 3: decoded weights feed the matmul; [P3] 5.2: the kernel
 * shape is tuned to the hardware).  tuning: NULL or zeroed = the library's
 * choice.  workspace: NULL, or device memory of workspace_bytes >=
 * df11_decode_gemm_workspace_bytes(w, B), 256-byte aligned, owned by the
 * caller and not used by any other work on the GPU until this call's work on
 * `stream` has finished: above 32 rows of x a packing kernel first writes x
 * into it in operand order (overwriting all of the bytes it needs, so its
 * contents need no clearing), and the product reads x from there (up_proj at
 * 64 / 128 / 256 rows: 63 / 103 / 97 us with x read in place, 47 / 63 / 85
 * us with x packed, the packing included).
 * y agrees with every choice within the float32 summation order.  Errors:
 * as df11_decode_gemm_out, E_ARG for a choice that does not apply (w_debug
 * or more than 64 rows of x on the segment-parallel kernel, w_debug or more
 * than 2 rows on the vector one, 32 rows or fewer on the wide one, split
 * without a kernel that takes it, parts or split above 1 with a BF16 y or
 * with one_writer) or a workspace too
 * small or misaligned, E_UNSUPPORTED when the chosen kernel's LDS does not
 * fit this weight. */
int df11_decode_gemm_ex(const df11_view *device_view, const uint16_t *x, uint32_t B, void *y, int y_dtype,
                        uint16_t *w_debug, const df11_gemm_tuning *tuning, void *workspace,
                        uint64_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * df11_decode_gemm_ex with the packed x kept in the library's own scratch,
 * a 16 MiB array in device memory that every device the library runs on
 * holds until the process ends; no allocation happens in the call.  The
 * scratch covers df11_decode_gemm_workspace_bytes(w, B) <= 16 MiB, that is
 * K * T <= 262144 (T = 2, 4, 8 batch tiles for B up to 64, 128, 256; K up to
 * 32768 at 256 rows of x).  All such calls on one GPU share its scratch:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it; calls ordered on one stream do not (each packs x afresh, nothing
 * has to start at zero).  Errors: as df11_decode_gemm_ex, and E_UNSUPPORTED
 * when the packed x would not fit the scratch. */
int df11_decode_gemm_noalloc(const df11_view *device_view, const uint16_t *x, uint32_t B, void *y,
                             int y_dtype, uint16_t *w_debug, const df11_gemm_tuning *tuning, void *stream);

/* ---------------------------------------------------------------- utilities */
const char *df11_status_string(int status);
const char *df11_last_error(void);
const char *df11_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DF11_H */
