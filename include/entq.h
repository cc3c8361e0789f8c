/*
 * entq.h -- C ABI of the MI355X entropy-coded weight decoder (libentq.so).
 *
 * What is decoded. Weights are stored as 8-bit codes of a full-range base
 * format (Int8 or Float8 e4m3) that have been flattened into a symbol stream
 * and compressed without loss by an ANS entropy coder, next to per-channel
 * (per-row) scales and metadata; the decoder runs on the GPU and fills a
 * buffer just before a transformer block's forward pass uses it [EntQuant,
 * "Float8@2bits: Entropy Coding Enables Data-Free Model Compression",
 * technical summary §2 "Codificación de Pesos" and "Decodificación en Tiempo
 * de Inferencia"]. The same decoder also serves BF16 weights whose 8-bit
 * exponent is the coded symbol while the sign+mantissa byte is stored raw,
 * rebuilt bit for bit [DFloat11 write-up, "Formato DFloat11"]. All matrices
 * of one block are decoded in one batch [DFloat11 write-up, "Descompresión
 * por bloque transformer"].
 *
 * Coder (range ANS, Duda 2013, with interleaved states, Giesen 2014; the
 * pages give no coder parameters, these are the library's format):
 *   - probability scale M = 2^12: a tensor's table freq[256] sums to 4096;
 *   - 32-bit state in [2^16, 2^32), 16-bit renormalisation words;
 *   - a tensor is cut into chunks of chunk_symbols symbols (the last one may
 *     be shorter); symbol i of a chunk belongs to lane i mod 64 of 64
 *     interleaved states; the lanes share one word stream, read front to back
 *     and, within a step of 64 symbols, in ascending lane order.
 *   Decoding symbol i (lane j): slot = x_j & 4095, s = owner of the slot
 *   (cum[s] <= slot < cum[s] + f[s]), x_j = f[s] * (x_j >> 12) + slot -
 *   cum[s]; then if x_j < 2^16, x_j = x_j << 16 | next word.
 *
 * Compressed layout (the "blob"), one region per chunk:
 *   uint32 states[64]   initial decoder state of lane j at index j
 *   uint16 words[n]     the chunk's word stream, in decoding order
 *   zero padding to a multiple of 16 bytes
 * all little-endian; every region starts at a multiple of 16 bytes.
 *
 * Outputs:
 *   ENTQ_OUT_CODES  uint8  out[i] = the decoded code byte;
 *   ENTQ_OUT_BF16   uint16 out[i] = RNE_bf16( fl32( value(code) * scale[row] ) )
 *                   where value is the two's-complement integer (INT8) or
 *                   the OCP e4m3 ("E4M3FN") value (E4M3; a NaN code
 *                   S.1111.111 has the NaN S << 31 | 0x7FF00000 as value:
 *                   sign kept, mantissa bits at the top of the payload, as
 *                   IEEE 754-2008 §6.2.3 widens a NaN), the product is one
 *                   IEEE single multiply rounded to nearest even (a NaN
 *                   operand comes out quieted with its payload, the code's
 *                   before the scale's; 0 * inf gives 0xFFC00000), and
 *                   RNE_bf16 rounds to nearest even (a NaN stays a quiet NaN
 *                   with its sign and top payload bits);
 *   entq_decode_bf16_split: uint16 out[i] = (sm & 0x80) << 8 | exp << 7 |
 *                   (sm & 0x7F), exp the decoded symbol, sm the raw byte.
 *
 * Ownership: every device buffer is allocated by the caller; the library
 * never allocates device memory (its only device memory of its own is the
 * fixed static array of entq_decode_gemm_static, part of its code object,
 * one per GPU it runs on). A plan is host memory owned by the library
 * until entq_plan_destroy; it points into the caller's device workspace,
 * which must outlive the plan and every decode enqueued with it.
 * Asynchrony: device work is enqueued on the given HIP stream (NULL = the
 * default stream); no call synchronises. Errors: argument, table, index and
 * alignment problems and launch failures return a negative entq_status;
 * corrupt compressed data is reported per chunk through chunk_status (after
 * the stream is synchronised). No exception crosses this interface.
 */
#ifndef ENTQ_H
#define ENTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENTQ_PROB_BITS 12
#define ENTQ_PROB_SCALE 4096u
#define ENTQ_LANES 64u
#define ENTQ_STATE_LOW 65536u
#define ENTQ_REGION_ALIGN 16u
#define ENTQ_TABLE_BYTES 512u   /* a per-chunk table: u16 freq[256] */

typedef enum {
    ENTQ_OK = 0,
    ENTQ_EINVAL = -1,       /* a NULL pointer, a bad size or kind           */
    ENTQ_EBADTABLE = -2,    /* a frequency table does not sum to 4096       */
    ENTQ_EBADINDEX = -3,    /* chunk index does not tile the tensors        */
    ENTQ_EALIGN = -4,       /* a region or buffer is misaligned             */
    ENTQ_EWORKSPACE = -5,   /* workspace too small                          */
    ENTQ_EHIP = -6,         /* a HIP call or kernel launch failed           */
    ENTQ_ENOMEM = -7,       /* host allocation failed                       */
    ENTQ_ESYMBOL = -8,      /* encoder: a symbol has frequency 0            */
    ENTQ_ETOOLARGE = -9     /* beyond the library's static scratch          */
} entq_status;

typedef enum { ENTQ_SYM_INT8 = 0, ENTQ_SYM_E4M3 = 1, ENTQ_SYM_BF16EXP = 2 } entq_symkind;
typedef enum { ENTQ_OUT_CODES = 0, ENTQ_OUT_BF16 = 1 } entq_outkind;

/* Per-chunk decode status written to chunk_status[k] (k = position in the
 * chunk index given to entq_plan). */
#define ENTQ_CHUNK_OK 0
#define ENTQ_CHUNK_BAD_STATE 1  /* a lane did not end at 2^16              */
#define ENTQ_CHUNK_BAD_WORDS 2  /* words ran out or were not all consumed  */
#define ENTQ_CHUNK_BAD_TABLE 3  /* (per-chunk tables) the chunk's table does not sum to 4096 */

/* A tensor whose symbols are in the library's tile order (entq_tile_order)
 * carries this flag in its kind: ENTQ_SYM_INT8 | ENTQ_LAYOUT_TILES, or E4M3,
 * or BF16EXP. The plan then requires rows a multiple of 16, chunk_symbols a
 * multiple of 256, chunk_symbols / 16 dividing cols, out_elem_offset a
 * multiple of 16 and shared tables (else ENTQ_EINVAL). Such tensors go to
 * entq_decode_gemm_tiles / entq_decode_gemm_tiles_bf16_split, and
 * entq_decode / entq_decode_bf16_split write their ordinary row-major
 * outputs (codes, bf16 or the source bf16) when every tensor of the plan is
 * in tile order (at most 16 tensors; a plan mixing the layouts or with more
 * tensors: ENTQ_EINVAL there). The
 * row-major fused calls (entq_decode_gemm*) refuse them. */
#define ENTQ_LAYOUT_TILES 0x100u

/* One tensor of a batch (40 bytes). rows x cols row-major; n_symbols must be
 * rows * cols. Output element i of the tensor goes to out[out_elem_offset +
 * i]; its scale is scales[scale_row_offset + i / cols]. */
typedef struct {
    uint32_t kind;            /* entq_symkind, | ENTQ_LAYOUT_TILES           */
    uint32_t rows, cols;
    uint32_t chunk_symbols;   /* C: a positive multiple of 64, <= 2^20       */
    uint64_t n_symbols;
    uint64_t out_elem_offset;
    uint64_t scale_row_offset;
} entq_tensor_desc;

/* One chunk (32 bytes): symbols [elem_offset, elem_offset + n_symbols) of
 * tensor `tensor`, its region at byte_offset in the blob. */
typedef struct {
    uint32_t tensor;
    uint32_t n_symbols;       /* 1 .. chunk_symbols                          */
    uint32_t n_words;         /* <= n_symbols                                */
    uint32_t reserved;        /* 0                                           */
    uint64_t byte_offset;     /* multiple of 16                              */
    uint64_t elem_offset;     /* k * chunk_symbols for the tensor's chunk k  */
} entq_chunk_desc;

/* Opaque plan handle (host memory owned by the library). */
typedef struct entq_plan_s entq_plan_t;

/* Bytes of device workspace a plan over n_tensors tensors and n_chunks
 * chunks needs. */
size_t entq_plan_workspace_bytes(int n_tensors, int64_t n_chunks);

/* Validates the batch and builds the decoder's device-side tables and chunk
 * lists in d_workspace (copied on `stream`).
 *   tensors      host [n_tensors]
 *   freq_tables  host [n_tensors][256]; each table of a non-empty tensor must
 *                sum to 4096 and give every coded symbol a nonzero entry
 *   chunk_index  host [n_chunks]: the chunks of every tensor must tile
 *                [0, n_symbols) exactly (any order); regions must lie inside
 *                [0, blob_bytes)
 *   blob_bytes   size of the compressed buffer later passed to decode
 *   d_workspace  device, >= entq_plan_workspace_bytes(), 256-byte aligned
 * Checks also that tensor outputs do not overlap. Returns ENTQ_OK and a new
 * plan in *out, or an error and *out = NULL. Host inputs may be freed after
 * return. The upload is ordered on `stream` only: a decode enqueued on
 * another stream must be ordered after it (an event or a stream wait).
 * entq_plan_destroy waits for the upload to finish before it frees the
 * plan's host copy. */
entq_status entq_plan(const entq_tensor_desc *tensors, int n_tensors,
                      const uint16_t *freq_tables,
                      const entq_chunk_desc *chunk_index, int64_t n_chunks,
                      uint64_t blob_bytes,
                      void *d_workspace, size_t workspace_bytes, void *stream,
                      entq_plan_t **out);

/* A plan over chunks that carry their own tables. EntroLLM names adaptive
 * entropy coding as its next step [EntroLLM summary, "Significado y
 * Afirmaciones"]; here every chunk is coded with the table of its own counts.
 * The region of a chunk is u16 freq[256] (ENTQ_TABLE_BYTES, sum 4096), then
 * the 64 states and the words as in a shared-table region, zero-padded to 16
 * bytes (entq_encode_tensor_adaptive writes it). Same arguments as entq_plan
 * without tables; every tensor needs chunk_symbols a multiple of 256 and
 * out_elem_offset a multiple of 16, and INT8 and E4M3 tensors cols a multiple
 * of 256 (else ENTQ_EINVAL). entq_decode and, for a plan of BF16EXP tensors,
 * entq_decode_bf16_split work on such a plan (a chunk whose table does not
 * sum to 4096 gets ENTQ_CHUNK_BAD_TABLE and no output); entq_decode_gemm and
 * entq_decode_gemm_bf16_split reject it. */
entq_status entq_plan_adaptive(const entq_tensor_desc *tensors, int n_tensors,
                               const entq_chunk_desc *chunk_index, int64_t n_chunks,
                               uint64_t blob_bytes, void *d_workspace, size_t workspace_bytes,
                               void *stream, entq_plan_t **out);

/* Decodes every chunk of the plan in one launch.
 *   d_compressed  device blob (16-byte aligned, blob_bytes long)
 *   d_out         device; uint8 [total] for ENTQ_OUT_CODES, uint16 (bf16
 *                 bit patterns) [total] for ENTQ_OUT_BF16, where total =
 *                 max(out_elem_offset + n_symbols) over tensors; 16-byte
 *                 aligned
 *   d_scales      device fp32, required for ENTQ_OUT_BF16 (INT8 and E4M3
 *                 tensors only; BF16EXP tensors need entq_decode_bf16_split),
 *                 ignored for ENTQ_OUT_CODES
 *   d_chunk_status device int32 [n_chunks] or NULL */
entq_status entq_decode(const entq_plan_t *plan, const void *d_compressed, void *d_out,
                        entq_outkind out_kind, const float *d_scales,
                        int32_t *d_chunk_status, void *stream);

/* Decodes a plan whose tensors are all ENTQ_SYM_BF16EXP into bf16 words
 * [DFloat11 write-up, "Formato DFloat11"]: the coded exponent bytes come
 * from d_exp_stream (the blob), the raw sign+mantissa byte of output element
 * i is d_signmant[i] (same indexing as d_out). d_out and d_signmant are
 * 16-byte aligned. The plan may be a shared-table (entq_plan) or a
 * per-chunk-table (entq_plan_adaptive) one. */
entq_status entq_decode_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                   const uint8_t *d_signmant, uint16_t *d_out,
                                   int32_t *d_chunk_status, void *stream);

void entq_plan_destroy(entq_plan_t *plan);

const char *entq_status_str(entq_status status);

/* Facts about a plan (for callers sizing buffers and for byte accounting):
 * total output elements, scale rows, chunks, tensors and blob bytes. */
entq_status entq_plan_info(const entq_plan_t *plan, uint64_t *out_elems, uint64_t *scale_rows,
                           int64_t *n_chunks, int *n_tensors, uint64_t *blob_bytes);

/* ---- Host-side encoder (offline compression; multi-threaded C++) ---- */

/* Counts of each byte value in symbols[0..n). */
entq_status entq_count_symbols(const uint8_t *symbols, uint64_t n, uint64_t counts[256],
                               int n_threads);

/* Quantises counts to a table summing to 4096: every present symbol gets at
 * least 1; the sum is corrected by taking from the largest frequencies
 * (smallest byte on ties) or giving to the most frequent symbol; a single
 * present symbol gets 4096. An all-zero count vector gives an all-zero
 * table (empty tensor). */
entq_status entq_build_freq(const uint64_t counts[256], uint16_t freq[256]);

/* Upper bound on the blob bytes one tensor can take. */
uint64_t entq_encode_bound(uint64_t n_symbols, uint32_t chunk_symbols);

/* Encodes n symbols of one tensor into consecutive chunk regions written to
 * out[0 ..). chunks_out[k] (k < ceil(n / C)) receives the chunk descriptors
 * with tensor = tensor_id and byte_offset = base_offset + the region's
 * position in out. *bytes_written is the total. Multi-threaded over chunks. */
entq_status entq_encode_tensor(const uint8_t *symbols, uint64_t n, uint32_t chunk_symbols,
                               const uint16_t freq[256], uint32_t tensor_id,
                               uint64_t base_offset, uint8_t *out, uint64_t out_cap,
                               entq_chunk_desc *chunks_out, uint64_t *bytes_written,
                               int n_threads);

/* entq_encode_tensor with per-chunk tables: chunk k is coded with
 * entq_build_freq of its own counts, written as the first ENTQ_TABLE_BYTES
 * of its region (see entq_plan_adaptive). */
entq_status entq_encode_tensor_adaptive(const uint8_t *symbols, uint64_t n,
                                        uint32_t chunk_symbols, uint32_t tensor_id,
                                        uint64_t base_offset, uint8_t *out, uint64_t out_cap,
                                        entq_chunk_desc *chunks_out, uint64_t *bytes_written,
                                        int n_threads);

/* Upper bound on the bytes of one tensor with per-chunk tables. */
uint64_t entq_encode_bound_adaptive(uint64_t n_symbols, uint32_t chunk_symbols);

/* Splits bf16 words into exponent bytes ((w >> 7) & 0xFF) and sign+mantissa
 * bytes ((w >> 15) << 7 | (w & 0x7F)). */
entq_status entq_bf16_split(const uint16_t *w, uint64_t n, uint8_t *exp_out, uint8_t *sm_out,
                            int n_threads);

/* ---- Fused decode + product with activations ----
 *
 * EntQuant expects fused kernels to make entropy-coded weights cheaper at
 * inference [EntQuant, "Float8@2bits: Entropy Coding Enables Data-Free Model
 * Compression", technical summary §5]; the discussion under the DFloat11
 * write-up proposes a matrix multiply that decompresses each tile. For every
 * tensor t of the plan, with W_t its weights as entq_decode(..., ENTQ_OUT_BF16)
 * would write them (bf16, rows x cols):
 *     Y_t[i][r] = sum_c X_t[i][c] * W_t[r][c]     (i < m, fp32 accumulation)
 * The decoded weights are never written to memory.
 *
 * io[t]: d_x = bf16 activations X_t, m rows of cols values, row stride ldx
 * elements (8-byte aligned, ldx a multiple of 4, ldx >= cols); d_y = fp32
 * results Y_t, m rows of `rows` values, row stride ldy >= rows (4-byte
 * aligned). All device memory, caller-owned; outputs of different tensors
 * must not overlap. 1 <= m <= 64.
 * Requirements on the plan's tensors (else ENTQ_EINVAL): kind INT8 or E4M3 (BF16
 * exponent streams: entq_decode_gemm_bf16_split),
 * cols a multiple of 256, chunk_symbols a multiple of cols (every chunk
 * holds whole rows). d_chunk_status as in entq_decode. Enqueued on stream;
 * the summation order is fixed (results are reproducible run to run).
 *
 * Two kernels compute the product. For m <= 4 (and plans of at most 16
 * tensors) it runs on the vector units inside the decode loop: each lane
 * adds the products of its 4 weights per 256 columns with v_dot2_f32_bf16,
 * the 64 lanes' sums of a weight row are added in a fixed tree, and no
 * workspace is used. Otherwise weight tiles go through the matrix cores
 * (v_mfma_f32_16x16x16_bf16) and partial sums are added across waves. Both
 * stay within cols * 2^-24 * sum_c |X[i][c] W[r][c]| of the exact product;
 * their summation orders differ, so results at m <= 4 and m > 4 are not
 * bitwise comparable.
 *
 * d_workspace: NULL, or device memory (256-byte aligned, at least
 * entq_decode_gemm_workspace_bytes(plan, m) bytes, else ENTQ_EALIGN /
 * ENTQ_EWORKSPACE) into which the call first copies each tensor's
 * activations in the order the kernel's waves read them, so that every wave
 * reads one contiguous run per 256 columns instead of 16 rows of 32 bytes.
 * The results are the same bit for bit either way; with more than 16
 * activation rows the workspace makes the call several times faster. The
 * workspace must not be used by other work while the call runs. For m <= 4
 * it is not touched. */
typedef struct {
    const void *d_x;
    uint64_t ldx;
    float *d_y;
    uint64_t ldy;
} entq_gemm_io;

/* Bytes of workspace entq_decode_gemm and entq_decode_gemm_bf16_split take
 * for this plan and m (0 for invalid arguments): for each non-empty tensor,
 * 2 bytes x 16 ceil(m / 16) rows x cols, rounded up to 256. */
uint64_t entq_decode_gemm_workspace_bytes(const entq_plan_t *plan, int m);

entq_status entq_decode_gemm(const entq_plan_t *plan, const void *d_compressed,
                             const float *d_scales, const entq_gemm_io *io, int m,
                             void *d_workspace, uint64_t workspace_bytes,
                             int32_t *d_chunk_status, void *stream);

/* entq_decode_gemm with the packed activations in the library's own static
 * device scratch instead of a caller's workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). It allocates nothing: the
 * scratch is a file-scope device array of ENTQ_GEMM_STATIC_SCRATCH_BYTES
 * that each GPU holds from the library's first use on it until the process
 * ends. Arguments and results as entq_decode_gemm (Int8 / E4M3 plans); the
 * results are bit for bit those of entq_decode_gemm. Returns ENTQ_ETOOLARGE
 * when entq_decode_gemm_workspace_bytes(plan, m) exceeds the scratch (16
 * MiB: every 70B-shaped layer at m <= 64), ENTQ_EHIP if the scratch's
 * address cannot be looked up on the stream's device. Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and must be ordered by
 * the caller. */
#define ENTQ_GEMM_STATIC_SCRATCH_BYTES (16u << 20)

entq_status entq_decode_gemm_static(const entq_plan_t *plan, const void *d_compressed,
                                    const float *d_scales, const entq_gemm_io *io, int m,
                                    int32_t *d_chunk_status, void *stream);

/* The same product for BF16 weights stored as a coded exponent stream plus
 * raw sign+mantissa bytes [DFloat11 write-up, "Formato DFloat11"]: W_t is
 * the bf16 that entq_decode_bf16_split would write (bit-exact original
 * weights), d_signmant as for that call (16-byte aligned, indexed like its
 * output). The plan's non-empty tensors must all be ENTQ_SYM_BF16EXP with
 * out_elem_offset a multiple of 16; the other requirements and io[] as for
 * entq_decode_gemm. */
entq_status entq_decode_gemm_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                        const uint8_t *d_signmant, const entq_gemm_io *io,
                                        int m, void *d_workspace, uint64_t workspace_bytes,
                                        int32_t *d_chunk_status, void *stream);

/* ---- Fused product on tile-ordered chunks ----
 *
 * The pages cut the coded stream into independently decodable segments
 * [EntroLLM, "Metodología", item 3] and leave the order of symbols inside a
 * segment open; the discussion under the DFloat11 write-up asks for tiles
 * decompressed inside the matrix multiply. In the library's tile order a
 * tensor [rows x cols] (rows a multiple of 16; C, the columns per chunk, a
 * multiple of 16 dividing cols) is cut into chunks of 16 rows x C columns:
 * chunk k = band b = k / (cols / C) (rows 16b .. 16b+15) and column chunk
 * c = k % (cols / C) (columns cC .. cC+C-1), and position p = 256 t + 64 s
 * + l (0 <= s < 4, 0 <= l < 64) of the chunk holds the weight at row
 * 16 b + l % 16, column c C + 16 t + 4 (l / 16) + s. Only the order of the
 * symbols changes; the table, coder and container are as for any tensor:
 * encode the reordered symbols with chunk_symbols = 16 C and mark the tensor
 * ENTQ_LAYOUT_TILES. */

/* The symbols of one row-major tensor (codes, rows x cols bytes) in tile
 * order with chunk_cols = C columns per chunk, into out (rows x cols bytes,
 * caller-owned, not overlapping codes). ENTQ_EINVAL if the shape does not
 * fit the tile order. n_threads <= 0: all hardware threads. */
entq_status entq_tile_order(const uint8_t *codes, uint32_t rows, uint32_t cols,
                            uint32_t chunk_cols, uint8_t *out, int n_threads);

/* The same on the device: d_codes (4-byte aligned) and d_out (rows x cols
 * bytes each, not overlapping) in device memory; enqueued on stream, for
 * the device encoder (entq_encode_device_batch) to code the result. */
entq_status entq_tile_order_device(const uint8_t *d_codes, uint32_t rows, uint32_t cols,
                                   uint32_t chunk_cols, uint8_t *d_out, void *stream);

/* Bytes of workspace entq_decode_gemm_tiles needs for this plan and m (0 for
 * invalid arguments): the activations packed in the order the waves read
 * them (as entq_decode_gemm_workspace_bytes counts them), and for each
 * tensor with cols / C > 1 column chunks 4 bytes x (cols / C) x m x rows of
 * partial sums, each rounded up to 256. */
uint64_t entq_decode_gemm_tiles_workspace_bytes(const entq_plan_t *plan, int m);

/* Y_t = X_t . W_t^T as entq_decode_gemm computes it (io[], m <= 64, fp32
 * results, W_t the bf16 of code x row scale rounded to nearest even), for a
 * plan whose non-empty tensors (at most 16; kind INT8 or E4M3) are in tile
 * order (kind | ENTQ_LAYOUT_TILES): rows a multiple of 16, chunk_symbols =
 * 16 C with C a multiple of 16 that divides cols (else ENTQ_EINVAL). Every
 * wave
 * decodes its own chunks and, for each 16 x 16 tile, issues one
 * v_mfma_f32_16x16x16_bf16
 * per 16 activation rows straight from its registers: no workgroup barrier
 * and no staging of weights. A first enqueued kernel copies the activations
 * into d_workspace in the order the waves read them (512 contiguous bytes
 * per 16 columns and 16 rows). A chunk's 16 x C product
 * goes to Y directly when C = cols; otherwise to a partial-sum slot of
 * d_workspace, and a last enqueued kernel adds a row's column chunks in
 * column order. d_workspace: required (256-byte aligned, at least
 * entq_decode_gemm_tiles_workspace_bytes, else ENTQ_EALIGN /
 * ENTQ_EWORKSPACE; not used by other work while the call runs). Results are reproducible run to run and stay within
 * cols * 2^-24 * sum_c |X[i][c] W[r][c]| of the exact product; their
 * summation order differs from entq_decode_gemm's. d_chunk_status as in
 * entq_decode. */
entq_status entq_decode_gemm_tiles(const entq_plan_t *plan, const void *d_compressed,
                                   const float *d_scales, const entq_gemm_io *io, int m,
                                   void *d_workspace, uint64_t workspace_bytes,
                                   int32_t *d_chunk_status, void *stream);

/* The same product for BF16 weights stored as a coded exponent stream plus
 * raw sign+mantissa bytes [DFloat11 write-up, "Formato DFloat11"], both in
 * tile order: the tensors are ENTQ_SYM_BF16EXP | ENTQ_LAYOUT_TILES, d_signmant
 * holds the tile-ordered sign+mantissa bytes indexed like the exponent
 * symbols (out_elem_offset + stream position; any alignment), W_t is the
 * original bf16 bit for bit. Other arguments, workspace and requirements as
 * for entq_decode_gemm_tiles. */
entq_status entq_decode_gemm_tiles_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                              const uint8_t *d_signmant, const entq_gemm_io *io,
                                              int m, void *d_workspace,
                                              uint64_t workspace_bytes, int32_t *d_chunk_status,
                                              void *stream);

/* ---- On-device encoder (one wavefront per chunk; same regions as the
 * host encoder, byte for byte) ----
 *
 * The pages compress with a GPU ANS library before deployment [EntQuant,
 * "Float8@2bits: Entropy Coding Enables Data-Free Model Compression",
 * technical summary §2 "Codificación de Pesos"]; these calls encode the
 * library's own format on the GPU. A tensor is encoded in three enqueued
 * steps:
 *   1. entq_count_symbols_device -> counts -> entq_build_freq_device (or a
 *      copy to the host and entq_build_freq there)
 *   2. entq_encode_device -> per-chunk word counts; region k takes
 *      entq_region_bytes(n_words[k]) bytes at a 16-byte-aligned offset, laid
 *      out on the device by entq_region_offsets_device (or on the host)
 *   3. entq_pack_device -> the regions in the caller's blob
 * Nothing needs to reach the host before step 3; the word counts and
 * offsets are read back once, after it, for the chunk index.
 * All buffers are caller-owned device memory; all work is enqueued on
 * `stream` and nothing synchronises. */

/* Adds the counts of each byte value in d_symbols[0..n) to d_counts[256]
 * (device u64, 8-byte aligned; the caller zeroes it first). d_symbols is
 * 16-byte aligned. */
entq_status entq_count_symbols_device(const uint8_t *d_symbols, uint64_t n, uint64_t *d_counts,
                                      void *stream);

/* Bytes of scratch entq_encode_device needs for n symbols in chunks of
 * chunk_symbols: per chunk 64 states and room for one word per symbol. */
uint64_t entq_encode_device_scratch_bytes(uint64_t n_symbols, uint32_t chunk_symbols);

/* Bytes of the region of a chunk with n_words words: 256 + 2 n_words,
 * rounded up to 16. */
uint64_t entq_region_bytes(uint32_t n_words);

/* Encodes the n symbols of one tensor (d_symbols, device, 16-byte aligned)
 * in chunks of chunk_symbols (a multiple of 64, at most 2^20) with the host
 * table freq[256] (sum 4096). Chunk k's final states and words go to
 * d_scratch (device, 16-byte aligned, at least
 * entq_encode_device_scratch_bytes; layout private to the library) and its
 * word count to d_n_words[k] (device u32), or 0xFFFFFFFF if the chunk holds
 * a symbol whose frequency is 0 (such a chunk cannot be coded; pack skips
 * it). Returns ENTQ_EBADTABLE for a table not summing to 4096. */
entq_status entq_encode_device(const uint8_t *d_symbols, uint64_t n, uint32_t chunk_symbols,
                               const uint16_t freq[256], void *d_scratch, uint64_t scratch_bytes,
                               uint32_t *d_n_words, void *stream);

/* One tensor of a batched device encode (all pointers device memory). */
typedef struct {
    const uint8_t *d_symbols;  /* n_symbols codes, 16-byte aligned */
    uint64_t n_symbols;
    uint32_t chunk_symbols;    /* multiple of 64, at most 2^20 */
    uint32_t reserved;
    const uint16_t *d_freq;    /* the tensor's table [256], sum 4096 */
    void *d_scratch;           /* entq_encode_device_scratch_bytes(n_symbols, chunk_symbols) */
    uint64_t scratch_bytes;
    uint32_t *d_n_words;       /* [ceil(n_symbols / chunk_symbols)] */
} entq_encode_job;

/* entq_encode_device for several tensors in as few launches as possible
 * (one per 16 tensors), so that small tensors' chunks run beside the large
 * ones'. The tables are read on the device: a table that does not sum to
 * 4096 (or has an entry above 4096) marks every chunk of its tensor with
 * 0xFFFFFFFF instead of an error code. Empty tensors are skipped. */
entq_status entq_encode_device_batch(const entq_encode_job *jobs, int n_jobs, void *stream);

/* Byte counts of several device arrays in one launch (one per 16 arrays):
 * job j adds the counts of d_symbols[0 .. n_symbols) (16-byte aligned) to
 * d_counts[256] (device u64, 8-byte aligned, zeroed by the caller). */
typedef struct {
    const uint8_t *d_symbols;
    uint64_t n_symbols;
    uint64_t *d_counts;
} entq_count_job;

entq_status entq_count_symbols_device_batch(const entq_count_job *jobs, int n_jobs,
                                            void *stream);

/* entq_pack_device for several tensors writing into one blob, in one launch
 * per 16 tensors; each job as that call's arguments (device pointers). */
typedef struct {
    const void *d_scratch;
    uint64_t n_symbols;
    uint32_t chunk_symbols;
    uint32_t reserved;
    const uint32_t *d_n_words;
    const uint64_t *d_byte_offsets;
} entq_pack_job;

entq_status entq_pack_device_batch(const entq_pack_job *jobs, int n_jobs, void *d_blob,
                                   void *stream);

/* Writes the regions of an encoded tensor into d_blob (device, 16-byte
 * aligned): region k (64 states, the chunk's words in decoding order, zero
 * padding) at byte d_byte_offsets[k] (device u64, multiples of 16, regions
 * not overlapping; the caller lays them out with entq_region_bytes). */
entq_status entq_pack_device(const void *d_scratch, uint64_t n, uint32_t chunk_symbols,
                             const uint32_t *d_n_words, const uint64_t *d_byte_offsets,
                             void *d_blob, void *stream);

/* Lays out consecutive regions: d_byte_offsets[k] = base_offset + the sum of
 * entq_region_bytes(d_n_words[i]) over i < k, and *d_end_offset = base_offset
 * + the sum over all n_chunks (device u32 / u64 / u64). A chunk marked
 * rejected (n_words above 2^20, as entq_encode_device's 0xFFFFFFFF) takes 0
 * bytes, so later regions stay inside the blob's bound. The word counts of
 * several tensors can be scanned in one call when their chunks are
 * consecutive in d_n_words. base_offset is a multiple of 16. */
entq_status entq_region_offsets_device(const uint32_t *d_n_words, uint64_t n_chunks,
                                      uint64_t base_offset, uint64_t *d_byte_offsets,
                                      uint64_t *d_end_offset, void *stream);

/* ---- On-device encoder with per-chunk tables (the regions of
 * entq_plan_adaptive, byte for byte equal to entq_encode_tensor_adaptive's)
 * [EntroLLM summary, "Significado y Afirmaciones"]:
 *   1. entq_count_chunks_device_batch -> per-chunk counts ->
 *      entq_build_freq_device (or on the host, entq_build_freq_chunks)
 *   2. entq_encode_device_adaptive_batch -> word counts
 *   3. entq_region_offsets_device_adaptive -> offsets
 *   4. entq_pack_device_adaptive_batch -> the regions, each headed by its
 *      chunk's table ---- */

/* Counts of every chunk of several device arrays, one launch per 16 arrays:
 * chunk k of job j (bytes k * chunk_symbols .. of d_symbols, 16-byte
 * aligned) writes its 256 counts to d_counts[256 k ..] (device u32, 4-byte
 * aligned, ceil(n_symbols / chunk_symbols) rows). */
typedef struct {
    const uint8_t *d_symbols;
    uint64_t n_symbols;
    uint32_t chunk_symbols;    /* multiple of 64, at most 2^20 */
    uint32_t reserved;
    uint32_t *d_counts;
} entq_chunk_count_job;

entq_status entq_count_chunks_device_batch(const entq_chunk_count_job *jobs, int n_jobs,
                                           void *stream);

/* Host: entq_build_freq applied to each of n_tables rows of 256 counts
 * (u32), written to freq[256 t ..]; n_threads <= 0 uses all cores. */
entq_status entq_build_freq_chunks(const uint32_t *counts, uint64_t n_tables, uint16_t *freq,
                                   int n_threads);

/* entq_build_freq on the device: n_tables rows of 256 counts (device, u32
 * when count_bytes is 4, u64 when 8; aligned to their size) to tables
 * d_freq[256 t ..] (device u16), one wavefront per table, same results as
 * the host call for totals below 2^48. Lets the counts -> tables -> encode
 * sequence run without a host round trip. */
entq_status entq_build_freq_device(const void *d_counts, uint32_t count_bytes, uint64_t n_tables,
                                   uint16_t *d_freq, void *stream);

/* entq_encode_device_batch with one table per chunk: job.d_freq holds
 * ceil(n_symbols / chunk_symbols) tables of 256 u16 (each summing to 4096),
 * the table of chunk k at d_freq[256 k]. A chunk whose table is invalid or
 * lacks one of its symbols gets word count 0xFFFFFFFF. */
entq_status entq_encode_device_adaptive_batch(const entq_encode_job *jobs, int n_jobs,
                                              void *stream);

/* entq_region_offsets_device for regions that start with their table:
 * each takes ENTQ_TABLE_BYTES + entq_region_bytes(n_words) bytes (0 if
 * rejected). */
entq_status entq_region_offsets_device_adaptive(const uint32_t *d_n_words, uint64_t n_chunks,
                                               uint64_t base_offset, uint64_t *d_byte_offsets,
                                               uint64_t *d_end_offset, void *stream);

/* entq_pack_device_batch for regions that start with their table: region k
 * = the 512 bytes of d_freq[256 k ..] (device u16, 4-byte aligned), then
 * the states and words as in a shared-table region. */
typedef struct {
    const void *d_scratch;
    uint64_t n_symbols;
    uint32_t chunk_symbols;
    uint32_t reserved;
    const uint32_t *d_n_words;
    const uint64_t *d_byte_offsets;
    const uint16_t *d_freq;
} entq_pack_adaptive_job;

entq_status entq_pack_device_adaptive_batch(const entq_pack_adaptive_job *jobs, int n_jobs,
                                            void *d_blob, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ENTQ_H */
