/*
 * bgg.h -- C ABI of libbgg.so: the linear-layer product y = W.x of a ternary
 * LLM whose weights are trits {-1, 0, +1} with one fp16 scale per 128 weights
 * along K, stored in block-Hadamard-rotated coordinates, in one of two
 * packings.  Built for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by address, title and paragraph or section):
 *   [A] allhereai.com/news/1346, "27B 模型压到 5.95GB，推理能力还保住 98%":
 *       method paragraph (trits, one FP16 scale shared by every 128 weights,
 *       block Hadamard rotation folded into storage); runtime paragraph (the
 *       runtime must apply the Hadamard transform to the activations; the
 *       wrong runtime can load the file and print garbage); packing
 *       paragraph (PTQ1_0 compact trits, PQ2_0 one trit per 2-bit slot, and
 *       which decodes faster where).
 *   [B] 10100.com/article/156675786, "Bonsai 2，把27B压进6个G", section
 *       "它怎么做到的": rotation before ternary rounding; the input needs the
 *       matching transform at inference, and skipping it fails silently.
 *   [C] wmrh.cn/news/471187, section "关键机制": five trits per byte, about
 *       1.6 bits per trit; FP16 group-wise scales.
 *
 * What the library computes (readings of the pages, fixed here):
 *   x'[m] = blockdiag(H_128 / sqrt(128)) x[m]   (Sylvester order, no signs)
 *   y[m][n] = sum_k S[n][k/128] * T[n][k] * x'[m][k]
 * with x and y fp16, x' computed in fp32, sums in fp32.
 *
 * Conventions for every call
 *   - The caller owns every buffer.  Pointers named *_dev are device
 *     pointers (hipMalloc or a framework's device allocator); the others are
 *     host pointers.  The library keeps no pointer after a call returns and
 *     allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls
 *     only enqueue work and never synchronise; argument errors are reported
 *     before anything is enqueued.  A failed launch returns BGG_ERR_HIP.
 *   - Nothing aborts or prints.  Every call returns a bgg_status; a
 *     thread-local message with details is kept for bgg_last_error().
 *   - Device pointers must be 16-byte aligned (fp16 activation rows: K is a
 *     multiple of 128, so every row is aligned when the base is).
 *   - Calls are re-entrant; calls that share a workspace must not overlap.
 */
#ifndef BGG_H
#define BGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Packings of the trits [A packing paragraph; C].  The two tags are checked
 * on every call, so a buffer packed one way cannot be run the other way (the
 * silent-garbage hazard of [A runtime paragraph]). */
typedef enum {
  BGG_FMT_PQ2_0 = 1,   /* one trit per 2-bit slot: code t+1 in {0,1,2}; 2.125 bits/weight */
  BGG_FMT_PTQ1_0 = 2,  /* five trits per byte, base 3 of t+1; 8/5 + 16/128 = 1.725 bits/weight */
  /* Sister formats, named on [C] (opening summary: 1-bit weights {-1, +1}
   * with an FP16 group scale at about 1.125 bits per weight; section
   * 后端支持现状: a ternary "Q2_0_g64" file form); their layouts are this
   * library's reading: */
  BGG_FMT_Q1_0 = 3,    /* one sign bit per weight (1 = +1, 0 = -1); 1 + 16/128 = 1.125 bits/weight */
  BGG_FMT_Q2_0_G64 = 4 /* the PQ2_0 row stream with one FP16 scale per 64; 2 + 16/64 = 2.25 */
} bgg_format;

typedef enum {
  BGG_OK = 0,
  BGG_ERR_NULL = 1,        /* a required pointer is NULL */
  BGG_ERR_FORMAT = 2,      /* unknown format tag */
  BGG_ERR_SHAPE = 3,       /* K not a positive multiple of 128, N < 1, M out of range */
  BGG_ERR_TRIT = 4,        /* a trit outside {-1, 0, 1} */
  BGG_ERR_PACKED_BYTE = 5, /* a PQ2_0 code of 3 or a PTQ1_0 byte >= 243 */
  BGG_ERR_BUFFER = 6,      /* buffer too small or misaligned */
  BGG_ERR_DESC = 7,        /* descriptor not made by bgg_describe, or it disagrees with the call */
  BGG_ERR_HIP = 8,         /* the HIP runtime reported an error */
  BGG_ERR_SCALE = 9        /* a scale that is not a finite fp16 */
} bgg_status;

/* Flags of bgg_ternary_gemv / bgg_ternary_gemm. */
enum {
  /* x is in model coordinates: the call applies the normalised block-128
   * transform first [A runtime paragraph; B].  Without it x must already be
   * x' (so projections that share an input can share one transform). */
  BGG_ROTATE_INPUT = 1u
};

#define BGG_GROUP 128     /* weights per scale = Hadamard block, along K [A method paragraph] */
#define BGG_ROW_TILE 64   /* rows per tile of the device layout (one row per lane) */
#define BGG_CHUNK 16      /* bytes of one row that one lane loads at once */
#define BGG_MAX_GEMV_M 16 /* largest token count of bgg_ternary_gemv */
#define BGG_READ_SLACK 8192 /* zero bytes after the scales of a packed buffer (see below) */

#define BGG_DESC_MAGIC 0x57474742u /* "BGGW" */
#define BGG_DESC_VERSION 3u

/*
 * Descriptor of a packed weight matrix W [N out][K in].  Host struct, filled
 * by bgg_describe, owned and passed back by the caller on every call.
 *
 * Device layout of the packed buffer (total_bytes):
 *   trit region, at offset 0: rows in tiles of 64; the bytes of each row in
 *     the format's canonical row stream (PQ2_0 and Q2_0_G64: row byte j
 *     holds trits 4j..4j+3, trit 4j+i in bits 2i..2i+1 as t+1; PTQ1_0: row
 *     byte j = sum_i (t_{5j+i}+1) 3^i, trits past K are 0; Q1_0: bit i of
 *     row byte j is weight 8j+i, 1 for +1), cut into 16-byte chunks.
 *     Chunk c of row 64*t + l sits at byte ((t*chunks + c)*64 + l)*16, so the
 *     64 rows of a tile read chunk c with one coalesced 1 KiB load.  Rows
 *     past N hold zero trits, bytes past the row stream hold zero trits.
 *   scale region, at scale_offset: fp16 scale s (weights s*scale_group ..)
 *     of row 64*t + l at byte scale_offset + ((t*scales + s)*64 + l)*2;
 *     rows past N hold 0.
 *   slack, at scale_offset + scale_bytes: BGG_READ_SLACK zero bytes.  The
 *     kernels read whole work units without bounds checks, up to seven
 *     chunks past a tile's last chunk and four groups past its last scale;
 *     those bytes meet zero activation terms and add nothing, and the slack
 *     keeps the reads of the last tile inside the buffer.
 */
typedef struct bgg_weights_desc {
  uint32_t magic;        /* BGG_DESC_MAGIC */
  uint32_t version;      /* BGG_DESC_VERSION */
  int32_t format;        /* bgg_format */
  int32_t row_tile;      /* BGG_ROW_TILE */
  int64_t N;             /* output rows */
  int64_t K;             /* input columns, a multiple of 128 */
  int64_t groups;        /* K / 128: blocks of the activation transform */
  int64_t row_tiles;     /* ceil(N / 64) */
  int64_t row_bytes;     /* canonical packed bytes per row: ceil(K/4), ceil(K/5) or K/8 */
  int64_t chunks;        /* ceil(row_bytes / 16) */
  uint64_t trit_bytes;   /* row_tiles * chunks * 1024 */
  uint64_t scale_offset; /* trit_bytes rounded up to 256 */
  uint64_t scale_bytes;  /* row_tiles * scales * 128 */
  uint64_t total_bytes;  /* scale_offset + scale_bytes + BGG_READ_SLACK */
  uint64_t format_bytes; /* N*row_bytes + N*scales*2: the format's own size, no padding */
  int64_t scale_group;   /* weights per fp16 scale: 128, or 64 for Q2_0_G64 */
  int64_t scales;        /* scales per row: K / scale_group */
} bgg_weights_desc;

/* Fill *out for a format and shape: the sizes of [A packing paragraph] and
 * [C] (bits per weight: 2 + 16/128 for PQ2_0, 8/5 + 16/128 for PTQ1_0) and
 * the device layout above.  Host only, no side effects.
 * Errors: BGG_ERR_NULL, BGG_ERR_FORMAT, BGG_ERR_SHAPE. */
bgg_status bgg_describe(int32_t format, int64_t N, int64_t K, bgg_weights_desc* out);

/* Pack trits and scales into the device layout (a0 of the path: offline,
 * once per matrix) [A method and packing paragraphs; C].
 *   trits   host int8 [N][K], row-major, values in {-1,0,1} ({-1,1} for Q1_0),
 *           rotated coordinates
 *   scales  host fp16 bits [N][K/scale_group], row-major
 *   packed  host buffer of desc->total_bytes; every byte is written
 * Errors: BGG_ERR_NULL, BGG_ERR_DESC, BGG_ERR_TRIT, BGG_ERR_SCALE (nothing
 * useful is left in packed after an error). */
bgg_status bgg_pack_weights(const bgg_weights_desc* desc, const int8_t* trits,
                            const uint16_t* scales, void* packed);

/* Lay out canonical row-stream bytes (the format's file form: the packings
 * of [A packing paragraph; C]) in the device layout without decoding them.
 *   canonical  host uint8 [N][desc->row_bytes]
 *   scales     host fp16 bits [N][K/scale_group]
 *   packed     host buffer of desc->total_bytes
 * Errors: BGG_ERR_NULL, BGG_ERR_DESC, BGG_ERR_PACKED_BYTE, BGG_ERR_SCALE. */
bgg_status bgg_repack_canonical(const bgg_weights_desc* desc, const uint8_t* canonical,
                                const uint16_t* scales, void* packed);

/* Check a host copy of a packed buffer: every code valid for its packing
 * [A packing paragraph; C: a PTQ1_0 byte holds five base-3 digits, so bytes
 * past 242 are invalid; a PQ2_0 code 3 is invalid], padding as laid out,
 * every scale a finite fp16 [A method paragraph].  Errors: BGG_ERR_NULL,
 * BGG_ERR_DESC, BGG_ERR_PACKED_BYTE, BGG_ERR_SCALE. */
bgg_status bgg_validate_packed(const bgg_weights_desc* desc, const void* packed);

/* Decode a packed device buffer back to trits and scales [A packing
 * paragraph; C] with the same device decoders the products use (PTQ1_0:
 * the one-token GEMV's LDS table, same builder, same addressing), for
 * checking; not on the hot path.
 *   packed_dev  device, desc->total_bytes
 *   trits_dev   device int8 [N][K]; scales_dev device fp16 bits [N][K/scale_group]
 * Invalid codes decode as t = 0.  Errors: BGG_ERR_NULL, BGG_ERR_DESC,
 * BGG_ERR_BUFFER, BGG_ERR_HIP. */
bgg_status bgg_unpack_weights(const bgg_weights_desc* desc, const void* packed_dev,
                              int8_t* trits_dev, uint16_t* scales_dev, void* stream);

/* x' = blockdiag(H_128/sqrt(128)) x for each of M rows of K fp16 values
 * [A runtime paragraph; B]: the butterflies run in fp32 and x' is rounded to
 * fp16 (nearest even) once.  x_dev and xr_dev are device fp16 [M][K]; they
 * may be the same buffer.  Errors: BGG_ERR_NULL, BGG_ERR_SHAPE (K % 128 or
 * M < 0), BGG_ERR_BUFFER (alignment), BGG_ERR_HIP.  M == 0 is a no-op. */
bgg_status bgg_hadamard_rotate(const void* x_dev, void* xr_dev, int64_t M, int64_t K,
                               void* stream);

/* Offline front end: float weights in model coordinates -> the trits and
 * fp16 scales that bgg_pack_weights takes [B 它怎么做到的: rotate the weight
 * matrix by a Hadamard transform, then round to -1, 0, +1; A method
 * paragraph: one FP16 scale per 128 weights].  For every 128-block of every
 * row: w' = H_128/sqrt(128) times the block (fp32 butterflies; the stored
 * rows are W blockdiag(Hn), so that W x = (W Hn)(Hn x)); the block's scale
 * s = fp16(mean |w'|), rounded to nearest even once (the pages give no scale
 * rule: this is the library's reading); trit = sign(w') where 2|w'| > s,
 * else 0 (the nearest of -s, 0, +s; a tie goes to 0).
 *   w_dev       device float32 [N][K], 16-byte aligned (read only)
 *   trits_dev   device int8 [N][K], 8-byte aligned (written)
 *   scales_dev  device fp16 bits [N][K/128], 2-byte aligned (written)
 * A block whose mean magnitude is past the fp16 range gets an infinite
 * scale, and a non-finite weight a non-finite scale: bgg_pack_weights
 * rejects both (BGG_ERR_SCALE).  Errors: BGG_ERR_NULL, BGG_ERR_SHAPE (K %
 * 128, N < 0, more than 2^40 weights), BGG_ERR_BUFFER (alignment),
 * BGG_ERR_HIP.  N == 0 is a no-op.  Asynchronous on stream. */
bgg_status bgg_rotate_ternarize(const void* w_dev, int64_t N, int64_t K, int8_t* trits_dev,
                                uint16_t* scales_dev, void* stream);

/* Device workspace bytes that bgg_ternary_gemv needs for M tokens (0 on a
 * bad descriptor, M outside 1..16, or K beyond what one call splits: K up
 * to 516096, 322560 for PTQ1_0).  Bookkeeping of this interface, no page
 * passage. */
size_t bgg_gemv_workspace_size(const bgg_weights_desc* desc, int64_t M);

/* Set the row words at the start of a GEMV workspace (the first
 * min(workspace_bytes, 16 MiB)) to zero on `stream`, with a fill kernel
 * (no memset node, so it may be captured in a graph).  For a new
 * workspace, one used for anything else, or one whose last GEMV call
 * failed; every successful GEMV call leaves the words zero by itself.
 * Bookkeeping of this interface, no page passage.
 * Errors: BGG_ERR_NULL, BGG_ERR_BUFFER (misaligned), BGG_ERR_HIP. */
bgg_status bgg_gemv_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-time product, 1 <= M <= 16 tokens: y = x' (S*T)^T with x' the
 * normalised block-128 Walsh-Hadamard transform of x [A method and runtime
 * paragraphs; B 它怎么做到的], for the packings of [A packing paragraph].
 *   packed_dev  device buffer made from bgg_pack_weights output
 *   x_dev       device fp16 [M][K] (model coordinates with BGG_ROTATE_INPUT,
 *               else already rotated)
 *   y_dev       device fp16 [M][N]
 *   workspace   device buffer of at least bgg_gemv_workspace_size(desc, M)
 *               bytes, 16-byte aligned.  Its first 16 MiB hold the row words
 *               of launches that split K (fixed-point partial sums, 8 MiB,
 *               then 8 MiB of coarse words), which must be zero when a call
 *               starts: zero-fill a new workspace once (or call
 *               bgg_gemv_workspace_reset); every GEMV call (any format, K, M
 *               or N) leaves them zero again.  A workspace used for anything
 *               else in between, or after a failed call, must be reset.
 *               The rest is scratch (encoded activations).
 * One launch transforms and encodes the activations and computes y (PQ2_0
 * up to 4 tokens, PTQ1_0 one token); otherwise it is bgg_gemv_prepare
 * followed by bgg_gemv_run.
 * Arithmetic.  x' is computed in fp32 and carried per 128-block as integers
 * |q| <= 2^14 with a power-of-two scale (absolute error at most 2^-14 of the
 * block's largest |x'|); each group's trit sum over q is exact, and is
 * scaled by the group's fp16 scale and accumulated in fp32.  Where K is
 * split over workgroups their partial rows are added as 64-bit fixed-point
 * integers (2^-30 below 2^17 in magnitude, 1/16 above), exact and
 * independent of the order, so the same inputs always give the same bits,
 * and a token's y does not depend on the other tokens of the call.  Every
 * fp16 x and scale is in range; y beyond the fp16 range is +-inf.  A NaN or
 * inf in a token's x makes that token's whole y row NaN.  y is rounded to
 * fp16 once.
 * Errors: BGG_ERR_NULL, BGG_ERR_DESC, BGG_ERR_SHAPE, BGG_ERR_BUFFER,
 * BGG_ERR_HIP.
 */
bgg_status bgg_ternary_gemv(const bgg_weights_desc* desc, const void* packed_dev,
                            const void* x_dev, void* y_dev, int64_t M, uint32_t flags,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * bgg_ternary_gemv for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same product, kernels and bits, with no workspace
 * argument.  Its workspace is a static device array of 32 MiB per GPU (held
 * by each GPU the library runs on until the process ends); a shape whose
 * bgg_gemv_workspace_size exceeds that is rejected with BGG_ERR_SHAPE
 * before anything is enqueued (32 MiB serves every format and M for K up to
 * 262144).  The call allocates nothing: the array's address on the current
 * device is looked up once, and the first call on a device clears the
 * array on `stream` ahead of its own kernels.  All calls on one GPU share
 * the array, so calls that overlap in time on one GPU race; calls that do
 * not overlap may run on any streams.
 * Arguments, flags and errors: as bgg_ternary_gemv (BGG_ERR_HIP also if the
 * array's address cannot be taken).
 */
bgg_status bgg_ternary_gemv_noalloc(const bgg_weights_desc* desc, const void* packed_dev,
                                    const void* x_dev, void* y_dev, int64_t M, uint32_t flags,
                                    void* stream);

/*
 * The two halves of bgg_ternary_gemv [A method and runtime paragraphs; B],
 * for projections that share an input (q, k and v, or gate and up, read the
 * same x): the activation transform of [A runtime paragraph] done once.
 *
 * bgg_gemv_prepare: transform (with BGG_ROTATE_INPUT) and encode the M
 * activation rows x_dev (fp16 [M][K]) into `workspace`.  What it writes
 * there depends only on the format, K and M of `desc`.
 *
 * bgg_gemv_run: y_dev (fp16 [M][N]) = the product of the packed matrix with
 * the activations last prepared in `workspace` (stream order).  Any matrix
 * whose descriptor has the same format and K may use one preparation, as
 * long as the workspace is at least bgg_gemv_workspace_size of that matrix;
 * runs that share a workspace must not overlap in time.
 * Errors of both: as bgg_ternary_gemv.
 */
bgg_status bgg_gemv_prepare(const bgg_weights_desc* desc, const void* x_dev, int64_t M,
                            uint32_t flags, void* workspace, size_t workspace_bytes, void* stream);
bgg_status bgg_gemv_run(const bgg_weights_desc* desc, const void* packed_dev, void* y_dev,
                        int64_t M, void* workspace, size_t workspace_bytes, void* stream);

/* The name under which a profiler lists the GEMV kernel that
 * bgg_ternary_gemv launches for M tokens (host only, bookkeeping of this
 * interface, no page passage; for matching profiles to calls): PQ2_0 with
 * one token "k_mxv1_pq2<5, T>" and two to four "k_mxv_pq2<8>" (one launch
 * that also transforms x); PTQ1_0 with one token "k_gemv_ptq1<1, H, 8,
 * true>" (one launch); otherwise the matrix-core kernel that follows the
 * preparation kernel "k_gemv_prep_mx<...>", e.g. "k_gemv_pq2_mx<5, 8>",
 * "k_gemv_ptq1_mx<8>", "k_gemv_q1_mx<5, 8>" or "k_gemv_q2g64_mx<4, 8>".
 * Errors: BGG_ERR_NULL, BGG_ERR_DESC, BGG_ERR_SHAPE, BGG_ERR_BUFFER (cap too
 * small for the name and its terminating zero). */
bgg_status bgg_gemv_kernel_name(const bgg_weights_desc* desc, int64_t M, char* out, size_t cap);

/* Device workspace bytes that bgg_ternary_gemm uses at most for M tokens
 * (0 on a bad descriptor or M < 1).  Bookkeeping of this interface, no page
 * passage. */
size_t bgg_gemm_workspace_size(const bgg_weights_desc* desc, int64_t M);

/*
 * Prompt-time product for any M >= 1, PQ2_0 and PTQ1_0 [A packing paragraph:
 * prompt processing, where PQ2_0 is the faster packing].  Trits are decoded
 * to fp16 s*t (exact) in registers and multiplied with fp16 x' tiles staged
 * in LDS on the matrix cores, fp32 accumulation, fp16 y.  PTQ1_0's base-3
 * bytes [C: five trits per byte] are turned into 2-bit codes (an LDS table
 * per byte value): when the workspace holds them, by rewriting the weights
 * once per call into the PQ2_0 layout, which the PQ2_0 product then reads;
 * else inside the product, for every block of 128 tokens.
 *   x_dev      device fp16 [M][K] (model coordinates with BGG_ROTATE_INPUT,
 *              else already rotated); y_dev device fp16 [M][N]
 *   workspace  device, 16-byte aligned, bgg_gemm_workspace_size(desc, M)
 *              bytes: x' when BGG_ROTATE_INPUT is set; then, for PTQ1_0,
 *              the weights rewritten to PQ2_0 (the PQ2_0 trit bytes of the
 *              same shape, 256-byte rounded); then, for shapes whose output
 *              blocks fill the GPU unevenly or not at all (few output rows,
 *              long K, short prompts), the fp32 partial sums of a K split
 *              into up to 32 ranges.  A smaller workspace (down to x' only,
 *              or NULL without BGG_ROTATE_INPUT) drops the later parts in
 *              that order: the results differ in the last-bit rounding;
 *              each choice gives bit-identical y for the same inputs.
 * Errors: BGG_ERR_NULL, BGG_ERR_DESC, BGG_ERR_FORMAT (Q1_0, Q2_0_G64),
 * BGG_ERR_SHAPE, BGG_ERR_BUFFER, BGG_ERR_HIP.
 */
bgg_status bgg_ternary_gemm(const bgg_weights_desc* desc, const void* packed_dev,
                            const void* x_dev, void* y_dev, int64_t M, uint32_t flags,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static English name of a status (bookkeeping, no page passage). */
const char* bgg_status_string(int32_t status);

/* Details of the last error raised on the calling thread ("" if none;
 * bookkeeping, no page passage). */
const char* bgg_last_error(void);

/* BGG_DESC_VERSION of the loaded library (bookkeeping, no page passage). */
uint32_t bgg_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BGG_H */
