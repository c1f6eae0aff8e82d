/*
 * qgemv.h -- C ABI of libqgemv.so: fused dequantize-and-multiply GEMV for
 * weight-only low-bit LLM linear layers at decode batch 1..16, on MI355X
 * (gfx950 / CDNA4).
 *
 * What is computed (every compute entry point):
 *
 *     y[m, n] = sum_k x[m, k] * w[n, k]        0 <= m < M, 0 <= n < N
 *
 * with the weight w given in a compressed form and dequantized on chip,
 * never written back to memory.  The compressed forms are those described by
 *   - QFactory: Accelerating Quantized LLM Serving with Qtile Graphs (ATC'25):
 *     group-wise asymmetric weight-only W8/W4/W2, group 128x1 ("Problem and
 *     motivation"; "Experiments"); zero points handled algebraically
 *     ("Key observations", observation 2);
 *   - Fast NF4 Dequantization Kernels for LLM Inference (abstract): 4-bit codes
 *     indexing a 16-level table with a block-wise absmax scale;
 *   - FlashQuant (abstract): an outlier-aware W4A16 layer = low-bit dense part
 *     plus fp16 outliers in a Tile-COO encoding, both applied in one kernel;
 *   - CodeGEMM (NeurIPS'25 notes, "Overall framework", "Key design 1/4"):
 *     vector-codebook weights evaluated through a Psumbook of precomputed
 *     centroid-activation partial sums, with per-group scales.
 *
 * Common conventions
 * ------------------
 * - Pointers marked [dev] are device pointers (HIP global memory); [host] are
 *   host pointers.  The caller allocates and frees every buffer; the library
 *   keeps no state between calls and allocates nothing.
 * - fp16 values are passed as uint16_t holding IEEE-754 binary16 bits.
 * - x is row-major [M, K] fp16; y is row-major [M, N] fp16 and is fully
 *   overwritten (no accumulate).  y must not overlap any input.
 * - Group size is 128 along K for scales and zero points (g = 128); K must be
 *   a multiple of 128.  1 <= M <= 16, N >= 1.
 * - x and every packed-weight buffer must be 16-byte aligned.
 * - Compute entry points enqueue work on `stream` and return at once; they
 *   never synchronize and never read device data on the host, so data
 *   values are not validated.  Arguments are validated before anything is
 *   enqueued: a failing call enqueues nothing and writes nothing.
 * - Return value: a qgemv_status.  QGEMV_ERR_HIP means a HIP call failed; its
 *   hipError_t is available from qgemv_last_hip_error() (per thread).
 * - Accuracy: every result satisfies |y - y_exact| <= 2e-3 * A + 1e-6 with
 *   A[m, n] = sum_k |x[m,k] * w[n,k]|; accumulation is fp32, output is
 *   rounded to nearest even.  (qgemv_w4a8 states y_exact over its int8
 *   activations, which it computes exactly.)
 *
 * Tuning overrides
 * ----------------
 * For tests and launch-shape sweeps only; normal use sets none of them.  They
 * are read only when QGEMV_TUNING is set in the environment at the library's
 * first call (checked once per process); then they are read on every call,
 * so a sweep can change them between calls.  Each forces a choice the library
 * otherwise makes itself.  A forced shape the kernels do not support is
 * rejected with an error status (or, for QGEMV_CODEBOOK_GEN_KS, ignored).
 *   QGEMV_TILE_CFG="tpw,wk[,mt[,v]]"   uniform kernels (qgemv_w2a16 .. qgemv_uniform)
 *   QGEMV_XLDS_MAX=bytes                uniform kernels: largest activation block
 *                                       staged in LDS (above it, per-wave loads)
 *   QGEMV_PLDS=0|1                      uniform kernels: stage the workgroup's scales
 *                                       and zero points in LDS (1, the default where
 *                                       aligned and they fit) or load them per lane
 *   QGEMV_FULL_ROUNDS=0|1               uniform VALU kernels with the deep chunk ring:
 *                                       when K/128 fills whole rounds of the ring, a
 *                                       kernel without the past-the-last-chunk selects
 *                                       (1, the default) or the general one (0)
 *   QGEMV_XDMA=0|1|2                    matrix-core uniform kernel with activations not
 *                                       staged whole: per-wave LDS ring of activation
 *                                       blocks off (0), where it measured faster (1,
 *                                       the default), wherever the shape allows (2)
 *   QGEMV_OUTLIER_CFG="tpw,wk[,mt[,v]]" qgemv_outlier's fused kernel
 *   QGEMV_OUTLIER_FORM=fused|split      qgemv_outlier: one kernel, or dense then sparse
 *   QGEMV_LUT4_CFG="tpw,ng,wk[,mt[,d]]" qgemv_lut4
 *   QGEMV_LUT4_BS=0|2                   qgemv_lut4: never stage the block scales in
 *                                       LDS (0), or stage them wherever the shape
 *                                       allows (2)
 *   QGEMV_CODEBOOK_CFG="kind,wk,..."    qgemv_codebook's kernel and shape
 *   QGEMV_CODEBOOK_GEN_KS=k             qgemv_codebook_gen: k K parts, or -wk for
 *                                       the stationary kernel with wk waves
 *   QGEMV_DENSE_CFG="tpw,s,wk"          qgemv_gemv_f16
 *   QGEMV_GEMM_KERNEL=1|2               qgemv_gemm_uniform: the GEMM at any M (1), or
 *                                       16-row slices of the decode kernel up to
 *                                       M = 64 (2)
 *   QGEMV_GEMM_MI, QGEMV_GEMM_NT        qgemv_gemm_uniform's GEMM block: 2 or 4
 *                                       16-row MFMA tiles of x by 2 or 4 16-row
 *                                       tile-rows of W per wave (32 or 64 x 128
 *                                       or 256)
 *   QGEMV_GEMM_KH=1|2                   qgemv_gemm_uniform's GEMM: K in one pass (1)
 *                                       or in two halves taken by the two halves
 *                                       of a 512-thread workgroup (2; only with
 *                                       2 tile-rows per wave and K/128 even,
 *                                       else 1)
 *   QGEMV_W4A8_WK, QGEMV_W4A8_TR        qgemv_w4a8: waves and tile-rows (1, 2) per
 *                                       workgroup
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t; NULL means the null stream. */
typedef struct ihipStream_t *qgemv_stream_t;

typedef enum {
  QGEMV_OK = 0,
  QGEMV_ERR_NULL = 1,        /* a required pointer is NULL                 */
  QGEMV_ERR_SHAPE = 2,       /* M, N, K outside the supported ranges       */
  QGEMV_ERR_ALIGN = 3,       /* a pointer breaks the 16-byte alignment rule */
  QGEMV_ERR_UNSUPPORTED = 4, /* bits / path / format not provided          */
  QGEMV_ERR_WORKSPACE = 5,   /* workspace missing or too small             */
  QGEMV_ERR_VALUE = 6,       /* bad data in an offline prep call, or y aliases an input */
  QGEMV_ERR_HIP = 7          /* a HIP runtime call failed                  */
} qgemv_status;

/* Kernel family for the uniform entry points (qgemv_uniform). */
typedef enum {
  QGEMV_PATH_AUTO = 0, /* measured dispatch by (bits, M, N, K)            */
  QGEMV_PATH_VALU = 1, /* VALU dot engine: v_dot2 on unpacked fp16 pairs   */
  QGEMV_PATH_MFMA = 2  /* MFMA dot engine: unpacked pairs as matrix-core B */
} qgemv_path;

#define QGEMV_GROUP 128
#define QGEMV_LUT_BLOCK 64
#define QGEMV_MAX_M 16
#define QGEMV_LUT4_MAX_K 48000
#define QGEMV_SPMV_MAX_K 1048576

/* Weight formats (one per compute family), for qgemv_workspace_bytes. */
typedef enum {
  QGEMV_W2 = 2,        /* qgemv_w2a16 / qgemv_uniform(2, ...)   */
  QGEMV_W4 = 4,        /* qgemv_w4a16 / qgemv_uniform(4, ...)   */
  QGEMV_W8 = 8,        /* qgemv_w8a16 / qgemv_uniform(8, ...)   */
  QGEMV_LUT4 = 16,     /* qgemv_lut4                            */
  QGEMV_OUTLIER4 = 17, /* qgemv_outlier                         */
  QGEMV_CODEBOOK = 18, /* qgemv_codebook                        */
  QGEMV_W4A8 = 19,     /* qgemv_w4a8                            */
  QGEMV_W4A8_SPLIT = 20, /* qgemv_w4a8_split                    */
  QGEMV_W4A8_ASYM = 21   /* qgemv_w4a8_asym                     */
} qgemv_variant;

/* Library version (major*10000 + minor*100 + patch). */
int qgemv_version(void);

/* Version of every packed format this library reads and writes: the device
 * and rows-of-64 code layouts, the plain zero-point packing and the Tile-COO
 * record.  Packed buffers are valid only for a library reporting the same
 * layout version; keep it beside stored packed weights and repack on a
 * mismatch. */
#define QGEMV_LAYOUT_VERSION 1
int qgemv_layout_version(void);

/* Scratch bytes the compute entry point of `variant` needs (or, for
 * QGEMV_CODEBOOK, uses to split K) at batch M and an N x K weight: 0 for the
 * variants that take no workspace (QGEMV_W2/W4/W8, QGEMV_LUT4, QGEMV_OUTLIER4),
 * qgemv_codebook_workspace_bytes(M, N, K) for QGEMV_CODEBOOK and
 * qgemv_w4a8_workspace_bytes(M, K) for QGEMV_W4A8 (and the split / asym
 * queries for QGEMV_W4A8_SPLIT / QGEMV_W4A8_ASYM).  Also 0 for an unknown
 * variant or a shape the variant rejects (its call then reports the error). */
size_t qgemv_workspace_bytes(int variant, int M, int N, int K);
/* Static string for a status code (never NULL). */
const char *qgemv_status_string(int status);
/* hipError_t of the last failed HIP call in this thread (0 if none). */
int qgemv_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Bit packing of b-bit codes (b in {2,4,8}), P = 32/b codes per uint32.
 *
 *   QGEMV_LAYOUT_PLAIN   row-major, each row in ceil(cols*b/32) words; word j
 *                        of a row holds columns [j*P, (j+1)*P), field f (bits
 *                        [b*f, b*f+b)) holding column j*P + f.  The "32/b
 *                        codes per uint32 along K" interchange format of the
 *                        workloads; zero points use this layout.
 *   QGEMV_LAYOUT_DEVICE  (cols % 128 == 0) tiles of 16 rows x 128 columns,
 *                        rows padded with code 0 to a multiple of 16.  Tile
 *                        (rt, g) starts at word (rt*G + g)*64*b, G = cols/128.
 *                        Inside a tile, lane l in [0,64) holds row 16*rt + l%16
 *                        and columns [128g + 32(l/16), +32) as b words: word i
 *                        of lane l is tile word (i/4)*256 + l*min(b,4) + i%4 and
 *                        covers columns 128g + 32(l/16) + P*i + [0,P), field f
 *                        holding offset 2f (f < P/2) or 2(f - P/2) + 1
 *                        (f >= P/2).  Every wave-wide load of a tile is then
 *                        one contiguous block and the two 16-bit halves of a
 *                        word are consecutive columns.  The weights of every
 *                        compute entry point use this layout.
 *
 *   QGEMV_LAYOUT_ROWS64  (b = 8 only) tiles of 64 rows x 16 columns, 1 KB each,
 *                        rows padded to a multiple of 64 and columns to a
 *                        multiple of 16; tile (rb, cb) starts at byte
 *                        (rb*ceil(cols/16) + cb)*1024 and its byte 16l + i
 *                        holds column 16cb + i of row 64rb + l.  A wave-wide
 *                        16-byte load gives every lane 16 codes of its own row.
 *                        The code format of qgemv_codebook.
 *
 * Unused fields (past cols, or padding rows) are zero.
 * ------------------------------------------------------------------------ */
typedef enum { QGEMV_LAYOUT_PLAIN = 0, QGEMV_LAYOUT_DEVICE = 1, QGEMV_LAYOUT_ROWS64 = 2 } qgemv_layout;

/* Number of uint32 words of a packed [rows, cols] matrix in `layout`
 * (0 on bad arguments, including cols % 128 != 0 for the device layout). */
size_t qgemv_packed_words(int bits, int layout, int rows, int cols);

/* codes [dev] uint8 [rows, cols], one code per byte (< 2^bits)
 * packed [dev] uint32 [qgemv_packed_words(bits, layout, rows, cols)]
 * Offline prep: synchronizes `stream`; returns QGEMV_ERR_VALUE (packed
 * contents then unspecified) if any code is >= 2^bits.  The out-of-range flag
 * is one device word per GPU: calls from several host threads are serialized
 * inside the library (each holds a lock from clearing the flag to reading it
 * back), so concurrent calls on different streams stay correct but do not
 * overlap. */
int qgemv_pack(int bits, int layout, int rows, int cols, const uint8_t *codes, uint32_t *packed,
               qgemv_stream_t stream);

/* Inverse of qgemv_pack.  Asynchronous. */
int qgemv_unpack(int bits, int layout, int rows, int cols, const uint32_t *packed, uint8_t *codes,
                 qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * Uniform group-wise asymmetric WbA16 (QFactory review: asymmetric W8/W4/W2,
 * group 128x1):
 *     w[n, k] = s[n, k/128] * (q[n, k] - z[n, k/128])
 *
 *   x      [dev] fp16   [M, K]
 *   wq     [dev] uint32 device-layout b-bit codes
 *                       [qgemv_packed_words(b, QGEMV_LAYOUT_DEVICE, N, K)]
 *   scales [dev] fp16   [N, K/128]
 *   zeros  [dev] uint32 plain-packed b-bit zero points [N, ceil((K/128)*b/32)]
 *   y      [dev] fp16   [M, N]
 * ------------------------------------------------------------------------ */
int qgemv_w2a16(int M, int N, int K, const uint16_t *x, const uint32_t *wq,
                const uint16_t *scales, const uint32_t *zeros, uint16_t *y,
                qgemv_stream_t stream);
int qgemv_w4a16(int M, int N, int K, const uint16_t *x, const uint32_t *wq,
                const uint16_t *scales, const uint32_t *zeros, uint16_t *y,
                qgemv_stream_t stream);
int qgemv_w8a16(int M, int N, int K, const uint16_t *x, const uint32_t *wq,
                const uint16_t *scales, const uint32_t *zeros, uint16_t *y,
                qgemv_stream_t stream);

/* Same computation with an explicit bit width and kernel family (qgemv_path);
 * the w{2,4,8}a16 calls are qgemv_uniform(b, QGEMV_PATH_AUTO, ...).
 *
 * Shapes: 1 <= M <= QGEMV_MAX_M, N >= 1, K a positive multiple of 128, each
 * operand under 2 GiB (QGEMV_ERR_SHAPE otherwise).  x and wq 16-byte aligned,
 * scales and y 2-byte, zeros 4-byte (QGEMV_ERR_ALIGN).  y must not overlap an
 * input (QGEMV_ERR_VALUE).  Checks run in the order null, bits/path, shape,
 * alignment, overlap; nothing is launched on an error.  Asynchronous on
 * `stream`; the caller owns every buffer.  The result is deterministic: the
 * same inputs give the same bits on every call. */
int qgemv_uniform(int bits, int path, int M, int N, int K, const uint16_t *x,
                  const uint32_t *wq, const uint16_t *scales, const uint32_t *zeros,
                  uint16_t *y, qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * LUT4: 4-bit codes with a 16-entry fp16 lookup table (NF4-style) and one
 * fp16 scale per 64 consecutive k of a row (Fast NF4 Dequantization Kernels
 * page: on-chip 16-level table, per-block scale):
 *     w[n, k] = lut[q[n, k]] * absmax[n, k/64]
 *
 *   x      [dev] fp16   [M, K]
 *   wq     [dev] uint32 4-bit codes in the device layout
 *                       [qgemv_packed_words(4, QGEMV_LAYOUT_DEVICE, N, K)]
 *   absmax [dev] fp16   [N, K/64]
 *   lut    [dev] fp16   [16]; any values (the table is an input, not a format)
 *   y      [dev] fp16   [M, N]
 *
 * Shapes as qgemv_uniform, plus K <= QGEMV_LUT4_MAX_K (the activation rows are
 * staged on chip beside the table; QGEMV_ERR_SHAPE beyond).  x and wq 16-byte aligned,
 * absmax, lut and y 2-byte aligned.  y must not overlap an input.  Asynchronous
 * on `stream`, deterministic, no allocation.
 * ------------------------------------------------------------------------ */
int qgemv_lut4(int M, int N, int K, const uint16_t *x, const uint32_t *wq,
               const uint16_t *absmax, const uint16_t *lut, uint16_t *y,
               qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * Outlier-aware W4A16 (FlashQuant abstract: a low-bit dense path and a
 * high-precision sparse path sharing activations and outputs in one kernel,
 * outliers in Tile-COO):
 *     y = x . (W_dense + S)^T
 * W_dense is the uniform 4-bit format of qgemv_w4a16 (its codes are used as
 * given, also at outlier positions); S holds fp16 outliers at unique
 * positions, encoded by qgemv_tilecoo_encode:
 *
 *   tile_ptr [dev] uint32 [qgemv_tilecoo_ptr_len(N, K)]: 16 x 128 tiles (the
 *                  tile of the dense layout) in row-tile-major order (tile
 *                  (r/16) * ceil(K/128) + c/128), exclusive prefix sum of
 *                  record counts; tile_ptr[last] = nnz
 *   tile_rec [dev] uint32 [nnz]: (fp16 value bits << 16) | (row % 16) << 8 |
 *                  (col % 128), sorted by (row, col) inside a tile; may be
 *                  NULL when nnz == 0
 *   nnz            number of records (0 <= nnz <= N*K, nnz*4 < 2^31)
 *
 * Other arguments, shapes and errors as qgemv_uniform (W4, `path` selects the
 * dense engine); tile_ptr and tile_rec 4-byte aligned.  Records are read as
 * given (their validity is the encoder's job; malformed ones give wrong
 * values, never an out-of-bounds access).  Asynchronous, deterministic, no
 * allocation.  On wide layers (N >= 16384) at M >= 4 the call runs the dense
 * kernel and then the sparse kernel of qgemv_spmv_tilecoo, the faster form
 * there; y is then rounded to fp16 twice (after each kernel).
 * ------------------------------------------------------------------------ */
int qgemv_outlier(int path, int M, int N, int K, const uint16_t *x, const uint32_t *wq,
                  const uint16_t *scales, const uint32_t *zeros, const uint32_t *tile_ptr,
                  const uint32_t *tile_rec, int64_t nnz, uint16_t *y, qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * Codebook GEMV with a Psumbook (CodeGEMM paper notes: m = 1 codebook of 256
 * centroids of v = 4 dims, b = 8-bit codes, one scale per g = 128 k):
 *     w[n, 4j + t] = scales[n, (4j + t)/128] * codebook[codes[n, j]][t]
 * computed by building, per 512-k range, the partial sums of every centroid
 * with every 4-wide activation segment on chip and accumulating by lookup.
 *
 *   x        [dev] fp16   [M, K]
 *   codes    [dev] uint32 the [N, K/4] uint8 code matrix packed with
 *                         qgemv_pack(8, QGEMV_LAYOUT_ROWS64, N, K/4, ...)
 *   codebook [dev] fp16   [256][4]
 *   scales   [dev] fp16   [N, K/128]
 *   y        [dev] fp16   [M, N]
 *   ws       [dev] optional workspace of at least
 *                  qgemv_codebook_workspace_bytes(M, N, K) bytes of scratch
 *                  (no initial contents needed) for fp32 partial sums.  With
 *                  it every workgroup builds the Psumbook of one K part once
 *                  and streams many weight rows through it; a second kernel on
 *                  the same stream adds the parts of every output in a fixed
 *                  order.  With NULL or a smaller ws each workgroup walks the
 *                  whole K for its rows, building one Psumbook per 256 k (same
 *                  result within the tolerance, slower).  One buffer may serve
 *                  several shapes; calls that share a workspace must not
 *                  overlap in time.
 *
 * Shapes: 1 <= M <= 16, N >= 1, K a positive multiple of 512 (QGEMV_ERR_SHAPE).
 * x, codes 16-byte aligned, codebook and ws 4-byte, scales and y 2-byte
 * (QGEMV_ERR_ALIGN).  Neither y nor ws may overlap an input, nor each other
 * (QGEMV_ERR_VALUE).  Asynchronous, deterministic for a given workspace size.
 * ------------------------------------------------------------------------ */
int qgemv_codebook(int M, int N, int K, const uint16_t *x, const uint32_t *codes,
                   const uint16_t *codebook, const uint16_t *scales, uint16_t *y, void *ws,
                   size_t ws_bytes, qgemv_stream_t stream);
/* Workspace bytes qgemv_codebook uses to split K for this shape (0 if it
 * never splits, or on bad arguments). */
size_t qgemv_codebook_workspace_bytes(int M, int N, int K);

/* ------------------------------------------------------------------------
 * General codebook GEMV (CodeGEMM paper notes, key design 3: one kernel for
 * any number of codebooks m, vector length v, code bits b and group size g),
 * with m additive codebooks:
 *     w[n, v*j + t] = scales[n, (v*j + t)/group] * sum_i codebooks[i][codes_i[n, j]][t]
 * computed through one Psumbook per codebook (as qgemv_codebook).
 *
 *   ncb        m, the number of codebooks: 1 <= ncb <= v/4 (at most 2 code
 *              bits per weight)
 *   v          vector length: 4, 8 or 16
 *   group      scale group along K: 32, 64 or 128
 *   x          [dev] fp16   [M, K]
 *   codes      [dev] uint32 ncb planes one after the other, plane i being
 *                          codebook i's [N, K/v] uint8 codes packed with
 *                          qgemv_pack(8, QGEMV_LAYOUT_ROWS64, N, K/v)
 *   codebooks  [dev] fp16   [ncb][256][v]
 *   scales     [dev] fp16   [N, K/group]
 *   y          [dev] fp16   [M, N] (written)
 *   ws         [dev] optional scratch of
 *                  qgemv_codebook_gen_workspace_bytes(M, N, K, ncb, v, group)
 *                  bytes for the fp32 partial sums of K parts (added by a
 *                  second kernel in a fixed order); NULL or smaller: one K
 *                  range per workgroup (same result within the tolerance,
 *                  slower).  Calls that share a workspace must not overlap.
 *
 * Shapes: 1 <= M <= 16, N >= 1, K a positive multiple of 256
 * (QGEMV_ERR_SHAPE); other ncb / v / group: QGEMV_ERR_UNSUPPORTED.  codes
 * 16-byte aligned, x and codebooks 8-byte, ws 4-byte, scales and y 2-byte
 * (QGEMV_ERR_ALIGN).  Neither y nor ws may overlap an input, nor each other
 * (QGEMV_ERR_VALUE).  Asynchronous, deterministic for a given workspace size.
 * ------------------------------------------------------------------------ */
int qgemv_codebook_gen(int M, int N, int K, int ncb, int v, int group, const uint16_t *x,
                       const uint32_t *codes, const uint16_t *codebooks, const uint16_t *scales,
                       uint16_t *y, void *ws, size_t ws_bytes, qgemv_stream_t stream);
/* Workspace bytes qgemv_codebook_gen uses to split K (0 if it never splits,
 * or on bad arguments). */
size_t qgemv_codebook_gen_workspace_bytes(int M, int N, int K, int ncb, int v, int group);

/* ------------------------------------------------------------------------
 * W4A8 GEMV with the padding strategy (ADAngel review: arbitrary-precision
 * quantization such as W4A8; DPR's padding extends the low-bit weights to
 * the activation width), on the int8 matrix cores:
 *     s_x[m]  = max_k |x[m, k]| / 127,  x_q = rint(x / s_x) clamped to +-127
 *               (fp32, round half to even; a zero row gives 0)
 *     y[m, n] = s_x[m] * sum_k s[n, k/128] * (q[n, k] - z[n, k/128]) * x_q[m, k]
 * x, wq, scales, zeros, y as qgemv_w4a16 (4-bit uniform format).
 *   ws [dev] scratch of qgemv_w4a8_workspace_bytes(M, K) bytes, 16-byte
 *      aligned: the int8 activations [M, K], then the fp32 scales [M] at the
 *      next 16-byte boundary (left there after the call).  Required
 *      (QGEMV_ERR_WORKSPACE if NULL or smaller).
 * Shapes and the other rules as qgemv_w4a16; ws may not overlap an input or
 * y (QGEMV_ERR_VALUE).  Two kernels on `stream`; deterministic.
 * ------------------------------------------------------------------------ */
int qgemv_w4a8(int M, int N, int K, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
               const uint32_t *zeros, uint16_t *y, void *ws, size_t ws_bytes, qgemv_stream_t stream);
/* Workspace bytes of qgemv_w4a8 (0 on bad arguments). */
size_t qgemv_w4a8_workspace_bytes(int M, int K);

/* ------------------------------------------------------------------------
 * W4A8 by the split strategy (ADAngel review, DPR: decomposition, partial
 * products, reconstruction; split sits between padding and bit-serial
 * decomposition): the same int8 activations and the same result as
 * qgemv_w4a8, with each x_q decomposed as 16 h + l (h in [-8, 7], l in
 * [0, 15]) and each 4-bit operand pair multiplied on the fp8 matrix cores
 * (small integers are exact in fp8 e4m3; v_mfma_f32_16x16x128_f8f6f4), the
 * two partial products added exactly in one fp32 accumulator.  The result is
 * bit for bit that of qgemv_w4a8.
 *   ws [dev] scratch of qgemv_w4a8_split_workspace_bytes(M, K) bytes,
 *      16-byte aligned: the high slices 16 h [M, K] and the low slices l
 *      [M, K] as fp8 e4m3 bytes, then the fp32 scales [M] (each part at a
 *      16-byte boundary).  Required (QGEMV_ERR_WORKSPACE if NULL or smaller).
 * Other arguments and rules as qgemv_w4a8.
 * ------------------------------------------------------------------------ */
int qgemv_w4a8_split(int M, int N, int K, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                     const uint32_t *zeros, uint16_t *y, void *ws, size_t ws_bytes, qgemv_stream_t stream);
size_t qgemv_w4a8_split_workspace_bytes(int M, int K);

/* ------------------------------------------------------------------------
 * W4A8 with asymmetric activations, zero points on both operands (QFactory
 * review, observation 2: the matmul of two zero-point operands expanded
 * through all-ones matrices, so no operand is dequantized element by
 * element):
 *     lo = min(min_k x[m, k], 0), hi = max(max_k x[m, k], 0)      (fp32)
 *     s_x[m] = (hi - lo) / 255, zx[m] = clamp(-128 - rint(lo / s_x), -128, 127)
 *     x_q[m, k] = clamp(rint(x / s_x) + zx, -128, 127)   (a zero row: all 0)
 *     y[m, n] = s_x[m] * sum_k s_w[n, k/128] (q - z[n, k/128]) (x_q - zx[m])
 * evaluated per group as sum q x_q - z sum x_q - zx sum q + 128 z zx on the
 * int8 matrix cores with the raw codes, every term an exact integer.
 *   ws [dev] scratch of qgemv_w4a8_asym_workspace_bytes(M, K) bytes, 16-byte
 *      aligned: x_q [M, K] int8, then s_x fp32 [16], zx int32 [16] and the
 *      group sums of x_q int32 [K/128][16] (each part at a 16-byte
 *      boundary).  Required.
 * Other arguments and rules as qgemv_w4a8.
 * ------------------------------------------------------------------------ */
int qgemv_w4a8_asym(int M, int N, int K, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                    const uint32_t *zeros, uint16_t *y, void *ws, size_t ws_bytes, qgemv_stream_t stream);
size_t qgemv_w4a8_asym_workspace_bytes(int M, int K);

/* qgemv_w4a8 without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation): the int8 activations and row scales go to a
 * scratch array inside the library, one per GPU, held until the process ends
 * (about 1 MiB each).  The call itself allocates and frees nothing.
 * M * K <= QGEMV_W4A8_NOALLOC_MAX_MK (QGEMV_ERR_WORKSPACE beyond); other
 * arguments, checks and results as qgemv_w4a8 (same kernels, same bits).
 * The calling thread's current device must be the device of `stream` and of
 * every buffer.  All calls on one GPU share its scratch and each leaves its
 * x_q and s_x there (every call rewrites what it reads): calls that overlap
 * in time on one GPU (other streams, other threads) race and must be
 * serialized by the caller. */
#define QGEMV_W4A8_NOALLOC_MAX_MK 1048576
int qgemv_w4a8_noalloc(int M, int N, int K, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                       const uint32_t *zeros, uint16_t *y, qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * Prefill-size GEMM of the uniform format (any M), the compute-bound regime
 * the decode kernels give way to as the batch grows (QFactory review, "Key
 * observations"; ADAngel review: batch growth turns kernels compute-bound):
 *     y = x . (s * (q - z))^T        x [dev] fp16 [M, K], y [dev] fp16 [M, N]
 * Other arguments as qgemv_uniform (bits 2, 4, 8; the same packed weights).
 * M >= 1 with M*K*2 and M*N*2 below 2^31, N >= 1, K a positive multiple of
 * 128 (QGEMV_ERR_SHAPE); alignment and overlap rules as qgemv_uniform.
 * Up to 16 rows: the decode kernel; 17 to 64: the decode kernel on each
 * 16-row slice of x or the GEMM, by a cost model of the two; beyond: a
 * GEMM on the matrix cores, 32- or 64-row x 128- or 256-column output
 * blocks, fp32 accumulation with one scale per group.  Asynchronous,
 * deterministic.
 * ------------------------------------------------------------------------ */
int qgemv_gemm_uniform(int bits, int M, int N, int K, const uint16_t *x, const uint32_t *wq,
                       const uint16_t *scales, const uint32_t *zeros, uint16_t *y,
                       qgemv_stream_t stream);

/* ------------------------------------------------------------------------
 * Unfused baselines: the kernel sequences that the fused entry points above
 * replace, for measuring what fusion buys.  Same results within the
 * tolerance; more HBM traffic and one more launch.
 *
 * Eager dequantization (Fast NF4 Dequantization Kernels page, method: codes
 * read from global memory, dequantized on chip, fp16 weights written back
 * for a separate matrix product; QFactory review, "Problem and motivation":
 * eager per-element dequantization), writing w [dev] fp16 [N, K] row-major:
 *
 *   qgemv_dequant       w[n, k] = s[n, k/128] * (q[n, k] - z[n, k/128]);
 *                       bits in {2, 4, 8}, wq / scales / zeros as qgemv_uniform
 *   qgemv_dequant_lut4  w[n, k] = lut[q[n, k]] * absmax[n, k/64];
 *                       wq / absmax / lut as qgemv_lut4
 *
 * Each weight is the exact product rounded once to fp16 (nearest even).
 * N >= 1, K a positive multiple of 128, N*K*2 < 2^31 (QGEMV_ERR_SHAPE); wq
 * and w 16-byte aligned, scales / absmax / lut 2-byte, zeros 4-byte
 * (QGEMV_ERR_ALIGN); w may not overlap an input (QGEMV_ERR_VALUE).
 * ------------------------------------------------------------------------ */
int qgemv_dequant(int bits, int N, int K, const uint32_t *wq, const uint16_t *scales,
                  const uint32_t *zeros, uint16_t *w, qgemv_stream_t stream);
int qgemv_dequant_lut4(int N, int K, const uint32_t *wq, const uint16_t *absmax,
                       const uint16_t *lut, uint16_t *w, qgemv_stream_t stream);

/* Dense fp16 GEMV over a dequantized (or any fp16) weight, the second kernel
 * of the eager pattern:
 *     y[m, n] = sum_k x[m, k] * w[n, k]     (fp32 accumulation, fp16 out)
 *   x [dev] fp16 [M, K], w [dev] fp16 [N, K] row-major, y [dev] fp16 [M, N].
 * 1 <= M <= 16, N >= 1, K a positive multiple of 128, N*K*2 < 2^31
 * (QGEMV_ERR_SHAPE); x and w 16-byte aligned, y 2-byte (QGEMV_ERR_ALIGN);
 * y may not overlap an input (QGEMV_ERR_VALUE).  Asynchronous, deterministic. */
int qgemv_gemv_f16(int M, int N, int K, const uint16_t *x, const uint16_t *w, uint16_t *y,
                   qgemv_stream_t stream);

/* Separate sparse kernel of the unfused outlier pattern (FlashQuant abstract:
 * the dense and the sparse path in two kernels sharing activations and
 * outputs).  Adds the Tile-COO outliers (format of qgemv_outlier) into y:
 *     y[m, n] = fp16(y[m, n] + sum over records (n, k, v) of v * x[m, k])
 * with the sum in fp32 in a fixed order; y is read and written (typically the
 * output of qgemv_w4a16 on the same stream).  Rows without outliers keep
 * their bits.  1 <= M <= 16, N >= 1, K a positive multiple of 128 and at most
 * QGEMV_SPMV_MAX_K, 0 <= nnz <= N*K, nnz*4 < 2^31 (QGEMV_ERR_SHAPE); x 16-byte
 * aligned, tile_ptr and tile_rec 4-byte, y 2-byte (QGEMV_ERR_ALIGN); y may not
 * overlap an input (QGEMV_ERR_VALUE).  Records are read as given (malformed
 * ones give wrong values, never an out-of-bounds access).  Asynchronous,
 * deterministic, no allocation. */
int qgemv_spmv_tilecoo(int M, int N, int K, const uint16_t *x, const uint32_t *tile_ptr,
                       const uint32_t *tile_rec, int64_t nnz, uint16_t *y, qgemv_stream_t stream);

/* Entries of tile_ptr for an N x K weight: ceil(N/16) * ceil(K/128) + 1
 * (0 on bad arguments). */
size_t qgemv_tilecoo_ptr_len(int N, int K);

/* Host-side Tile-COO encoder (offline prep; HOST pointers, synchronous).
 *   rows, cols [host] int32 [nnz]: outlier coordinates, 0 <= row < N, 0 <= col < K
 *   val_bits   [host] uint16 [nnz]: fp16 bit patterns of the values
 *   tile_ptr   [host] uint32 [qgemv_tilecoo_ptr_len(N, K)]   (written)
 *   tile_rec   [host] uint32 [nnz]                            (written)
 * Returns QGEMV_ERR_VALUE for a coordinate out of range, a repeated position
 * or an inf/NaN value, QGEMV_ERR_SHAPE for bad N, K or nnz. */
int qgemv_tilecoo_encode(int N, int K, int64_t nnz, const int32_t *rows, const int32_t *cols,
                         const uint16_t *val_bits, uint32_t *tile_ptr, uint32_t *tile_rec);

/* ------------------------------------------------------------------------
 * Measurement: a plain streaming read of a device buffer, the achievable HBM
 * read bandwidth the GEMV kernels are compared with.  Reads every byte of
 * src [dev] once with 16-byte non-temporal loads (a wave-wide load is one
 * contiguous 1 KB burst, as in the weight streams), grid-stride over
 * `workgroups` x `threads`.  Writes sink[0] [dev] only if the XOR of all the
 * data equals a fixed improbable pattern (the result is never needed).
 * bytes a positive multiple of 16, threads a multiple of 64 in [64, 1024],
 * workgroups >= 1 (QGEMV_ERR_SHAPE); src 16-byte aligned, sink 4-byte
 * (QGEMV_ERR_ALIGN).  Asynchronous on `stream`.
 * ------------------------------------------------------------------------ */
int qgemv_stream_read(const void *src, size_t bytes, uint32_t *sink, int workgroups, int threads,
                      qgemv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
