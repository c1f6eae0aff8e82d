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
 *   rounded to nearest even.
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
  QGEMV_PATH_VALU = 1, /* VALU GEMV: dot2 on packed fp16, DPP K-reduction */
  QGEMV_PATH_MFMA = 2  /* MFMA skinny GEMM: dequant into matrix-core operands */
} qgemv_path;

#define QGEMV_GROUP 128
#define QGEMV_LUT_BLOCK 64
#define QGEMV_MAX_M 16

/* Library version (major*10000 + minor*100 + patch). */
int qgemv_version(void);
/* Static string for a status code (never NULL). */
const char *qgemv_status_string(int status);
/* hipError_t of the last failed HIP call in this thread (0 if none). */
int qgemv_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Bit packing of b-bit codes (b in {2,4,8}).
 *
 * A [rows, cols] code matrix is stored row-major, each row in
 * ceil(cols*b/32) uint32 words; word j of a row holds the P = 32/b codes of
 * columns [j*P, (j+1)*P).  Two field orders inside a word:
 *
 *   QGEMV_LAYOUT_PLAIN   field f (bits [b*f, b*f+b)) holds column j*P + f --
 *                        the "32/b codes per uint32 along K" interchange format
 *                        of the workloads; zero points use this layout.
 *   QGEMV_LAYOUT_DEVICE  field f holds column j*P + 2f for f < P/2 and
 *                        j*P + 2(f - P/2) + 1 for f >= P/2, so the two 16-bit
 *                        halves of a word carry consecutive columns (k, k+1);
 *                        the weights of every compute entry point use this.
 *
 * Both layouts have the same size; unused high fields of a row's last word
 * are zero.
 * ------------------------------------------------------------------------ */
typedef enum { QGEMV_LAYOUT_PLAIN = 0, QGEMV_LAYOUT_DEVICE = 1 } qgemv_layout;

/* Number of uint32 words of a packed [rows, cols] matrix (0 on bad args). */
size_t qgemv_packed_words(int bits, int rows, int cols);

/* codes [dev] uint8 [rows, cols], one code per byte (< 2^bits)
 * packed [dev] uint32 [qgemv_packed_words(bits, rows, cols)]
 * Offline prep: synchronizes `stream`; returns QGEMV_ERR_VALUE (packed
 * contents then unspecified) if any code is >= 2^bits. */
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
 *   wq     [dev] uint32 device-packed b-bit codes [N, K*b/32]
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
 * the w{2,4,8}a16 calls are qgemv_uniform(b, QGEMV_PATH_AUTO, ...). */
int qgemv_uniform(int bits, int path, int M, int N, int K, const uint16_t *x,
                  const uint32_t *wq, const uint16_t *scales, const uint32_t *zeros,
                  uint16_t *y, qgemv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
