/*
 * Plain C reference of the uniform group-wise asymmetric GEMV: test
 * infrastructure only (the oracle side; only tests and the CPU-baseline leg
 * of the benchmark load it).  It shares no code with the HIP library: its own
 * fp16 decoding, its own bit loop over the plain packing, its own sums.
 *
 * What it computes (QFactory (ATC'25) review, "Problem and motivation" and
 * "Experiments": weight-only group-wise asymmetric W8/W4/W2, group 128x1;
 * dequantization read as w = s * (q - z) with an integer zero point of the
 * code's width):
 *
 *   w[n][k] = s[n][k / g] * (q[n][k] - z[n][k / g])
 *   y[m][n] = sum_k x[m][k] * w[n][k]          in double
 *   A[m][n] = sum_k |x[m][k] * w[n][k]|        the tolerance scale
 *
 * for rows n in [row0, row1), written at y[m * (row1 - row0) + (n - row0)].
 * Codes and zero points are in the plain packing: element k of a row of c
 * columns sits in word k / P of the row's ceil(c / P) words, bits
 * [b (k % P), b (k % P) + b), P = 32 / b.  x, s are IEEE binary16 bit
 * patterns.  Every product has at most 11 + 8 + 11 significant bits, so it is
 * exact in double; only the summation rounds.
 *
 * Rows are split over `threads` OpenMP threads (0: the runtime's default).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16 bit pattern -> double (normals, subnormals, zeros, inf, NaN) */
static double half_to_double(uint16_t h) {
  const int sign = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* field k of a plain-packed row of b-bit values */
static unsigned plain_field(const uint32_t *row, int bits, int k) {
  const int per = 32 / bits;
  return (row[k / per] >> (bits * (k % per))) & ((1u << bits) - 1u);
}

int qref_gemv_uniform(int bits, int M, int N, int K, int g, const uint16_t *x, const uint32_t *codes,
                      const uint16_t *scales, const uint32_t *zeros, int row0, int row1, double *y, double *A,
                      int threads) {
  if (!(bits == 2 || bits == 4 || bits == 8) || M < 1 || N < 1 || K < 1 || g < 1 || K % g)
    return 1;
  if (row0 < 0 || row1 > N || row0 > row1) return 2;
  const int per = 32 / bits, G = K / g;
  const int cw = (K + per - 1) / per, zw = (G + per - 1) / per;
  const int nr = row1 - row0;
  double *xd = (double *)malloc(sizeof(double) * (size_t)M * K);
  if (!xd) return 3;
  for (size_t i = 0; i < (size_t)M * K; ++i) xd[i] = half_to_double(x[i]);
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(static)
#endif
  for (int n = row0; n < row1; ++n) {
    double *w = (double *)malloc(sizeof(double) * (size_t)K);
    if (!w) continue;
    const uint32_t *qr = codes + (size_t)n * cw, *zr = zeros + (size_t)n * zw;
    for (int gi = 0; gi < G; ++gi) {
      const double s = half_to_double(scales[(size_t)n * G + gi]);
      const double z = (double)plain_field(zr, bits, gi);
      for (int k = gi * g; k < (gi + 1) * g; ++k) w[k] = s * ((double)plain_field(qr, bits, k) - z);
    }
    for (int m = 0; m < M; ++m) {
      const double *xr = xd + (size_t)m * K;
      double acc = 0.0, aacc = 0.0;
      for (int k = 0; k < K; ++k) {
        const double p = xr[k] * w[k];
        acc += p;
        aacc += fabs(p);
      }
      y[(size_t)m * nr + (n - row0)] = acc;
      A[(size_t)m * nr + (n - row0)] = aacc;
    }
    free(w);
  }
  free(xd);
  return 0;
}

int qref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
