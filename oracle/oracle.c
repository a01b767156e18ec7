/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, double-precision CPU implementation of the verify-pass
 * product Y[N][M] = X[N][K] * W^T for weights stored as NVFP4 or as
 * row-scaled FP8-E4M3.  It exists so that the HIP path can be checked
 * against something obviously correct.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product
 * library never does, and this file shares no code, header or table with
 * the HIP sources.
 *
 * What it follows:
 *  - crit-hub engine card "mtp7-device-confidence", section "Design"
 *    (row "GEMVs"): the verify pass multiplies FP8 and NVFP4 weight bytes
 *    by BF16 activations for 1-8 columns; section "Checks": such GEMVs are
 *    checked against an FP64 reference.
 *  - crit README (mcpkit.com listing), "Kernel workbench": each kernel is
 *    compared with an FP64 reference on every shape.
 *  - The bit layouts of E2M1, E4M3 and BF16 are not given on those pages;
 *    they are taken from the OCP Microscaling Formats (MX) v1.0 and OCP
 *    8-bit Floating Point (OFP8) specifications and from the definition of
 *    bfloat16 as the upper half of an IEEE binary32.
 *
 * Arithmetic: every weight is decoded from its bit fields with ldexp() into
 * a double, every product is exact in double (at most 2+4+8 significant
 * bits before the FP32 tensor scale, 2+4+8+24 after), and the only rounding
 * is in the K-sum.  Alongside y the oracle returns a = sum |w * x|, the
 * scale of the tolerance |y_gpu - y| <= 1e-3 * a.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoders (format definitions, bit fields -> value) -------- */

/* E2M1: bit 3 sign, bits 2:1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: value = m * 2^-1.  No Inf, no NaN. */
double oracle_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? ldexp((double)m, -1) : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* E4M3 (the "FN" variant): bit 7 sign, bits 6:3 exponent (bias 7), bits 2:0
 * mantissa.  Exponent field 0 is subnormal: value = m * 2^-9.  The two
 * encodings S.1111.111 are NaN; there is no Inf. */
double oracle_e4m3(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  if (e == 15u && m == 7u) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* BF16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---- the two products ------------------------------------------------- */

/* NVFP4 weights.
 *   codes  [M][K/2]  byte j of row m holds k = 2j in its low nibble and
 *                    k = 2j+1 in its high nibble
 *   scales [M][K/16] E4M3; scale b of row m covers k in [16b, 16b+16)
 *   g                FP32 per-tensor multiplier
 *   x      [N][K]    BF16 bits, row-major
 *   rows   list of nrows row indices to compute, or NULL for all M rows
 *   y, a   [N][nrows] doubles: y = sum_k w[m][k] x[n][k], a = sum |w x|
 * where w[m][k] = e2m1(code) * e4m3(scale) * g.
 * K must be a multiple of 16 (whole scale blocks). */
void oracle_gemm_nvfp4(const uint8_t* codes, const uint8_t* scales, float g,
                       const uint16_t* x, int M, int K, int N,
                       const int64_t* rows, int nrows, double* y, double* a) {
  const int64_t R = rows ? nrows : M;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < R; ++r) {
      const int64_t m = rows ? rows[r] : r;
      const uint8_t* crow = codes + m * (int64_t)(K / 2);
      const uint8_t* srow = scales + m * (int64_t)(K / 16);
      for (int k = 0; k < K; ++k) {
        unsigned byte = crow[k / 2];
        unsigned code = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
        w[k] = oracle_e2m1(code) * oracle_e4m3(srow[k / 16]) * (double)g;
      }
      for (int n = 0; n < N; ++n) {
        const uint16_t* xr = x + (int64_t)n * K;
        double s = 0.0, s_abs = 0.0;
        for (int k = 0; k < K; ++k) {
          double p = w[k] * oracle_bf16(xr[k]);
          s += p;
          s_abs += fabs(p);
        }
        y[(int64_t)n * R + r] = s;
        a[(int64_t)n * R + r] = s_abs;
      }
    }
    free(w);
  }
}

/* Row-scaled FP8-E4M3 weights.
 *   w         [M][K] E4M3 bytes
 *   row_scale [M]    FP32; w[m][k] = e4m3(byte) * row_scale[m]
 * Other arguments as above. */
void oracle_gemm_fp8row(const uint8_t* wq, const float* row_scale,
                        const uint16_t* x, int M, int K, int N,
                        const int64_t* rows, int nrows, double* y, double* a) {
  const int64_t R = rows ? nrows : M;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < R; ++r) {
      const int64_t m = rows ? rows[r] : r;
      const uint8_t* wrow = wq + m * (int64_t)K;
      for (int k = 0; k < K; ++k) w[k] = oracle_e4m3(wrow[k]) * (double)row_scale[m];
      for (int n = 0; n < N; ++n) {
        const uint16_t* xr = x + (int64_t)n * K;
        double s = 0.0, s_abs = 0.0;
        for (int k = 0; k < K; ++k) {
          double p = w[k] * oracle_bf16(xr[k]);
          s += p;
          s_abs += fabs(p);
        }
        y[(int64_t)n * R + r] = s;
        a[(int64_t)n * R + r] = s_abs;
      }
    }
    free(w);
  }
}

/* Number of OpenMP threads a parallel region here would use. */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
}

/* Sets the OpenMP thread count of later parallel regions (n >= 1); used
 * only to time the oracle on one thread against all of them. */
void oracle_set_num_threads(int n) {
  if (n >= 1) omp_set_num_threads(n);
}
