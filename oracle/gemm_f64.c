/*
 * Oracle for the tiled GEMM: a plain, slow FP64 triple loop on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (for 0 <= i < M, 0 <= j < N):
 *
 *     out[i,j] = alpha * sum_{k=0}^{K-1} a(i,k) * b(k,j)  +  beta * c(i,j)
 *
 * with every product and partial sum in IEEE binary64, k ascending, a(i,k)
 * and b(k,j) the exact values of the input patterns (16-bit bfloat16 or
 * binary16, 32-bit binary32 words, or 8-bit E4M3 / E5M2 codes), and c(i,j) the
 * FP32 value of the existing output.  The beta term is left out entirely when
 * beta == 0 (the existing output is then never read, so NaN there cannot leak
 * in).  This is the epilogue form "alpha * accumulator + beta * old C" of the
 * Phobos page "Tiles and shared memory" (section "var and let") and the
 * scaling epilogue of the Tylo.jl page "Layouts, storage and ownership"
 * (section "Plans describe work, callers establish readiness"), over an
 * accumulator that is the plain dot product of row i of A and column j of B.
 *
 * Storage: A is row-major with row stride lda (element (i,k) at i*lda + k);
 * B is K-outer/N-inner with row stride ldb (element (k,j) at k*ldb + j);
 * C and out are row-major with strides ldc and ldo.
 *
 * The decoders below are written from the formats' definitions:
 *   bfloat16 = the upper half of an IEEE binary32 pattern;
 *   binary16 = 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits,
 *              subnormals scaled by 2^-24, exponent 31 = Inf/NaN;
 *   binary32 = 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits,
 *              subnormals scaled by 2^-149, exponent 255 = Inf/NaN;
 *   E4M3     = the OCP 8-bit format with 1 sign bit, 4 exponent bits (bias 7),
 *              3 fraction bits, subnormals scaled by 2^-9, no infinities:
 *              exponent 15 with fraction 7 is NaN, every other code is finite
 *              (largest 448);
 *   E5M2     = the OCP 8-bit format with 1 sign bit, 5 exponent bits (bias 15),
 *              2 fraction bits, subnormals scaled by 2^-16, exponent 31 =
 *              Inf/NaN.
 * Both operands have the same element width: 16-bit patterns (A and B each
 * bfloat16 or binary16), 32-bit words (both binary32) or 8-bit codes (A and B
 * each E4M3 or E5M2).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F16 1
#define ORACLE_F32 2
#define ORACLE_F8E4M3 3
#define ORACLE_F8E5M2 4

double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t word = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

double oracle_f16_to_f64(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 10) & 0x1f;
  int frac = bits & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24);               /* zero or subnormal */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac | 0x400), expo - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -mag : mag;
}

double oracle_f32_to_f64(uint32_t bits) {
  int sign = (int)(bits >> 31);
  int expo = (int)((bits >> 23) & 0xff);
  uint32_t frac = bits & 0x7fffffu;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -149);                  /* zero or subnormal */
  } else if (expo == 255) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac | 0x800000u), expo - 150); /* (1 + f/2^23) * 2^(e-127) */
  }
  return sign ? -mag : mag;
}

double oracle_f8e4m3_to_f64(uint8_t bits) {
  int sign = bits >> 7;
  int expo = (bits >> 3) & 0xf;
  int frac = bits & 0x7;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -9);                    /* zero or subnormal: (f/8) * 2^-6 */
  } else if (expo == 15 && frac == 7) {
    mag = NAN;                                        /* the only NaN code (per sign) */
  } else {
    mag = ldexp((double)(frac | 0x8), expo - 10);     /* (1 + f/8) * 2^(e-7) */
  }
  return sign ? -mag : mag;
}

double oracle_f8e5m2_to_f64(uint8_t bits) {
  int sign = bits >> 7;
  int expo = (bits >> 2) & 0x1f;
  int frac = bits & 0x3;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -16);                   /* zero or subnormal: (f/4) * 2^-14 */
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac | 0x4), expo - 17);     /* (1 + f/4) * 2^(e-15) */
  }
  return sign ? -mag : mag;
}

static int is_byte_type(int type) { return type == ORACLE_F8E4M3 || type == ORACLE_F8E5M2; }

/* Bytes per element of an operand type. */
static int width(int type) { return type == ORACLE_F32 ? 4 : is_byte_type(type) ? 1 : 2; }

static double decode8(uint8_t bits, int type) {
  return type == ORACLE_F8E4M3 ? oracle_f8e4m3_to_f64(bits) : oracle_f8e5m2_to_f64(bits);
}

static double decode(uint16_t bits, int type) {
  return type == ORACLE_BF16 ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);
}

/* Element idx of an operand stored as 16-bit patterns, 32-bit words or 8-bit codes. */
static double element(const void* base, int type, int64_t idx) {
  if (type == ORACLE_F32) return oracle_f32_to_f64(((const uint32_t*)base)[idx]);
  if (is_byte_type(type)) return decode8(((const uint8_t*)base)[idx], type);
  return decode(((const uint16_t*)base)[idx], type);
}

/* Decode n 16-bit patterns (test helper: lets the suite compare the decoders
 * with other implementations of the same formats). */
void oracle_decode(const uint16_t* src, int type, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = decode(src[i], type);
}

/* Decode n 8-bit codes of type ORACLE_F8E4M3 or ORACLE_F8E5M2 (same purpose). */
void oracle_decode8(const uint8_t* src, int type, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = decode8(src[i], type);
}

/* Decode n binary32 words (same purpose). */
void oracle_decode32(const uint32_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f32_to_f64(src[i]);
}

/*
 * Returns 0 on success, -1 on a bad argument.  nthreads <= 0 lets OpenMP pick.
 * C may be NULL when beta == 0.
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const void* A, int a_type, int64_t lda,
                    const void* B, int b_type, int64_t ldb,
                    const float* C, int64_t ldc,
                    double alpha, double beta,
                    double* out, int64_t ldo, int nthreads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (a_type < ORACLE_BF16 || a_type > ORACLE_F8E5M2 || b_type < ORACLE_BF16 || b_type > ORACLE_F8E5M2) return -1;
  if (width(a_type) != width(b_type)) return -1;
  if (beta != 0.0 && C == NULL && M > 0 && N > 0) return -1;
  if (M == 0 || N == 0) return 0;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif

  int failed = 0;
#pragma omp parallel
  {
    double* acc = (double*)malloc((size_t)N * sizeof(double));
    if (!acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double a = element(A, a_type, i * lda + k);
          for (int64_t j = 0; j < N; ++j) acc[j] += a * element(B, b_type, k * ldb + j);
        }
        for (int64_t j = 0; j < N; ++j) {
          double v = alpha * acc[j];
          if (beta != 0.0) v += beta * (double)C[i * ldc + j];
          out[i * ldo + j] = v;
        }
      }
      free(acc);
    }
  }
  return failed ? -1 : 0;
}

/* Threads an OpenMP parallel region would use (reported with timings). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
