/*
 * CPU oracle for the dense GEMM path -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library.  The GPU library never links, includes or calls it, and
 * it includes nothing from the GPU library.
 *
 * What it computes (plain definitions, accumulated in IEEE double):
 *
 *   fp32 row-major SGEMM   C = alpha * A * B + beta * C
 *     The operation of the cp.async SGEMM example on the page "异步拷贝与
 *     Hopper/Blackwell 新特性" (section "cp.async 与多级流水", file
 *     gemm_cp_async.cu): each output is alpha times the K-long dot product of
 *     row i of A[M][K] with column j of B[K][N], plus beta times the old C.
 *     The plain triple loop of page 1 ("第 6 章 Shared Memory & Tile",
 *     section 6.1) fixes the row-major indexing A[row*K+k], B[k*N+col].
 *     beta == 0 is read as BLAS does: C is then write-only and its old value
 *     (NaN included) never reaches the result.
 *
 *   16-bit "NT" GEMM       C = A * B^T,  A[M][K], B[N][K] row-major, binary16
 *     or bfloat16 (and the fused write-back C = act(A * B^T + bias) +
 *     residual, see oracle_epilogue16)
 *     The definition in section "0. Naive Implementation" of the page
 *     "从零开始的 AI Infra: 算子基础与GPU架构": C[m][n] is the sum over k of
 *     A[m*K+k] * B[n*K+k], and the result is rounded to half.  Section "19.
 *     去掉转置" confirms that B[n][k] lives at n*K+k.  The page accumulates in
 *     float; this oracle accumulates in double and rounds the double sum to
 *     binary16 once, round-to-nearest-even, subnormals kept, overflow to inf.
 *     Page 1 ("第 6 章 Shared Memory & Tile", section 6.3.3) names bf16 as the
 *     other 16-bit input type of the matrix units; the bfloat16 product is the
 *     same definition with that format's decoding and rounding.
 *
 *   Other layouts (A stored K x M, B stored K x N) are the same products of
 *   transposed operands; the Python layer transposes before calling.
 *
 * Loop order: i-k-j with a double row accumulator for the fp32 product, i-j-k
 * for the 16-bit NT product.  Rows are shared out over OpenMP threads; every output
 * is still one sequential sum, so the thread count never changes a result.
 * Build with -O2 -fopenmp -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE 754 binary16, written out from the format's definition ---------
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-24
 *   exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)
 *   exponent 31     : inf (fraction 0) or NaN                                */

double oracle_half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t oracle_half_from_double(double x) {
  if (isnan(x)) return 0x7e00;
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7c00);
  /* a = m * 2^e with m in [0.5, 1): floor(log2 a) = e - 1. */
  int e;
  frexp(a, &e);
  int E = e - 1;
  if (E < -14) E = -14;            /* below the normal range: subnormal ulp */
  const int q = E - 10;            /* the ulp of binary16 at this magnitude is 2^q */
  const double s = ldexp(a, -q);   /* exact: a power-of-two scaling */
  double r = floor(s);
  const double frac = s - r;       /* exact: s < 2^12 */
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  /* value = r * 2^q; r in [0, 2048]; renormalise when rounding carried. */
  int qq = q;
  long ri = (long)r;
  if (ri == 0) return sign;
  if (ri < 1024) {                 /* only reachable when q == -24: subnormal */
    return (uint16_t)(sign | ri);
  }
  while (ri >= 2048) { ri >>= 1; ++qq; }
  const int field = qq + 25;       /* (1024 + f) * 2^(field-25) */
  if (field >= 31) return (uint16_t)(sign | 0x7c00);
  return (uint16_t)(sign | (field << 10) | (ri - 1024));
}

void oracle_half_round_array(long n, const double* x, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = oracle_half_from_double(x[i]);
}

void oracle_half_decode_array(long n, const uint16_t* h, double* out) {
  for (long i = 0; i < n; ++i) out[i] = oracle_half_to_double(h[i]);
}

/* ---- bfloat16, written out from the format's definition --------------------
 * The upper half of an IEEE binary32: 1 sign bit, 8 exponent bits (bias 127),
 * 7 fraction bits.
 *   exponent 0      : subnormal, value = fraction * 2^-133
 *   exponent 1..254 : normal,    value = (128 + fraction) * 2^(exponent-134)
 *   exponent 255    : inf (fraction 0) or NaN                                */

double oracle_bf16_to_double(uint16_t b) {
  const int sign = (b >> 15) & 1;
  const int e = (b >> 7) & 0xff;
  const int f = b & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133);
  } else if (e == 255) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(128 + f), e - 134);
  }
  return sign ? -v : v;
}

/* Round a double to the nearest bfloat16, ties to even. */
uint16_t oracle_bf16_from_double(double x) {
  if (isnan(x)) return 0x7fc0;
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7f80);
  int e;
  frexp(a, &e);
  int E = e - 1;                   /* floor(log2 a) */
  if (E < -126) E = -126;          /* below the normal range: subnormal ulp */
  const int q = E - 7;             /* the ulp of bfloat16 at this magnitude is 2^q */
  const double s = ldexp(a, -q);   /* exact: a power-of-two scaling */
  double r = floor(s);
  const double frac = s - r;       /* exact: s < 2^9 */
  const int odd = fmod(r, 2.0) != 0.0;
  if (frac > 0.5 || (frac == 0.5 && odd)) r += 1.0;
  /* value = r * 2^q; r in [0, 256]; renormalise when rounding carried. */
  int qq = q;
  long ri = (long)r;
  if (ri == 0) return sign;
  if (ri < 128) {                  /* only reachable when q == -133: subnormal */
    return (uint16_t)(sign | ri);
  }
  while (ri >= 256) { ri >>= 1; ++qq; }
  const int field = qq + 134;      /* (128 + f) * 2^(field-134) */
  if (field >= 255) return (uint16_t)(sign | 0x7f80);
  return (uint16_t)(sign | (field << 7) | (ri - 128));
}

void oracle_bf16_round_array(long n, const double* x, uint16_t* out) {
  for (long i = 0; i < n; ++i) out[i] = oracle_bf16_from_double(x[i]);
}

void oracle_bf16_decode_array(long n, const uint16_t* b, double* out) {
  for (long i = 0; i < n; ++i) out[i] = oracle_bf16_to_double(b[i]);
}

/* The decoder of a 16-bit storage format: 0 binary16, 1 bfloat16. */
typedef double (*decode16_fn)(uint16_t);
static decode16_fn decoder16(int fmt) {
  return fmt == 1 ? oracle_bf16_to_double : oracle_half_to_double;
}

/* ---- fp32 row-major C = alpha*A*B + beta*C -------------------------------
 * Cref[i*ldr + j] = alpha * sum_k A[i*lda+k]*B[k*ldb+j]  (+ beta*Cin[i*ldc+j]
 * when beta != 0), all in double.  Cin may be NULL when beta == 0. */
void oracle_gemm_f32(int M, int N, int K, double alpha,
                     const float* A, long lda, const float* B, long ldb,
                     double beta, const float* Cin, long ldc,
                     double* Cref, long ldr) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < M; ++i) {
    double* acc = Cref + (long)i * ldr;
    for (int j = 0; j < N; ++j) acc[j] = 0.0;
    for (int k = 0; k < K; ++k) {
      const double a = (double)A[(long)i * lda + k];
      const float* brow = B + (long)k * ldb;
      for (int j = 0; j < N; ++j) acc[j] += a * (double)brow[j];
    }
    for (int j = 0; j < N; ++j) {
      double c = alpha * acc[j];
      if (beta != 0.0) c += beta * (double)Cin[(long)i * ldc + j];
      acc[j] = c;
    }
  }
}

/* The same definition, evaluated one output at a time at the given
 * (rows[t], cols[t]) coordinates.  For sampling products too large to
 * evaluate in full. */
void oracle_gemm_f32_points(int K, double alpha,
                            const float* A, long lda, const float* B, long ldb,
                            double beta, const float* Cin, long ldc,
                            long count, const int* rows, const int* cols,
                            double* out) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < count; ++t) {
    const long i = rows[t], j = cols[t];
    double acc = 0.0;
    for (int k = 0; k < K; ++k)
      acc += (double)A[i * lda + k] * (double)B[(long)k * ldb + j];
    double c = alpha * acc;
    if (beta != 0.0) c += beta * (double)Cin[i * ldc + j];
    out[t] = c;
  }
}

/* ---- 16-bit C = A * B^T ---------------------------------------------------
 * Cref[i*ldr + j] = sum_k A[i*lda+k] * B[j*ldb+k] in double (the value before
 * the final rounding).  A and B are bit patterns of format `fmt` (0 binary16,
 * 1 bfloat16). */
void oracle_gemm_16_nt(int fmt, int M, int N, int K,
                       const uint16_t* A, long lda, const uint16_t* B, long ldb,
                       double* Cref, long ldr) {
  const decode16_fn dec = decoder16(fmt);
  /* Decode B once; A is decoded one row at a time. */
  double* Bd = (double*)malloc(sizeof(double) * (size_t)N * (size_t)(K > 0 ? K : 1));
  for (long j = 0; j < N; ++j)
    for (int k = 0; k < K; ++k) Bd[j * K + k] = dec(B[j * ldb + k]);
#pragma omp parallel
  {
    double* arow = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
      for (int k = 0; k < K; ++k) arow[k] = dec(A[(long)i * lda + k]);
      for (int j = 0; j < N; ++j) {
        const double* brow = Bd + (long)j * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += arow[k] * brow[k];
        Cref[(long)i * ldr + j] = acc;
      }
    }
    free(arow);
  }
  free(Bd);
}

void oracle_gemm_16_nt_points(int fmt, int K,
                              const uint16_t* A, long lda, const uint16_t* B, long ldb,
                              long count, const int* rows, const int* cols,
                              double* out) {
  const decode16_fn dec = decoder16(fmt);
#pragma omp parallel for schedule(static)
  for (long t = 0; t < count; ++t) {
    const long i = rows[t], j = cols[t];
    double acc = 0.0;
    for (int k = 0; k < K; ++k) acc += dec(A[i * lda + k]) * dec(B[j * ldb + k]);
    out[t] = acc;
  }
}

/* ---- fused write-back of a 16-bit product ----------------------------------
 * Page 1 ("第 6 章 Shared Memory & Tile", section 6.5.4) folds the work that
 * follows a GEMM into its write-back: the column's bias is added to the
 * accumulator, the sum goes through an activation, and the residual stream
 * is added, before the one store of the output.  For output (i, j), in
 * double:
 *     v = acc + bias[j]              (bias NULL: nothing added)
 *     v = act(v)                     act 0: v;  1 (ReLU): v if v > 0 else 0;
 *                                    2 (SiLU): v / (1 + e^(-v))
 *     v = v + residual[i*ldres + j]  (residual NULL: nothing added)
 * bias and residual are bit patterns of format `fmt` (0 binary16, 1
 * bfloat16).  acc[t] is the product's sum at output (rows[t], cols[t]);
 * out[t] is the value before the output rounding. */
void oracle_epilogue16(int fmt, long count, const double* acc, const int* rows, const int* cols,
                       const uint16_t* bias, int act, const uint16_t* res, long ldres,
                       double* out) {
  const decode16_fn dec = decoder16(fmt);
#pragma omp parallel for schedule(static)
  for (long t = 0; t < count; ++t) {
    const long i = rows[t], j = cols[t];
    double v = acc[t];
    if (bias) v += dec(bias[j]);
    if (act == 1) {
      v = v > 0.0 ? v : 0.0;
    } else if (act == 2) {
      v = v / (1.0 + exp(-v));
    }
    if (res) v += dec(res[i * ldres + j]);
    out[t] = v;
  }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
