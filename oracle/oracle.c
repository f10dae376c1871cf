/*
 * Plain CPU oracle for the sharded matmul A[I,J].B[J,K] -> C[I,K].
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header or constant with the HIP library, and nothing in the HIP library
 * calls it.
 *
 * Everything is computed in IEEE double precision with naive loops. The
 * operand elements are read exactly as stored (double, float, or bfloat16
 * bit patterns) and widened losslessly to double.
 *
 * Sources (the pages this follows):
 *  - lingze.zone "Cheetsheet for the four cases of sharded matmul", the
 *    definition of the product with J contracted (top of the page), and
 *    section "Case 3": each device sums its own slice of J.
 *  - semiaifoundry.com "Sharded matrix multiplication and result ownership",
 *    section "The mechanism" (steps 2-4: disjoint slices of the contracted
 *    dimension, local partials over all output coordinates, addition of
 *    matching coordinates) and "Engineering example" (the 2x2 case).
 *  - mbrenndoerfer.com "Row Parallelism": Y = X A = sum_i X_i A_i, block
 *    form of the product.
 *  - ana-alekseeva.com "The simple maths behind parallel training", section
 *    "MLP block": GeLU between the column-split and row-split weights.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

static double bf16_bits_to_double(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double elem(const void* base, int kind, int64_t idx) {
  if (kind == ORC_F64) return ((const double*)base)[idx];
  if (kind == ORC_F32) return (double)((const float*)base)[idx];
  return bf16_bits_to_double(((const uint16_t*)base)[idx]);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Product of an I x J view of A and a J x K view of B:
 *   C[t, k] = sum over j = 0..J-1 (ascending) of A[i_t, j] * B[j, k]
 * where i_t = rows[t] when rows != NULL (a sample of output rows), else t.
 * Views are row-major with leading dimensions lda, ldb, ldc (elements).
 * Each output element accumulates its J products in ascending j.
 */
int orc_matmul(const void* A, int akind, int64_t lda,
               const void* B, int bkind, int64_t ldb,
               double* C, int64_t ldc,
               int64_t I, int64_t J, int64_t K,
               const int64_t* rows, int64_t nrows) {
  if (!A || !B || !C || I < 0 || J < 0 || K < 0) return 1;
  int64_t n_out = rows ? nrows : I;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_out; ++t) {
    int64_t i = rows ? rows[t] : t;
    double* c = C + t * ldc;
    for (int64_t k = 0; k < K; ++k) c[k] = 0.0;
    for (int64_t j = 0; j < J; ++j) {
      double a = elem(A, akind, i * lda + j);
      if (bkind == ORC_F64) {
        const double* b = (const double*)B + j * ldb;
        for (int64_t k = 0; k < K; ++k) c[k] += a * b[k];
      } else if (bkind == ORC_F32) {
        const float* b = (const float*)B + j * ldb;
        for (int64_t k = 0; k < K; ++k) c[k] += a * (double)b[k];
      } else {
        const uint16_t* b = (const uint16_t*)B + j * ldb;
        for (int64_t k = 0; k < K; ++k) c[k] += a * bf16_bits_to_double(b[k]);
      }
    }
  }
  return 0;
}

/* Single entries: out[t] = sum_j A[ri[t], j] * B[j, ci[t]], j ascending. */
int orc_entries(const void* A, int akind, int64_t lda,
                const void* B, int bkind, int64_t ldb, int64_t J,
                const int64_t* ri, const int64_t* ci, int64_t n, double* out) {
  if (!A || !B || !ri || !ci || !out || J < 0) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t) {
    double s = 0.0;
    for (int64_t j = 0; j < J; ++j)
      s += elem(A, akind, ri[t] * lda + j) * elem(B, bkind, j * ldb + ci[t]);
    out[t] = s;
  }
  return 0;
}

/* y[i] = sum_j M[i, j] * v[j] (j ascending), M an R x Cc view. */
int orc_matvec(const void* M, int kind, int64_t ld, int64_t R, int64_t Cc,
               const double* v, double* y) {
  if (!M || !v || !y) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < R; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < Cc; ++j) s += elem(M, kind, i * ld + j) * v[j];
    y[i] = s;
  }
  return 0;
}

/*
 * Sum of N partials in rank order: out[e] = (((P_0[e] + P_1[e]) + P_2[e]) ...)
 * with P_r = P + r * stride. The addition of contributions with matching
 * output coordinates (semiaifoundry.com, "The mechanism", step 4).
 */
int orc_sum_ranked(const double* P, int64_t n, int N, int64_t stride, double* out) {
  if (!P || !out || N < 1) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    double s = P[e];
    for (int r = 1; r < N; ++r) s += P[(int64_t)r * stride + e];
    out[e] = s;
  }
  return 0;
}

/*
 * GeLU, tanh form (Hendrycks & Gimpel 2016):
 *   gelu(x) = 0.5 x (1 + tanh( sqrt(2/pi) (x + 0.044715 x^3) )).
 * The pages name GeLU between the two MLP weights without defining it; the
 * tanh form is the one the workload names.
 */
double orc_gelu_tanh(double x) {
  const double c = sqrt(2.0 / 3.14159265358979323846);
  return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

int orc_gelu_tanh_array(const double* x, double* y, int64_t n) {
  if (!x || !y) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) y[e] = orc_gelu_tanh(x[e]);
  return 0;
}

/*
 * Round a double to the nearest bfloat16 value, ties to even, directly from
 * double (no intermediate float, so no double rounding). Returns the bit
 * pattern. bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction
 * bits; 8 significant bits for normals; smallest subnormal 2^-133; largest
 * finite (2 - 2^-7) * 2^127.
 */
uint16_t orc_round_bf16(double x) {
  if (isnan(x)) return (uint16_t)0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (isinf(ax)) return sign | 0x7F80;
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e);                    /* ax = m * 2^e, 0.5 <= m < 1 */
  int qexp = e - 8;                 /* spacing of 8-significant-bit numbers */
  if (qexp < -133) qexp = -133;     /* subnormal spacing floor */
  double q = ldexp(1.0, qexp);
  double r = nearbyint(ax / q) * q; /* exact scaling; nearbyint rounds ties to even */
  double maxf = ldexp(255.0, 120);  /* (2 - 2^-7) * 2^127 */
  if (r > maxf) return sign | 0x7F80;
  /* r is representable: encode it */
  float f = (float)r;               /* exact: r has <= 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | ((bits >> 16) & 0x7FFF));
}

int orc_round_bf16_array(const double* x, uint16_t* out, int64_t n) {
  if (!x || !out) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) out[e] = orc_round_bf16(x[e]);
  return 0;
}
