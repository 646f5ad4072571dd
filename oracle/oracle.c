/*
 * fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark
 * CPU baseline).  Plain loops; no blocking, no reordering of any sum.
 * See oracle.h for the definitions and the pages they follow.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 -> fp64, exact: the bf16 pattern is the upper half of an fp32 pattern. */
static double widen(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE 754 binary16 -> fp64, exact, from the format's definition: sign bit,
 * 5-bit exponent e (bias 15), 10-bit fraction m.  e = 0: m * 2^-24
 * (subnormal or zero); 0 < e < 31: (1024 + m) * 2^(e - 25); e = 31: infinity
 * (m = 0) or NaN. */
static double widen_f16(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* Element decoding by format: ORACLE_BF16 or ORACLE_F16. */
static double widen_fmt(int fmt, uint16_t h) { return fmt == ORACLE_F16 ? widen_f16(h) : widen(h); }

void oracle_widen(int fmt, int64_t n, const uint16_t* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen_fmt(fmt, in[i]);
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j], k ascending.  The k loop sits
 * outside the j loop so that B is read along its rows; each C[i][j] still
 * receives its terms one by one in ascending k, exactly as the definition. */
void oracle_gemm_rows_fmt(int fmt, int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t sam, int64_t sak,
                          const uint16_t* B, int64_t sbk, int64_t sbn,
                          int64_t row0, int64_t nrows, double* C, double* S) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = row0 + r;
    double* c = C + r * N;
    double* s = S ? S + r * N : NULL;
    for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
    if (s)
      for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = widen_fmt(fmt, A[i * sam + k * sak]);
      const uint16_t* brow = B + k * sbk;
      for (int64_t j = 0; j < N; ++j) {
        const double p = a * widen_fmt(fmt, brow[j * sbn]);
        c[j] += p;
        if (s) s[j] += fabs(p);
      }
    }
  }
}

void oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t sam, int64_t sak,
                      const uint16_t* B, int64_t sbk, int64_t sbn,
                      int64_t row0, int64_t nrows, double* C, double* S) {
  oracle_gemm_rows_fmt(ORACLE_BF16, M, N, K, A, sam, sak, B, sbk, sbn, row0, nrows, C, S);
}

void oracle_gemm_entries_fmt(int fmt, int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t sam, int64_t sak,
                             const uint16_t* B, int64_t sbk, int64_t sbn,
                             int64_t n, const int64_t* rows, const int64_t* cols,
                             double* out, double* S) {
  (void)M;
  (void)N;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t e = 0; e < n; ++e) {
    const int64_t i = rows[e], j = cols[e];
    double c = 0.0, s = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = widen_fmt(fmt, A[i * sam + k * sak]) * widen_fmt(fmt, B[k * sbk + j * sbn]);
      c += p;
      s += fabs(p);
    }
    out[e] = c;
    if (S) S[e] = s;
  }
}

void oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, int64_t sam, int64_t sak,
                         const uint16_t* B, int64_t sbk, int64_t sbn,
                         int64_t n, const int64_t* rows, const int64_t* cols,
                         double* out, double* S) {
  oracle_gemm_entries_fmt(ORACLE_BF16, M, N, K, A, sam, sak, B, sbk, sbn, n, rows, cols, out, S);
}

/* Per candidate, as the layer is stated: build the candidate's full input X by
 * stacking the request's user rows above the candidate's item rows, then
 * Y[m][d] = sum_{n=0}^{Nu+Ni-1} W[n][m] * X[n][d] in ascending n. */
void oracle_lincomp_naive(int64_t R, int64_t C, int64_t Nu, int64_t Ni, int64_t D, int64_t Mo,
                          const uint16_t* user, int64_t su_r, int64_t su_n,
                          const uint16_t* item, int64_t si_r, int64_t si_c, int64_t si_n,
                          const uint16_t* W, int64_t sw_n,
                          int64_t npairs, const int64_t* rr, const int64_t* cc,
                          double* Y, double* S) {
  (void)R;
  (void)C;
  const int64_t Nin = Nu + Ni;
#pragma omp parallel
  {
    double* X = (double*)malloc(sizeof(double) * (size_t)(Nin * D));
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
      const int64_t r = rr[p], c = cc[p];
      for (int64_t n = 0; n < Nu; ++n)
        for (int64_t d = 0; d < D; ++d) X[n * D + d] = widen(user[r * su_r + n * su_n + d]);
      for (int64_t n = 0; n < Ni; ++n)
        for (int64_t d = 0; d < D; ++d)
          X[(Nu + n) * D + d] = widen(item[r * si_r + c * si_c + n * si_n + d]);
      double* y = Y + p * Mo * D;
      double* s = S ? S + p * Mo * D : NULL;
      for (int64_t m = 0; m < Mo; ++m) {
        double* yr = y + m * D;
        double* sr = s ? s + m * D : NULL;
        for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;
        if (sr)
          for (int64_t d = 0; d < D; ++d) sr[d] = 0.0;
        for (int64_t n = 0; n < Nin; ++n) {
          const double w = widen(W[n * sw_n + m]);
          const double* xr = X + n * D;
          for (int64_t d = 0; d < D; ++d) {
            const double t = w * xr[d];
            yr[d] += t;
            if (sr) sr[d] += fabs(t);
          }
        }
      }
    }
    free(X);
  }
}

/* The rewrite that handles the request-shared user rows once: U = W_u^T . user[r]
 * and V = W_i^T . item[r][c] are separate sums; Y = U + V. */
void oracle_lincomp_dedup(int64_t R, int64_t C, int64_t Nu, int64_t Ni, int64_t D, int64_t Mo,
                          const uint16_t* user, int64_t su_r, int64_t su_n,
                          const uint16_t* item, int64_t si_r, int64_t si_c, int64_t si_n,
                          const uint16_t* W, int64_t sw_n,
                          int64_t npairs, const int64_t* rr, const int64_t* cc,
                          double* Y) {
  (void)R;
  (void)C;
#pragma omp parallel
  {
    double* U = (double*)malloc(sizeof(double) * (size_t)(Mo * D));
    double* V = (double*)malloc(sizeof(double) * (size_t)(Mo * D));
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
      const int64_t r = rr[p], c = cc[p];
      for (int64_t m = 0; m < Mo; ++m) {
        for (int64_t d = 0; d < D; ++d) U[m * D + d] = 0.0, V[m * D + d] = 0.0;
        for (int64_t n = 0; n < Nu; ++n) {
          const double w = widen(W[n * sw_n + m]);
          for (int64_t d = 0; d < D; ++d) U[m * D + d] += w * widen(user[r * su_r + n * su_n + d]);
        }
        for (int64_t n = 0; n < Ni; ++n) {
          const double w = widen(W[(Nu + n) * sw_n + m]);
          for (int64_t d = 0; d < D; ++d)
            V[m * D + d] += w * widen(item[r * si_r + c * si_c + n * si_n + d]);
        }
      }
      double* y = Y + p * Mo * D;
      for (int64_t e = 0; e < Mo * D; ++e) y[e] = U[e] + V[e];
    }
    free(U);
    free(V);
  }
}

/* GEMM epilogue on n values of one row of C, in place, as stated: x = c +
 * bias[j]; then ReLU max(x, 0), GELU x * Phi(x) = x/2 (1 + erf(x / sqrt 2)),
 * or SiLU x / (1 + exp(-x)), all in fp64.  S[j] (the bound's sum of
 * |terms|) gains |bias[j]|: the bias is one more term of the sum.  GELU is
 * evaluated as x/2 erfc(-x / sqrt 2), the same value, so that large
 * negative x keeps its relative accuracy. */
void oracle_epilogue(int act, int64_t rows, int64_t N, double* C, double* S, const float* bias) {
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < N; ++j) {
      const double b = bias ? (double)bias[j] : 0.0;
      const double x = C[i * N + j] + b;
      double y = x;
      if (act == ORACLE_ACT_RELU)
        y = x > 0.0 ? x : 0.0;
      else if (act == ORACLE_ACT_GELU)
        y = 0.5 * x * erfc(-x / sqrt(2.0)); /* = x/2 (1 + erf(x / sqrt 2)), without cancellation for x < 0 */
      else if (act == ORACLE_ACT_SILU)
        y = x / (1.0 + exp(-x));
      C[i * N + j] = y;
      if (S) S[i * N + j] += fabs(b);
    }
}
