/*
 * fp64 CPU oracle for the GEMM and the RecSys linear-compression layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and never calls it.
 *
 * Inputs are bf16 bit patterns (uint16), or for the _fmt GEMM entry points
 * IEEE binary16 (fp16) patterns.  Each value is widened exactly (bf16: bits
 * << 16 is the fp32 pattern; fp16: decoded from its sign, exponent and
 * fraction fields), every product of two such values is exact in fp64 (at
 * most 11 + 11 significant bits), and each output is one sum taken in
 * ascending index order.  S (optional) is the matching
 * sum of |products|, which sets the acceptance bound.
 *
 * Pages: "Triton 3.7 permite extender el compilador de GPU sin forks"
 * (the persistent and pipelined GEMM listings compute C = A.B over strided
 * operands a_ptr/b_ptr with strides stride_am, stride_ak, stride_bk,
 * stride_bn); "Meta accelere un noyau GPU d'un facteur 4 avec TLX" (section
 * on what a four-fold speed-up means: the linear-compression kernel and its
 * repeated per-buyer features).
 */
#ifndef RLL_ORACLE_H
#define RLL_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_BF16 0
#define ORACLE_F16 2 /* IEEE binary16 */

void oracle_set_threads(int n);

/* out[i] = exact fp64 value of the fmt-format pattern in[i]. */
void oracle_widen(int fmt, int64_t n, const uint16_t* in, double* out);
int oracle_get_threads(void);

/* Rows [row0, row0 + nrows) of C = A.B into C[nrows][N] (row-major, fp64),
 * A[i][k] = A[i*sam + k*sak], B[k][j] = B[k*sbk + j*sbn].  S may be NULL. */
void oracle_gemm_rows(int64_t M, int64_t N, int64_t K,
                      const uint16_t* A, int64_t sam, int64_t sak,
                      const uint16_t* B, int64_t sbk, int64_t sbn,
                      int64_t row0, int64_t nrows, double* C, double* S);

/* The same with A and B in format fmt (ORACLE_BF16 or ORACLE_F16). */
void oracle_gemm_rows_fmt(int fmt, int64_t M, int64_t N, int64_t K,
                          const uint16_t* A, int64_t sam, int64_t sak,
                          const uint16_t* B, int64_t sbk, int64_t sbn,
                          int64_t row0, int64_t nrows, double* C, double* S);
void oracle_gemm_entries_fmt(int fmt, int64_t M, int64_t N, int64_t K,
                             const uint16_t* A, int64_t sam, int64_t sak,
                             const uint16_t* B, int64_t sbk, int64_t sbn,
                             int64_t n, const int64_t* rows, const int64_t* cols,
                             double* out, double* S);

/* GEMM epilogue, in place on C[rows][N] (fp64): x = C + bias[j] (bias may be
 * NULL), then the activation act (ORACLE_ACT_*), in fp64.  S (may be NULL)
 * gains |bias[j]|.  Page "Meta accelere un noyau GPU d'un facteur 4 avec
 * TLX", section on where to start (fuse steps, measure again). */
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_GELU 2
#define ORACLE_ACT_SILU 3
void oracle_epilogue(int act, int64_t rows, int64_t N, double* C, double* S, const float* bias);

/* n single entries (rows[e], cols[e]) of C = A.B.  S may be NULL. */
void oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, int64_t sam, int64_t sak,
                         const uint16_t* B, int64_t sbk, int64_t sbn,
                         int64_t n, const int64_t* rows, const int64_t* cols,
                         double* out, double* S);

/* Linear compression, per candidate as stated: X = [user[r]; item[r][c]]
 * ((Nu+Ni) x D), Y = W^T . X (Mo x D).  user[r][n][d] = user[r*su_r + n*su_n + d],
 * item[r][c][n][d] = item[r*si_r + c*si_c + n*si_n + d], W[n][m] = W[n*sw_n + m].
 * Computes npairs candidates (rr[p], cc[p]) into Y[p][Mo][D]; S may be NULL. */
void oracle_lincomp_naive(int64_t R, int64_t C, int64_t Nu, int64_t Ni, int64_t D, int64_t Mo,
                          const uint16_t* user, int64_t su_r, int64_t su_n,
                          const uint16_t* item, int64_t si_r, int64_t si_c, int64_t si_n,
                          const uint16_t* W, int64_t sw_n,
                          int64_t npairs, const int64_t* rr, const int64_t* cc,
                          double* Y, double* S);

/* The deduplicated rewrite, used only to check that it leaves results
 * unchanged: U[r] = W[0:Nu]^T . user[r] once, V = W[Nu:]^T . item[r][c],
 * Y = U[r] + V.  Same arguments as oracle_lincomp_naive (no S). */
void oracle_lincomp_dedup(int64_t R, int64_t C, int64_t Nu, int64_t Ni, int64_t D, int64_t Mo,
                          const uint16_t* user, int64_t su_r, int64_t su_n,
                          const uint16_t* item, int64_t si_r, int64_t si_c, int64_t si_n,
                          const uint16_t* W, int64_t sw_n,
                          int64_t npairs, const int64_t* rr, const int64_t* cc,
                          double* Y);

#ifdef __cplusplus
}
#endif
#endif
