/*
 * Reference attention in fp64 -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the GPU path is checked against. Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the HIP library and is built
 * by the host C compiler (no fast-math, so every operation rounds as IEEE
 * double says).
 *
 * What it computes is the plain definition of scaled dot-product attention
 * ("4.4 Writing GPU Kernels with Triton", section "Kernel 4: A Simplified
 * FlashAttention": the attention of Q, K, V for one head, with the scale
 * 1/sqrt(d) by default and, for causal attention, query i seeing only the
 * keys j <= i -- the same page's test block builds exactly this reference:
 * full scores, lower-triangular mask with -inf, softmax, times V). It is
 * written as three passes per query row, the numerically stable softmax of
 * that page's section "Kernel 2: Fused Softmax" (subtract the row maximum
 * before exponentiating):
 *
 *   pass 1  s_j = scale * sum_c q_ic k_jc      for every visible key j
 *           m   = max_j s_j
 *   pass 2  e_j = exp(s_j - m),  l = sum_j e_j
 *   pass 3  O_ic = sum_j (e_j / l) v_jc,       LSE_i = m + ln l
 *
 * Keys hidden by the causal mask are left out of every sum; that is the
 * same as giving them the score -inf, because exp(-inf) = 0.
 *
 * The natural-log LSE is the quantity the same page's kernel writes for the
 * backward pass (its notes on "Base consistency: exp2 and the saved L").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of this file only. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

/* One query row: row `i` of head `bh`. q points at the head's [Nq][d]
 * queries, k and v at its [N][d] keys and values (N keys). `s` is scratch
 * of N doubles. */
static void oracle_one_row(const double *q, const double *k, const double *v,
                           int64_t N, int64_t d, int causal, double scale,
                           int64_t i, double *s, double *o_row, double *lse) {
  const int64_t n_keys = causal ? i + 1 : N; /* keys 0..n_keys-1 are visible */
  const double *qi = q + i * d;

  /* pass 1: scores and their maximum */
  double m = -INFINITY;
  for (int64_t j = 0; j < n_keys; ++j) {
    const double *kj = k + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }

  /* pass 2: exponentials relative to the maximum, and their sum */
  double l = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }

  /* pass 3: normalised weights times V, and the log-sum-exp */
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) {
    const double w = s[j] / l;
    const double *vj = v + j * d;
    for (int64_t c = 0; c < d; ++c) o_row[c] += w * vj[c];
  }
  *lse = m + log(l);
}

/*
 * attn_oracle_rows_qk -- attention for a list of query rows, with Nq query
 * rows and Nk keys per head (cross-attention when they differ; the page
 * "Programming an attention kernel in Triton", section "Kernel 4: bringing
 * it together, a self-attention kernel", validates its kernel on such
 * shapes). The
 * causal mask (query i sees keys j <= i) is defined here for Nq == Nk only.
 *
 * q        : [B][H][Nq][d] row-major fp64;  k, v : [B][H][Nk][d] (callers
 *            upcast the exact values the GPU receives).
 * rows     : flat query row ids r = (b*H + h)*Nq + i, or NULL for every row.
 * o        : [nrows][d] fp64 out;  lse : [nrows] fp64 out (natural log).
 * nthreads : OpenMP threads (<= 0: the runtime default).
 * Returns ORACLE_OK, or ORACLE_BAD_ARG for a bad size, row id or a causal
 * mask with Nq != Nk.
 */
int attn_oracle_rows_qk(const double *q, const double *k, const double *v,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        double scale, const int64_t *rows, int64_t nrows,
                        double *o, double *lse, int nthreads) {
  if (!q || !k || !v || !o || !lse) return ORACLE_BAD_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || nrows < 0) return ORACLE_BAD_ARG;
  if (causal && Nq != Nk) return ORACLE_BAD_ARG;
  const int64_t N = Nk;
  const int64_t total = B * H * Nq;
  if (!rows && nrows != total) return ORACLE_BAD_ARG;
  if (rows) {
    for (int64_t r = 0; r < nrows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return ORACLE_BAD_ARG;
  }
  int bad_alloc = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad_alloc)
#endif
  {
    double *s = (double *)malloc((size_t)N * sizeof(double));
    if (!s) {
      bad_alloc = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
      for (int64_t r = 0; r < nrows; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t bh = flat / Nq, i = flat % Nq;
        const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;
        const size_t head = (size_t)bh * (size_t)N * (size_t)d;
        oracle_one_row(q + qhead, k + head, v + head, N, d, causal, scale, i, s,
                       o + r * d, lse + r);
      }
      free(s);
    }
  }
  (void)nthreads;
  return bad_alloc ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* attn_oracle_rows -- the same with Nq = Nk = N (self-attention). */
int attn_oracle_rows(const double *q, const double *k, const double *v,
                     int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                     double scale, const int64_t *rows, int64_t nrows,
                     double *o, double *lse, int nthreads) {
  return attn_oracle_rows_qk(q, k, v, B, H, N, N, d, causal, scale, rows, nrows, o, lse,
                             nthreads);
}

/* Threads an OpenMP region of this library would use by default. */
int attn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
