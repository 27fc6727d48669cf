/*
 * Reference attention backward in fp64 -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the GPU backward is checked against. Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the HIP library (nor with the
 * forward oracle) and is built by the host C compiler without fast-math.
 *
 * What it computes: the gradients of attention O = softmax(scale Q K^T [+
 * causal mask]) V with respect to Q, K and V, given the upstream gradient dO,
 * written out from the definitions that "4.4 Writing GPU Kernels with
 * Triton", section "Kernel 5: FlashAttention Backward", recalls:
 *
 *   P_ij  = exp(s_ij - m_i) / l_i            (the softmax of row i; s_ij =
 *                                             scale q_i . k_j over the visible
 *                                             keys j, m_i their maximum,
 *                                             l_i = sum_j exp(s_ij - m_i))
 *   O_i   = sum_j P_ij v_j
 *   dV_j  = sum_i P_ij dO_i                  (dV = P^T dO)
 *   dP_ij = dO_i . v_j                       (dP = dO V^T)
 *   D_i   = dO_i . O_i                       (rowsum(dO * O), the page's
 *                                             "Preprocessing" section)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j            (dQ = dS K, scaled)
 *   dK_j  = scale sum_i dS_ij q_i            (dK = dS^T Q, scaled)
 *
 * The page writes the scale as 1/sqrt(d), its default; here it is the scale
 * the forward used. With a causal mask, query i sees the keys j <= i; hidden
 * pairs are left out of every sum (the same as P_ij = 0).
 *
 * dQ_i needs only row i. dK_j and dV_j need every row that sees key j, so
 * for them the row statistics m_i, l_i and D_i of the whole head are found
 * first (three passes per row, as in the forward's stable softmax).
 *
 * A head has Nq query rows and Nk keys; they differ for cross-attention
 * (which "Programming an attention kernel in Triton", section "Kernel 4:
 * bringing it together, a self-attention kernel", tests its kernel on),
 * where the causal mask is not defined.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

static double dot(const double *a, const double *b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Row statistics of query i of one head (N keys): m_i, l_i, and
 * D_i = dO_i . O_i with O_i formed here. `s` and `o_row` are scratch (N and
 * d doubles). */
static void row_stats(const double *q, const double *k, const double *v, const double *dout,
                      int64_t N, int64_t d, int causal, double scale, int64_t i, double *s,
                      double *o_row, double *m_out, double *l_out, double *D_out) {
  const int64_t n_keys = causal ? i + 1 : N;
  double m = -INFINITY;
  for (int64_t j = 0; j < n_keys; ++j) {
    s[j] = scale * dot(q + i * d, k + j * d, d);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) l += exp(s[j] - m);
  for (int64_t c = 0; c < d; ++c) o_row[c] = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) {
    const double p = exp(s[j] - m) / l;
    for (int64_t c = 0; c < d; ++c) o_row[c] += p * v[j * d + c];
  }
  *m_out = m;
  *l_out = l;
  *D_out = dot(dout + i * d, o_row, d);
}

/* dQ_i of one head (N keys). */
static void dq_row(const double *q, const double *k, const double *v, const double *dout,
                   int64_t N, int64_t d, int causal, double scale, int64_t i, double *s,
                   double *o_row, double *dq) {
  double m, l, D;
  row_stats(q, k, v, dout, N, d, causal, scale, i, s, o_row, &m, &l, &D);
  const int64_t n_keys = causal ? i + 1 : N;
  for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
  for (int64_t j = 0; j < n_keys; ++j) {
    const double p = exp(scale * dot(q + i * d, k + j * d, d) - m) / l;
    const double dp = dot(dout + i * d, v + j * d, d);
    const double ds = p * (dp - D);
    for (int64_t c = 0; c < d; ++c) dq[c] += ds * k[j * d + c];
  }
  for (int64_t c = 0; c < d; ++c) dq[c] *= scale;
}

/* dK_j and dV_j of one head (N query rows) from the head's row statistics. */
static void dkdv_row(const double *q, const double *k, const double *v, const double *dout,
                     int64_t N, int64_t d, int causal, double scale, int64_t j,
                     const double *m, const double *l, const double *D, double *dk,
                     double *dv) {
  for (int64_t c = 0; c < d; ++c) dk[c] = dv[c] = 0.0;
  const int64_t i0 = causal ? j : 0; /* the rows that see key j */
  for (int64_t i = i0; i < N; ++i) {
    const double p = exp(scale * dot(q + i * d, k + j * d, d) - m[i]) / l[i];
    const double dp = dot(dout + i * d, v + j * d, d);
    const double ds = p * (dp - D[i]);
    for (int64_t c = 0; c < d; ++c) {
      dv[c] += p * dout[i * d + c];
      dk[c] += ds * q[i * d + c];
    }
  }
  for (int64_t c = 0; c < d; ++c) dk[c] *= scale;
}

/*
 * attn_bwd_oracle_rows_qk -- gradients for lists of query and key rows, Nq
 * query rows and Nk keys per head.
 *
 * q, dout : [B][H][Nq][d] and k, v : [B][H][Nk][d], row-major fp64 (callers
 *           upcast the exact values the GPU receives).
 * qrows / nq : flat query row ids (b*H + h)*Nq + i whose dQ is wanted, or
 *              NULL with nq = B*H*Nq for all of them in order.
 * krows / nk : flat key row ids (b*H + h)*Nk + j whose dK and dV are wanted,
 *              or NULL with nk = B*H*Nk for all.
 * dq : [nq][d] out;  dk, dv : [nk][d] out.
 * nthreads : OpenMP threads (<= 0: the runtime default).
 * Returns ORACLE_OK, ORACLE_BAD_ARG (also for a causal mask with Nq != Nk)
 * or ORACLE_NO_MEMORY.
 */
int attn_bwd_oracle_rows_qk(const double *q, const double *k, const double *v,
                            const double *dout, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                            int64_t d, int causal, double scale, const int64_t *qrows, int64_t nq,
                            double *dq, const int64_t *krows, int64_t nk, double *dk, double *dv,
                            int nthreads) {
  if (!q || !k || !v || !dout) return ORACLE_BAD_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || nq < 0 || nk < 0) return ORACLE_BAD_ARG;
  if (causal && Nq != Nk) return ORACLE_BAD_ARG;
  if ((nq > 0 && !dq) || (nk > 0 && (!dk || !dv))) return ORACLE_BAD_ARG;
  const int64_t BH = B * H, total = BH * Nq, ktotal = BH * Nk;
  if ((!qrows && nq != 0 && nq != total) || (!krows && nk != 0 && nk != ktotal))
    return ORACLE_BAD_ARG;
  for (int64_t r = 0; qrows && r < nq; ++r)
    if (qrows[r] < 0 || qrows[r] >= total) return ORACLE_BAD_ARG;
  for (int64_t r = 0; krows && r < nk; ++r)
    if (krows[r] < 0 || krows[r] >= ktotal) return ORACLE_BAD_ARG;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#endif
  int bad = 0;

  /* dQ: independent rows. */
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
  {
    double *s = (double *)malloc((size_t)(Nk + d) * sizeof(double));
    if (!s) {
      bad = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
      for (int64_t r = 0; r < nq; ++r) {
        const int64_t flat = qrows ? qrows[r] : r;
        const int64_t bh = flat / Nq, i = flat % Nq;
        const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;
        const size_t khead = (size_t)bh * (size_t)Nk * (size_t)d;
        dq_row(q + qhead, k + khead, v + khead, dout + qhead, Nk, d, causal, scale, i, s, s + Nk,
               dq + r * d);
      }
      free(s);
    }
  }
  if (bad) return ORACLE_NO_MEMORY;
  if (nk == 0) return ORACLE_OK;

  /* dK, dV: row statistics of every head that a requested key belongs to. */
  char *need = (char *)calloc((size_t)BH, 1);
  double *m = (double *)malloc((size_t)total * sizeof(double));
  double *l = (double *)malloc((size_t)total * sizeof(double));
  double *D = (double *)malloc((size_t)total * sizeof(double));
  if (!need || !m || !l || !D) {
    free(need), free(m), free(l), free(D);
    return ORACLE_NO_MEMORY;
  }
  for (int64_t r = 0; r < nk; ++r) need[(krows ? krows[r] : r) / Nk] = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
  {
    double *s = (double *)malloc((size_t)(Nk + d) * sizeof(double));
    if (!s) {
      bad = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
      for (int64_t flat = 0; flat < total; ++flat) {
        const int64_t bh = flat / Nq, i = flat % Nq;
        if (!need[bh]) continue;
        const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;
        const size_t khead = (size_t)bh * (size_t)Nk * (size_t)d;
        row_stats(q + qhead, k + khead, v + khead, dout + qhead, Nk, d, causal, scale, i, s,
                  s + Nk, m + flat, l + flat, D + flat);
      }
      free(s);
    }
  }
  if (!bad) {
#ifdef _OPENMP
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 8)
#endif
    for (int64_t r = 0; r < nk; ++r) {
      const int64_t flat = krows ? krows[r] : r;
      const int64_t bh = flat / Nk, j = flat % Nk;
      const size_t qhead = (size_t)bh * (size_t)Nq * (size_t)d;
      const size_t khead = (size_t)bh * (size_t)Nk * (size_t)d;
      const size_t rows = (size_t)bh * (size_t)Nq;
      dkdv_row(q + qhead, k + khead, v + khead, dout + qhead, Nq, d, causal, scale, j, m + rows,
               l + rows, D + rows, dk + r * d, dv + r * d);
    }
  }
  free(need), free(m), free(l), free(D);
  (void)nthreads;
  return bad ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* attn_bwd_oracle_rows -- the same with Nq = Nk = N (self-attention). */
int attn_bwd_oracle_rows(const double *q, const double *k, const double *v, const double *dout,
                         int64_t B, int64_t H, int64_t N, int64_t d, int causal, double scale,
                         const int64_t *qrows, int64_t nq, double *dq, const int64_t *krows,
                         int64_t nk, double *dk, double *dv, int nthreads) {
  return attn_bwd_oracle_rows_qk(q, k, v, dout, B, H, N, N, d, causal, scale, qrows, nq, dq, krows,
                                 nk, dk, dv, nthreads);
}
