/*
 * attn_oracle.c -- fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file, and everything else under oracle/,
 * is the checker that the GPU path is compared against.  Only the tests,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * HIP library never calls it.
 *
 * What it computes follows the page "GPU 内核与 FlashAttention" (hs-black,
 * scaling-gpu-kernels), section 10 (standard attention: S = Q K^T, P = softmax(S),
 * O = P V, with the usual 1/sqrt(d) factor on S) and section 11.1 (safe
 * softmax: subtract the row maximum before exponentiating), and the
 * log-sum-exp side output L = m + log(l) of sections 13.2 and 14.1.  The
 * logit scale is an argument (the configurations use 1/sqrt(d)).  The page
 * "Flash Attention实现深度解析" (maplevalley), section 3.1, fixes the packed
 * variable-length layout [total, heads, d] with prefix offsets and an
 * LSE of shape [batch, heads, max_seqlen].
 *
 * Everything is plain fp64: the caller decodes the 16-bit inputs exactly
 * into double arrays.  Rows are independent; OpenMP spreads them over the
 * host cores.  No blocking, fusion or reordering beyond the definition:
 * for every query row the scores are formed, their maximum taken, the
 * shifted exponentials summed, and the output is the normalised weighted
 * sum of value rows.
 *
 * Two options of the same page, section 14:
 *  - causal (section 14.4): the score of key j for query i is -infinity when
 *    j > i, indices counted from the start of the sequence (for Nq != Nk this
 *    is the literal j > i, top-left aligned); exp(-inf) = 0, so row i is the
 *    softmax over keys 0..i.  Key 0 is visible to every row, so m is finite.
 *  - grouped K/V heads (section 14.2, MQA/GQA): k and v have heads_kv heads,
 *    heads_kv divides heads, and query head h reads K/V head
 *    h / (heads / heads_kv); nothing is copied.
 *
 * oracle_attention_bwd() is the backward pass of the same page, section 13.1:
 * with dO given and the scores s_ij = scale <q_i, k_j> (masked as above),
 *   P = softmax rows, dV = P^T dO, dP_ij = <do_i, v_j>, D_i = sum_j P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - D_i), dQ = scale dS K, dK = scale dS^T Q
 * (the factor scale because the page's S = Q K^T carries no scale here).  D_i is
 * taken from its definition P_i: . dP_i:, not from the page's simplification
 * <do_i, o_i> that the GPU path uses.  With grouped K/V heads the dK and dV of
 * a K/V head sum the contributions of every query head that reads it.
 *
 * oracle_attention_online() is the second function: the one-pass blockwise
 * recurrence of section 11.2 (two-block merge of (m, l)) and section 11.3
 * (running unnormalised output rescaled by exp(m - m'), divided by l at the
 * end), also in fp64.  It exists so that tests can show the recurrence the
 * GPU kernel relies on reaches the same result as the definition; with the
 * causal option it also skips every key block lying wholly above the
 * diagonal and masks inside the others (section 14.4), which must still
 * give the definition's result.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Address of element [row, head, t] in a [rows, heads, d] (dense: [batch*n, heads, d]) array. */
static inline int64_t at(int64_t row, int64_t head, int64_t t, int64_t heads, int64_t d) {
  return (row * heads + head) * d + t;
}

/* One query row of the definition.  qrow0/krow0 are the first token rows of
 * this sequence in the q and k/v arrays; i the query index in the sequence;
 * h the query head and hk the K/V head it reads. */
static void one_row(const double *q, const double *k, const double *v, double *o_row,
                    double *lse_out, int64_t qrow0, int64_t krow0, int64_t i, int64_t nk,
                    int64_t h, int64_t hk, int64_t heads, int64_t heads_kv, int64_t d,
                    double scale, int causal, double *s) {
  /* s_j = scale * <q_i, k_j>; -inf above the diagonal when causal */
  for (int64_t j = 0; j < nk; ++j) {
    double acc = 0.0;
    for (int64_t t = 0; t < d; ++t)
      acc += q[at(qrow0 + i, h, t, heads, d)] * k[at(krow0 + j, hk, t, heads_kv, d)];
    s[j] = scale * acc;
    if (causal && j > i) s[j] = -INFINITY;
  }
  /* m = max_j s_j */
  double m = -INFINITY;
  for (int64_t j = 0; j < nk; ++j) if (s[j] > m) m = s[j];
  /* l = sum_j exp(s_j - m) */
  double l = 0.0;
  for (int64_t j = 0; j < nk; ++j) l += exp(s[j] - m);
  /* O_i = sum_j (exp(s_j - m) / l) v_j */
  for (int64_t t = 0; t < d; ++t) o_row[t] = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    double p = exp(s[j] - m) / l;
    for (int64_t t = 0; t < d; ++t) o_row[t] += p * v[at(krow0 + j, hk, t, heads_kv, d)];
  }
  *lse_out = m + log(l);
}

/*
 * Full attention.
 *  q, o:   dense [batch, nq, heads, d]; varlen (cu != NULL) packed [cu[batch], heads, d]
 *  k, v:   dense [batch, nk, heads_kv, d]; varlen packed [cu[batch], heads_kv, d]
 *  lse:    [batch, heads, nq]  (varlen: nq is the row pitch, i.e. max length; rows past a
 *          sequence's length are left untouched)
 *  cu:     NULL for dense, else batch+1 non-decreasing prefix offsets shared by q and k.
 *  causal: nonzero masks key j > query i (per sequence).
 * Returns 0, -1 if scratch memory could not be obtained, -2 if heads_kv does not divide heads.
 */
int oracle_attention(const double *q, const double *k, const double *v, double *o, double *lse,
                     int64_t batch, int64_t nq, int64_t nk, int64_t heads, int64_t heads_kv,
                     int64_t d, double scale, int causal, const int64_t *cu) {
  if (heads_kv <= 0 || heads % heads_kv != 0) return -2;
  const int64_t group = heads / heads_kv;
  int64_t max_nk = nk;
  if (cu) {
    max_nk = 0;
    for (int64_t b = 0; b < batch; ++b) if (cu[b + 1] - cu[b] > max_nk) max_nk = cu[b + 1] - cu[b];
  }
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for collapse(3) schedule(dynamic, 4)
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < nq; ++i) {
          if (!s) continue;
          int64_t lq = cu ? cu[b + 1] - cu[b] : nq;
          int64_t lk = cu ? cu[b + 1] - cu[b] : nk;
          if (i >= lq || lk <= 0) continue;
          int64_t qrow0 = cu ? cu[b] : b * nq;
          int64_t krow0 = cu ? cu[b] : b * nk;
          one_row(q, k, v, o + at(qrow0 + i, h, 0, heads, d), lse + (b * heads + h) * nq + i,
                  qrow0, krow0, i, lk, h, h / group, heads, heads_kv, d, scale, causal, s);
        }
    free(s);
  }
  return failed ? -1 : 0;
}

/*
 * Selected rows only (for sampled checks at full size).  rows is n_rows triples
 * (b, h, i); o_rows is [n_rows, d], lse_rows [n_rows].  Layout and cu as above.
 */
int oracle_attention_rows(const double *q, const double *k, const double *v, double *o_rows,
                          double *lse_rows, int64_t batch, int64_t nq, int64_t nk, int64_t heads,
                          int64_t heads_kv, int64_t d, double scale, int causal,
                          const int64_t *cu, const int64_t *rows, int64_t n_rows) {
  if (heads_kv <= 0 || heads % heads_kv != 0) return -2;
  const int64_t group = heads / heads_kv;
  int64_t max_nk = nk;
  if (cu) {
    max_nk = 0;
    for (int64_t b = 0; b < batch; ++b) if (cu[b + 1] - cu[b] > max_nk) max_nk = cu[b + 1] - cu[b];
  }
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    if (!s) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!s) continue;
      int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      int64_t lk = cu ? cu[b + 1] - cu[b] : nk;
      int64_t qrow0 = cu ? cu[b] : b * nq;
      int64_t krow0 = cu ? cu[b] : b * nk;
      one_row(q, k, v, o_rows + r * d, lse_rows + r, qrow0, krow0, i, lk, h, h / group, heads,
              heads_kv, d, scale, causal, s);
    }
    free(s);
  }
  return failed ? -1 : 0;
}

/*
 * The blockwise one-pass recurrence (dense layout, heads_kv = heads), block = key-block
 * size.  State per query row: running max m (starts at -inf), running denominator l
 * (starts at 0) and unnormalised output ot (starts at 0).  For each key block:
 * m' = max(m, max of the block's scores); l <- exp(m - m') l + sum exp(s - m');
 * ot <- exp(m - m') ot + sum exp(s - m') v; m <- m'.  At the end O = ot / l and
 * LSE = m + log l.  exp(m - m') with m = -inf is taken as 0 (nothing accumulated yet).
 * Causal: a block whose first key is past i is skipped whole; inside the others a key
 * past i scores -inf.
 */
int oracle_attention_online(const double *q, const double *k, const double *v, double *o,
                            double *lse, int64_t batch, int64_t nq, int64_t nk, int64_t heads,
                            int64_t d, double scale, int causal, int64_t block) {
  if (block <= 0) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)block);
    double *ot = (double *)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
    if (!s || !ot) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for collapse(3) schedule(dynamic, 4)
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t h = 0; h < heads; ++h)
        for (int64_t i = 0; i < nq; ++i) {
          if (!s || !ot) continue;
          double m = -INFINITY, l = 0.0;
          for (int64_t t = 0; t < d; ++t) ot[t] = 0.0;
          for (int64_t j0 = 0; j0 < nk; j0 += block) {
            if (causal && j0 > i) break; /* this block and every later one lie above the diagonal */
            int64_t nb = nk - j0 < block ? nk - j0 : block;
            double mb = -INFINITY;
            for (int64_t jj = 0; jj < nb; ++jj) {
              double acc = 0.0;
              for (int64_t t = 0; t < d; ++t)
                acc += q[at(b * nq + i, h, t, heads, d)] * k[at(b * nk + j0 + jj, h, t, heads, d)];
              s[jj] = scale * acc;
              if (causal && j0 + jj > i) s[jj] = -INFINITY;
              if (s[jj] > mb) mb = s[jj];
            }
            double mn = m > mb ? m : mb;
            double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
            l *= alpha;
            for (int64_t t = 0; t < d; ++t) ot[t] *= alpha;
            for (int64_t jj = 0; jj < nb; ++jj) {
              double p = exp(s[jj] - mn);
              l += p;
              for (int64_t t = 0; t < d; ++t) ot[t] += p * v[at(b * nk + j0 + jj, h, t, heads, d)];
            }
            m = mn;
          }
          for (int64_t t = 0; t < d; ++t) o[at(b * nq + i, h, t, heads, d)] = ot[t] / l;
          lse[(b * heads + h) * nq + i] = m + log(l);
        }
    free(s);
    free(ot);
  }
  return failed ? -1 : 0;
}

/*
 * Backward pass (page "GPU 内核与 FlashAttention", section 13.1).  Layouts as in
 * oracle_attention: q, dout, dq [rows, heads, d]; k, v, dk, dv [rows, heads_kv, d]; dense rows
 * = batch * n, packed rows = cu[batch].  dq, dk and dv are overwritten.  One OpenMP task per
 * (sequence, K/V head) owns that head's dk and dv rows, so nothing is shared between threads.
 * Returns 0, -1 if scratch memory could not be obtained, -2 if heads_kv does not divide heads.
 */
int oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dout,
                         double *dq, double *dk, double *dv, int64_t batch, int64_t nq, int64_t nk,
                         int64_t heads, int64_t heads_kv, int64_t d, double scale, int causal,
                         const int64_t *cu) {
  if (heads_kv <= 0 || heads % heads_kv != 0) return -2;
  const int64_t group = heads / heads_kv;
  int64_t max_nk = nk;
  if (cu) {
    max_nk = 0;
    for (int64_t b = 0; b < batch; ++b) if (cu[b + 1] - cu[b] > max_nk) max_nk = cu[b + 1] - cu[b];
  }
  int failed = 0;
#pragma omp parallel
  {
    /* per thread: the scores / probabilities of one row and its dP, then dS */
    double *p = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    if (!p || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t hk = 0; hk < heads_kv; ++hk) {
        if (!p || !dp) continue;
        int64_t lq = cu ? cu[b + 1] - cu[b] : nq;
        int64_t lk = cu ? cu[b + 1] - cu[b] : nk;
        int64_t qrow0 = cu ? cu[b] : b * nq;
        int64_t krow0 = cu ? cu[b] : b * nk;
        for (int64_t j = 0; j < lk; ++j)
          for (int64_t t = 0; t < d; ++t) {
            dk[at(krow0 + j, hk, t, heads_kv, d)] = 0.0;
            dv[at(krow0 + j, hk, t, heads_kv, d)] = 0.0;
          }
        for (int64_t h = hk * group; h < (hk + 1) * group; ++h)
          for (int64_t i = 0; i < lq; ++i) {
            const double *qi = q + at(qrow0 + i, h, 0, heads, d);
            const double *doi = dout + at(qrow0 + i, h, 0, heads, d);
            double *dqi = dq + at(qrow0 + i, h, 0, heads, d);
            /* P_i: = softmax of the (masked) scores */
            double m = -INFINITY;
            for (int64_t j = 0; j < lk; ++j) {
              double acc = 0.0;
              for (int64_t t = 0; t < d; ++t) acc += qi[t] * k[at(krow0 + j, hk, t, heads_kv, d)];
              p[j] = (causal && j > i) ? -INFINITY : scale * acc;
              if (p[j] > m) m = p[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < lk; ++j) l += exp(p[j] - m);
            for (int64_t j = 0; j < lk; ++j) p[j] = exp(p[j] - m) / l;
            /* dP_ij = <do_i, v_j>;  D_i = sum_j P_ij dP_ij */
            double di = 0.0;
            for (int64_t j = 0; j < lk; ++j) {
              double acc = 0.0;
              for (int64_t t = 0; t < d; ++t) acc += doi[t] * v[at(krow0 + j, hk, t, heads_kv, d)];
              dp[j] = acc;
              di += p[j] * acc;
            }
            /* dS_ij = P_ij (dP_ij - D_i); dq_i = scale sum_j dS_ij k_j; dk_j += scale dS_ij q_i;
             * dv_j += P_ij do_i */
            for (int64_t t = 0; t < d; ++t) dqi[t] = 0.0;
            for (int64_t j = 0; j < lk; ++j) {
              double ds = p[j] * (dp[j] - di);
              for (int64_t t = 0; t < d; ++t) {
                dqi[t] += scale * ds * k[at(krow0 + j, hk, t, heads_kv, d)];
                dk[at(krow0 + j, hk, t, heads_kv, d)] += scale * ds * qi[t];
                dv[at(krow0 + j, hk, t, heads_kv, d)] += p[j] * doi[t];
              }
            }
          }
      }
    free(p);
    free(dp);
  }
  return failed ? -1 : 0;
}

/*
 * Row statistics of query row i of head h (section 13.1): fills p[j] = P_ij over the lk keys
 * (0 above the diagonal when causal), dp[j] = <do_i, v_j>, and returns D_i = sum_j P_ij dP_ij;
 * *lse_out = m + log l.
 */
static double bwd_row(const double *q, const double *k, const double *v, const double *dout,
                      int64_t qrow0, int64_t krow0, int64_t i, int64_t lk, int64_t h, int64_t hk,
                      int64_t heads, int64_t heads_kv, int64_t d, double scale, int causal,
                      double *p, double *dp, double *lse_out) {
  const double *qi = q + at(qrow0 + i, h, 0, heads, d);
  const double *doi = dout + at(qrow0 + i, h, 0, heads, d);
  double m = -INFINITY;
  for (int64_t j = 0; j < lk; ++j) {
    double acc = 0.0;
    for (int64_t t = 0; t < d; ++t) acc += qi[t] * k[at(krow0 + j, hk, t, heads_kv, d)];
    p[j] = (causal && j > i) ? -INFINITY : scale * acc;
    if (p[j] > m) m = p[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < lk; ++j) l += exp(p[j] - m);
  for (int64_t j = 0; j < lk; ++j) p[j] = exp(p[j] - m) / l;
  double di = 0.0;
  for (int64_t j = 0; j < lk; ++j) {
    double acc = 0.0;
    for (int64_t t = 0; t < d; ++t) acc += doi[t] * v[at(krow0 + j, hk, t, heads_kv, d)];
    dp[j] = acc;
    di += p[j] * acc;
  }
  *lse_out = m + log(l);
  return di;
}

/*
 * Selected rows of the backward pass (for sampled checks at full size), the same definition
 * as oracle_attention_bwd:
 *  - qrows: n_qrows triples (b, h, i); dq_rows [n_qrows, d] receives dQ of query row i of head h;
 *  - krows: n_krows triples (b, hk, j); dk_rows, dv_rows [n_krows, d] receive dK, dV of key j of
 *    K/V head hk (summed over the query heads of its group).  For a key row every query row of
 *    the group's heads contributes P_ij and dS_ij, which need that row's LSE and D; those are
 *    computed for all rows of (b, hk) once, when the key rows move to a new (b, hk), so key rows
 *    should be grouped by (b, hk).
 * Layouts and cu as in oracle_attention.  Returns 0, -1 if memory could not be obtained, -2 if
 * heads_kv does not divide heads.
 */
int oracle_attention_bwd_rows(const double *q, const double *k, const double *v, const double *dout,
                              int64_t batch, int64_t nq, int64_t nk, int64_t heads, int64_t heads_kv,
                              int64_t d, double scale, int causal, const int64_t *cu,
                              const int64_t *qrows, int64_t n_qrows, double *dq_rows,
                              const int64_t *krows, int64_t n_krows, double *dk_rows, double *dv_rows) {
  if (heads_kv <= 0 || heads % heads_kv != 0) return -2;
  const int64_t group = heads / heads_kv;
  int64_t max_nk = nk, max_nq = nq;
  if (cu) {
    max_nk = 0;
    for (int64_t b = 0; b < batch; ++b) if (cu[b + 1] - cu[b] > max_nk) max_nk = cu[b + 1] - cu[b];
    max_nq = max_nk;
  }
  int failed = 0;
  /* dQ rows: one query row each */
#pragma omp parallel
  {
    double *p = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    double *dp = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
    if (!p || !dp) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_qrows; ++r) {
      if (!p || !dp) continue;
      int64_t b = qrows[3 * r], h = qrows[3 * r + 1], i = qrows[3 * r + 2];
      int64_t lk = cu ? cu[b + 1] - cu[b] : nk;
      int64_t qrow0 = cu ? cu[b] : b * nq;
      int64_t krow0 = cu ? cu[b] : b * nk;
      double lse;
      double di = bwd_row(q, k, v, dout, qrow0, krow0, i, lk, h, h / group, heads, heads_kv, d, scale,
                          causal, p, dp, &lse);
      for (int64_t t = 0; t < d; ++t) dq_rows[r * d + t] = 0.0;
      for (int64_t j = 0; j < lk; ++j) {
        double ds = p[j] * (dp[j] - di);
        for (int64_t t = 0; t < d; ++t) dq_rows[r * d + t] += scale * ds * k[at(krow0 + j, h / group, t, heads_kv, d)];
      }
    }
    free(p);
    free(dp);
  }
  if (failed) return -1;
  /* dK, dV rows: LSE and D of every query row of the group, then the sums over query rows */
  double *lse_all = (double *)malloc(sizeof(double) * (size_t)(group * (max_nq > 0 ? max_nq : 1)));
  double *d_all = (double *)malloc(sizeof(double) * (size_t)(group * (max_nq > 0 ? max_nq : 1)));
  if (!lse_all || !d_all) {
    free(lse_all);
    free(d_all);
    return -1;
  }
  int64_t cur_b = -1, cur_hk = -1;
  for (int64_t r = 0; r < n_krows && !failed; ++r) {
    int64_t b = krows[3 * r], hk = krows[3 * r + 1], j = krows[3 * r + 2];
    int64_t lq = cu ? cu[b + 1] - cu[b] : nq;
    int64_t lk = cu ? cu[b + 1] - cu[b] : nk;
    int64_t qrow0 = cu ? cu[b] : b * nq;
    int64_t krow0 = cu ? cu[b] : b * nk;
    if (b != cur_b || hk != cur_hk) {
#pragma omp parallel
      {
        double *p = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(max_nk > 0 ? max_nk : 1));
        if (!p || !dp) {
#pragma omp atomic write
          failed = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t g = 0; g < group; ++g)
          for (int64_t i = 0; i < lq; ++i) {
            if (!p || !dp) continue;
            double lse;
            d_all[g * max_nq + i] = bwd_row(q, k, v, dout, qrow0, krow0, i, lk, hk * group + g, hk, heads,
                                            heads_kv, d, scale, causal, p, dp, &lse);
            lse_all[g * max_nq + i] = lse;
          }
        free(p);
        free(dp);
      }
      cur_b = b;
      cur_hk = hk;
      if (failed) break;
    }
    for (int64_t t = 0; t < d; ++t) {
      dk_rows[r * d + t] = 0.0;
      dv_rows[r * d + t] = 0.0;
    }
    for (int64_t g = 0; g < group; ++g) {
      int64_t h = hk * group + g;
      for (int64_t i = 0; i < lq; ++i) {
        if (causal && j > i) continue; /* P_ij = 0 */
        const double *qi = q + at(qrow0 + i, h, 0, heads, d);
        const double *doi = dout + at(qrow0 + i, h, 0, heads, d);
        double s = 0.0, dpij = 0.0;
        for (int64_t t = 0; t < d; ++t) {
          s += qi[t] * k[at(krow0 + j, hk, t, heads_kv, d)];
          dpij += doi[t] * v[at(krow0 + j, hk, t, heads_kv, d)];
        }
        double pij = exp(scale * s - lse_all[g * max_nq + i]);
        double ds = pij * (dpij - d_all[g * max_nq + i]);
        for (int64_t t = 0; t < d; ++t) {
          dv_rows[r * d + t] += pij * doi[t];
          dk_rows[r * d + t] += scale * ds * qi[t];
        }
      }
    }
  }
  free(lse_all);
  free(d_all);
  return failed ? -1 : 0;
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
