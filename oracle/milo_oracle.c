/*
 * milo_oracle.c -- fp64 CPU oracle for attention over a block-wise low-rank
 * compressed KV cache.  TEST INFRASTRUCTURE ONLY: it is called by the tests,
 * by the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no code with the HIP library.
 *
 * What it computes (MILO summary, "4.4 MILO Workflow": at inference MILO
 * retrieves the selected blocks, reconstructs them and applies attention;
 * "4.2 Block-wise Low-Rank Compression": each block's keys and values are
 * approximated separately, K_b ~= U_b W_b and V_b ~= U'_b W'_b):
 *
 *   for every sequence i and KV head g
 *     K = [ U_1 W_1 ; ... ; U_n W_n ; K_tail ]     (dense reconstruction)
 *     V = [ U'_1 W'_1 ; ... ; U'_n W'_n ; V_tail ]
 *   for every query row (position j, query head h of group g = h / G)
 *     s_t = scale * <K_t, q>      over every block token and the visible tail
 *     a   = softmax(s)            (exact two-pass: max, then sum)
 *     o   = sum_t a_t V_t,  lse = max + log(sum exp(s - max))
 *
 * Readings where the pages are silent (each listed with its reason in the
 * design notes): query head h reads KV head h / G; every block token is
 * visible; tail token l is visible to query position j iff
 * l <= tail_len - q_len + j (bottom-right causal; with q_len = 1 the whole
 * tail); a rank-0 factor contributes zeros that still count in the softmax;
 * with nothing visible, o = 0 and lse = -inf.
 *
 * All arithmetic is double precision on the exact stored input values.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t n_seq, q_len, n_q_heads, n_kv_heads, head_dim;
  double scale;
  const double* q;          /* [n_seq][q_len][n_q_heads][head_dim]                    */
  const int64_t* seq_blk;   /* [n_seq+1]: blocks of sequence i are seq_blk[i]..[i+1]  */
  const int32_t* blk_tok;   /* per block: T_b                                          */
  const int32_t* blk_rk;    /* per block: r_b  (keys)                                  */
  const int32_t* blk_rv;    /* per block: r'_b (values)                                */
  const int64_t* blk_base;  /* per block: offset in fac of KV head 0's factors         */
  const double* fac;        /* per (block, kv head), heads consecutive:
                               U[T][r] | W[r][d] | U'[T][r'] | W'[r'][d]               */
  int32_t tail_cap;
  const double* k_tail;     /* [n_seq][n_kv_heads][tail_cap][head_dim]                 */
  const double* v_tail;
  const int32_t* tail_len;  /* [n_seq]                                                 */
  double* out;              /* [n_seq][q_len][n_q_heads][head_dim]                     */
  double* lse;              /* [n_seq][q_len][n_q_heads]                               */
  const int32_t* sel;       /* optional: n_sel triples (seq, q_pos, q_head) to compute */
  int32_t n_sel;
} milo_oracle_args;

/* K_b = U_b W_b and V_b = U'_b W'_b for one block and KV head, written as rows
 * of the dense per-(sequence, head) matrices. */
static void reconstruct_block(const double* f, int T, int r, int rv, int d,
                              double* K, double* V) {
  const double* U = f;
  const double* W = U + (size_t)T * r;
  const double* Up = W + (size_t)r * d;
  const double* Wp = Up + (size_t)T * rv;
  for (int t = 0; t < T; ++t) {
    double* kr = K + (size_t)t * d;
    double* vr = V + (size_t)t * d;
    for (int c = 0; c < d; ++c) { kr[c] = 0.0; vr[c] = 0.0; }
    for (int k = 0; k < r; ++k) {
      const double u = U[(size_t)t * r + k];
      const double* wr = W + (size_t)k * d;
      for (int c = 0; c < d; ++c) kr[c] += u * wr[c];
    }
    for (int k = 0; k < rv; ++k) {
      const double u = Up[(size_t)t * rv + k];
      const double* wr = Wp + (size_t)k * d;
      for (int c = 0; c < d; ++c) vr[c] += u * wr[c];
    }
  }
}

/* Plain softmax attention of one query row over the first n rows of K, V. */
static void attend_row(const double* qv, const double* K, const double* V, int64_t n, int d,
                       double scale, double* s, double* o, double* lse) {
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (n == 0) { *lse = -INFINITY; return; }
  double mx = -INFINITY;
  for (int64_t t = 0; t < n; ++t) {
    double acc = 0.0;
    const double* kr = K + (size_t)t * d;
    for (int c = 0; c < d; ++c) acc += kr[c] * qv[c];
    s[t] = scale * acc;
    if (s[t] > mx) mx = s[t];
  }
  double z = 0.0;
  for (int64_t t = 0; t < n; ++t) { s[t] = exp(s[t] - mx); z += s[t]; }
  for (int64_t t = 0; t < n; ++t) {
    const double a = s[t] / z;
    const double* vr = V + (size_t)t * d;
    for (int c = 0; c < d; ++c) o[c] += a * vr[c];
  }
  *lse = mx + log(z);
}

/* Returns 0 on success, -1 on a bad argument, -2 if memory ran out. */
int milo_oracle_attend(const milo_oracle_args* a) {
  if (!a || a->n_seq < 0 || a->q_len < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1 ||
      a->head_dim < 1 || a->n_q_heads % a->n_kv_heads != 0 || !a->q || !a->seq_blk ||
      !a->out || !a->lse)
    return -1;
  const int d = a->head_dim, Q = a->q_len, Hq = a->n_q_heads, Hkv = a->n_kv_heads;
  const int G = Hq / Hkv;

  for (int i = 0; i < a->n_seq; ++i) {
    for (int g = 0; g < Hkv; ++g) {
      /* which query rows of this (sequence, KV head) are wanted */
      int want = 0;
      if (!a->sel) want = 1;
      else
        for (int e = 0; e < a->n_sel && !want; ++e)
          if (a->sel[3 * e] == i && a->sel[3 * e + 2] / G == g) want = 1;
      if (!want) continue;

      const int64_t b0 = a->seq_blk[i], b1 = a->seq_blk[i + 1];
      const int L = a->tail_cap > 0 ? a->tail_len[i] : 0;
      int64_t nblk_tok = 0;
      for (int64_t b = b0; b < b1; ++b) nblk_tok += a->blk_tok[b];
      const int64_t n_all = nblk_tok + L;
      double* K = (double*)malloc(sizeof(double) * (size_t)(n_all ? n_all : 1) * d);
      double* V = (double*)malloc(sizeof(double) * (size_t)(n_all ? n_all : 1) * d);
      if (!K || !V) { free(K); free(V); return -2; }

      /* row offset of each block inside K, V */
      int64_t* row0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(b1 - b0 + 1));
      if (!row0) { free(K); free(V); return -2; }
      row0[0] = 0;
      for (int64_t b = b0; b < b1; ++b) row0[b - b0 + 1] = row0[b - b0] + a->blk_tok[b];

#pragma omp parallel for schedule(dynamic, 1)
      for (int64_t b = b0; b < b1; ++b) {
        const int T = a->blk_tok[b], r = a->blk_rk[b], rv = a->blk_rv[b];
        const size_t head_sz = (size_t)T * r + (size_t)r * d + (size_t)T * rv + (size_t)rv * d;
        const double* f = a->fac + a->blk_base[b] + (size_t)g * head_sz;
        reconstruct_block(f, T, r, rv, d, K + (size_t)row0[b - b0] * d, V + (size_t)row0[b - b0] * d);
      }
      for (int t = 0; t < L; ++t) {
        const size_t src = (((size_t)i * Hkv + g) * a->tail_cap + t) * d;
        memcpy(K + (size_t)(nblk_tok + t) * d, a->k_tail + src, sizeof(double) * d);
        memcpy(V + (size_t)(nblk_tok + t) * d, a->v_tail + src, sizeof(double) * d);
      }

      /* every query row (j, h) of this group */
      const int n_rows = Q * G;
#pragma omp parallel
      {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_all ? n_all : 1));
#pragma omp for schedule(dynamic, 1)
        for (int row = 0; row < n_rows; ++row) {
          const int j = row / G, h = g * G + row % G;
          int take = !a->sel;
          for (int e = 0; e < a->n_sel && !take; ++e)
            if (a->sel[3 * e] == i && a->sel[3 * e + 1] == j && a->sel[3 * e + 2] == h) take = 1;
          if (!take || !s) continue;
          /* visible tail: tokens l <= L - Q + j */
          int64_t vis_tail = (int64_t)L - Q + j + 1;
          if (vis_tail < 0) vis_tail = 0;
          if (vis_tail > L) vis_tail = L;
          const size_t qi = (((size_t)i * Q + j) * Hq + h);
          attend_row(a->q + qi * d, K, V, nblk_tok + vis_tail, d, a->scale, s,
                     a->out + qi * d, a->lse + qi);
        }
        free(s);
      }
      free(row0);
      free(K);
      free(V);
    }
  }
  return 0;
}

/* Threads the oracle's parallel regions use. */
int milo_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
