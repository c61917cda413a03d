/*
 * Sanitizer driver for the fp64 oracle (test infrastructure).  Compiles the
 * oracle's source into this program and runs it on random tiny problems:
 * empty sequences and blocks, rank-0 factors, ragged tails, causal chunks
 * and selected-row subsets.  Every value row is made exactly 1 (U' a column
 * of ones, W' a row of ones, the tail's V all ones), so every output element
 * must be 1 for a row that sees any token and 0 (lse -inf) for one that sees
 * none; that checks the result without restating the oracle's arithmetic.
 * Built with gcc -fsanitize=address,undefined by tests/test_sanitize.py.
 */
#include "../../oracle/milo_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {   /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static double unif(void) { return (rnd() / 4294967296.0) * 2.0 - 1.0; }

int main(void) {
  int failures = 0, rows_checked = 0;
  for (int trial = 0; trial < 300; ++trial) {
    const int n_seq = 1 + rnd() % 3, q_len = 1 + rnd() % 4, hkv = 1 + rnd() % 2, grp = 1 + rnd() % 3;
    const int hq = hkv * grp, d = (rnd() & 1) ? 8 : 16;
    const int tail_cap = rnd() % 10;
    int64_t* seq_blk = malloc(sizeof(int64_t) * (n_seq + 1));
    int nblk_total = 0;
    seq_blk[0] = 0;
    for (int i = 0; i < n_seq; ++i) {
      nblk_total += rnd() % 4;
      seq_blk[i + 1] = nblk_total;
    }
    int32_t* tok = malloc(sizeof(int32_t) * (nblk_total + 1));
    int32_t* rk = malloc(sizeof(int32_t) * (nblk_total + 1));
    int32_t* rv = malloc(sizeof(int32_t) * (nblk_total + 1));
    int64_t* base = malloc(sizeof(int64_t) * (nblk_total + 1));
    int64_t nfac = 0;
    static const int toks[4] = {0, 1, 5, 17};
    for (int b = 0; b < nblk_total; ++b) {
      tok[b] = toks[rnd() % 4];
      rk[b] = rnd() % (d + 1);
      rv[b] = 1;                                  /* values: U' = ones column, W' = ones row */
      base[b] = nfac;
      nfac += (int64_t)hkv * ((int64_t)tok[b] * rk[b] + (int64_t)rk[b] * d + (int64_t)tok[b] * rv[b] +
                              (int64_t)rv[b] * d);
    }
    double* fac = malloc(sizeof(double) * (nfac + 1));
    for (int b = 0; b < nblk_total; ++b)
      for (int g = 0; g < hkv; ++g) {
        const int64_t per = (int64_t)tok[b] * rk[b] + (int64_t)rk[b] * d + (int64_t)tok[b] * rv[b] +
                            (int64_t)rv[b] * d;
        double* f = fac + base[b] + g * per;
        const int64_t nuw = (int64_t)tok[b] * rk[b] + (int64_t)rk[b] * d;
        for (int64_t x = 0; x < nuw; ++x) f[x] = unif();
        for (int64_t x = nuw; x < per; ++x) f[x] = 1.0;
      }
    const size_t nq = (size_t)n_seq * q_len * hq * d;
    double* q = malloc(sizeof(double) * nq);
    for (size_t x = 0; x < nq; ++x) q[x] = 3.0 * unif();
    const size_t nt = (size_t)n_seq * hkv * tail_cap * d;
    double* kt = malloc(sizeof(double) * (nt + 1));
    double* vt = malloc(sizeof(double) * (nt + 1));
    for (size_t x = 0; x < nt; ++x) { kt[x] = unif(); vt[x] = 1.0; }
    int32_t* tl = malloc(sizeof(int32_t) * n_seq);
    for (int i = 0; i < n_seq; ++i) tl[i] = tail_cap ? (int32_t)(rnd() % (tail_cap + 1)) : 0;
    double* out = malloc(sizeof(double) * nq);
    double* lse = malloc(sizeof(double) * ((size_t)n_seq * q_len * hq));
    for (size_t x = 0; x < nq; ++x) out[x] = NAN;
    const int n_sel = (rnd() & 1) ? 1 + (int)(rnd() % 5) : 0;
    int32_t* sel = malloc(sizeof(int32_t) * 3 * (n_sel + 1));
    for (int k = 0; k < n_sel; ++k) {
      sel[3 * k] = rnd() % n_seq;
      sel[3 * k + 1] = rnd() % q_len;
      sel[3 * k + 2] = rnd() % hq;
    }
    milo_oracle_args a = {n_seq, q_len, hq, hkv, d, 1.0 / sqrt((double)d), q, seq_blk, tok, rk, rv, base, fac,
                          tail_cap, kt, vt, tl, out, lse, n_sel ? sel : NULL, n_sel};
    if (milo_oracle_attend(&a) != 0) {
      fprintf(stderr, "trial %d: oracle returned an error\n", trial);
      ++failures;
    }
    /* check every computed row */
    for (int i = 0; i < n_seq; ++i)
      for (int j = 0; j < q_len; ++j)
        for (int h = 0; h < hq; ++h) {
          int wanted = n_sel == 0;
          for (int k = 0; k < n_sel; ++k)
            wanted |= sel[3 * k] == i && sel[3 * k + 1] == j && sel[3 * k + 2] == h;
          if (!wanted) continue;
          int visible = 0;
          for (int64_t b = seq_blk[i]; b < seq_blk[i + 1]; ++b) visible += tok[b];
          const int vis_tail = tl[i] - q_len + j + 1;
          visible += q_len == 1 ? tl[i] : (vis_tail > 0 ? vis_tail : 0);
          const size_t row = ((size_t)(i * q_len + j) * hq + h);
          for (int c = 0; c < d; ++c) {
            const double o = out[row * d + c];
            const double want = visible ? 1.0 : 0.0;
            if (!(fabs(o - want) <= 1e-12)) {
              if (failures < 10) fprintf(stderr, "trial %d row (%d,%d,%d): out %g, want %g\n", trial, i, j, h, o, want);
              ++failures;
            }
          }
          if (visible ? !isfinite(lse[row]) : !(isinf(lse[row]) && lse[row] < 0)) ++failures;
          ++rows_checked;
        }
    free(seq_blk); free(tok); free(rk); free(rv); free(base); free(fac); free(q);
    free(kt); free(vt); free(tl); free(out); free(lse); free(sel);
  }
  printf("oracle driver: %d rows checked, %d failures\n", rows_checked, failures);
  return failures == 0 ? 0 : 1;
}
