/*
 * CPU oracle for the attention forward and backward passes -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load this
 * code.  It shares nothing with the GPU library: no headers, no helpers, no
 * tables.  Everything is double precision, row by row, with no blocking beyond
 * what each definition states.
 *
 * Tensor layouts (the pages' [batch, seqlen, heads, head_dim] convention, from
 * "flash attention V2 code walk-through", tensor-shape table):
 *   q [B, Sq, Hq, d]   k, v [B, Sk, Hkv, d]   o [B, Sq, Hq, d]   lse [B, Hq, Sq]
 * Inputs are either double arrays (in_bf16 = 0) or bf16 bit patterns
 * (in_bf16 = 1), which are widened exactly to double.
 *
 * Definitions followed:
 *  - Scores s_j = scale * <q_i, k_j> and O = softmax(s) V, with the full score
 *    row and probability row materialised: "FlashAttention 1, 2, 3" explainer,
 *    shape section (S = QK^T/sqrt(d), P = softmax_rows(S + mask), O = PV) and
 *    the naive three-step section.  `scale` replaces 1/sqrt(d) as given.
 *  - GQA: query head h reads key/value head h / (Hq/Hkv) ("flash attention V2
 *    code walk-through", parallelism section: the decode reshape groups
 *    consecutive query heads per KV head).
 *  - Causal mask aligned to the bottom-right: key j is visible to query i iff
 *    j <= i + Sk - Sq ("03 forward CUDA kernel" section 8; walk-through
 *    Is_causal mask pictures for Sq=2,Sk=5 and Sq=5,Sk=2).  Masked scores are
 *    set to -inf after scaling and before the max (explainer, causal/tail
 *    section).
 *  - A row with no visible key returns O = 0 and LSE = -inf (explainer,
 *    one-row runnable logic; forward-kernel page section 7.3).
 *  - LSE = m + ln(l), natural log (explainer, one-row runnable logic and the
 *    backward-recompute section).
 *  - Online variant: the explainer's per-row loop over key tiles with state
 *    (m, l, o), alpha = exp(m - m') applied to both l and o, fully masked tiles
 *    skipped, alpha taken as 0 on the first tile with a valid key.
 *  - Split variant: the key tiles are cut into num_splits contiguous ranges of
 *    ceil(n_tiles / num_splits) tiles (walk-through, split-KV block range);
 *    each range yields (O_s, LSE_s) or (0, -inf) when empty; the combine takes
 *    LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s
 *    (forward-kernel page section 7.3).
 *  - Mask and bias variants (walk-through, the split-KV kernel's template flags
 *    Is_local, Has_alibi and Is_softcap, and its n_block_min / n_block_max
 *    clipping).  With diag = i + Sk - Sq, the key aligned with query i:
 *      sliding window: key j is visible iff diag - window_left <= j <= diag +
 *        window_right; a negative bound means no limit on that side.  Causal
 *        keeps its own limit j <= diag, so causal with a window is the window
 *        with its right side at most 0 (the pages treat the two as exclusive;
 *        this is the reading that agrees with both);
 *      ALiBi: -slope_{b,h} * |diag - j| is added to the score of key j;
 *      soft cap: the scaled score s becomes c * tanh(s / c) (c > 0; a tanh
 *        limit on the logits, the page names no formula; this is its plain form).
 *    The order is: scale, soft cap, ALiBi bias, then the mask.  The soft cap acts
 *    on the dot-product logit alone and the bias is added to the capped logit.
 *  - FP8 forward (explainer, FlashAttention-3 precision section: FP8 inputs with a
 *    scale per block, the scales carried into the computation, softmax statistics and
 *    scaling in fp32, and an orthogonal transform of Q and K that keeps QK^T).  The
 *    format is OCP FP8 E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *    exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; no infinities; the
 *    largest finite value is 448.  A tensor x [B, S, H, d] is quantized per (b, h,
 *    block of 128 rows): amax = max |x| over the block, scale = fp32(amax / 448) (1 for
 *    an all-zero block), code = nearest E4M3 value to fp32(x / scale), ties to the even
 *    code, saturating at +-448.  The optional rotation applies the Walsh-Hadamard
 *    transform along d (butterflies of distance 1, 2, 4, ..., d/2, each pair (a, b)
 *    becoming (a + b, a - b) in fp32) and then multiplies by fp32(1 / sqrt(d)).  The FP8
 *    attention is the plain definition on the dequantized tensors code * scale.
 *  - Backward (explainer, sections "backward: from the softmax derivative",
 *    "training: backward recomputation" and "backward: back to Q, K, V"): with the
 *    dense probability row P of the plain definition and the upstream gradient dO,
 *      D    = sum_c dO_c O_c            (one scalar per row; equals sum_j P_j dP_j)
 *      dP_j = <dO, v_j>
 *      dS_j = P_j (dP_j - D)
 *      dQ   = scale * sum_j dS_j k_j     dK_j += scale * dS_j q     dV_j += P_j dO
 *    The scale enters dQ and dK as the 1/sqrt(d) of the page's table does.  Masked
 *    keys have P = dS = 0; a row with no visible key contributes nothing.  With GQA,
 *    dK and dV of a key/value head sum over the Hq/Hkv query heads that read it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int in_bf16;
  const void *q, *k, *v;
  int B, Sq, Sk, Hq, Hkv, d, causal;
  double scale;
  int window_left, window_right; /* -1: no limit on that side */
  const double *alibi;           /* slopes [B, Hq], or NULL */
  double softcap;                /* 0: none */
} problem;

static double elem(const void *base, int in_bf16, int64_t idx) {
  if (in_bf16) {
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return ((const double *)base)[idx];
}

static int check(const problem *p) {
  if (!p->q || !p->k || !p->v) return 1;
  if (p->B < 0 || p->Sq < 0 || p->Sk < 0 || p->Hq < 1 || p->Hkv < 1 || p->d < 1) return 2;
  if (p->Hq % p->Hkv != 0) return 3;
  if (p->window_left < -1 || p->window_right < -1) return 7;
  if (!(p->softcap >= 0.0) || isinf(p->softcap)) return 8;
  return 0;
}

static int64_t q_index(const problem *p, int b, int i, int h, int c) {
  return (((int64_t)b * p->Sq + i) * p->Hq + h) * p->d + c;
}

static int64_t kv_index(const problem *p, int b, int j, int hk, int c) {
  return (((int64_t)b * p->Sk + j) * p->Hkv + hk) * p->d + c;
}

static int kv_head(const problem *p, int h) { return h / (p->Hq / p->Hkv); }

/* Visibility of key j to query i: the bottom-right causal limit and the sliding window,
 * both measured from diag = i + Sk - Sq. */
static int visible(const problem *p, int i, int j) {
  const long long diag = (long long)i + p->Sk - p->Sq;
  if (p->causal && !(j <= diag)) return 0;
  if (p->window_left >= 0 && j < diag - p->window_left) return 0;
  if (p->window_right >= 0 && j > diag + p->window_right) return 0;
  return 1;
}

/* Logit of query (b,i,h) against key j: the scaled dot product, soft-capped when a cap
 * is set, plus the ALiBi bias when slopes are given. */
static double score(const problem *p, int b, int h, int i, int j) {
  int hk = kv_head(p, h);
  double acc = 0.0;
  for (int c = 0; c < p->d; ++c)
    acc += elem(p->q, p->in_bf16, q_index(p, b, i, h, c)) *
           elem(p->k, p->in_bf16, kv_index(p, b, j, hk, c));
  double s = p->scale * acc;
  if (p->softcap > 0.0) s = p->softcap * tanh(s / p->softcap);
  if (p->alibi) {
    const double dist = (double)((long long)i + p->Sk - p->Sq - j);
    s -= p->alibi[(int64_t)b * p->Hq + h] * fabs(dist);
  }
  return s;
}

/* Full score row S[0..Sk) with the mask applied, and its probability row P.
 * Returns the number of visible keys; m and l receive max and sum of exp. */
static int prob_row(const problem *p, int b, int h, int i, double *s, double *prob,
                    double *m_out, double *l_out) {
  int nvis = 0;
  for (int j = 0; j < p->Sk; ++j) s[j] = score(p, b, h, i, j);
  for (int j = 0; j < p->Sk; ++j) {
    if (visible(p, i, j))
      ++nvis;
    else
      s[j] = -INFINITY;
  }
  if (nvis == 0) {
    for (int j = 0; j < p->Sk; ++j) prob[j] = 0.0;
    *m_out = -INFINITY;
    *l_out = 0.0;
    return 0;
  }
  double m = -INFINITY;
  for (int j = 0; j < p->Sk; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (int j = 0; j < p->Sk; ++j) {
    prob[j] = exp(s[j] - m);
    l += prob[j];
  }
  for (int j = 0; j < p->Sk; ++j) prob[j] /= l;
  *m_out = m;
  *l_out = l;
  return nvis;
}

/* One row of the plain definition: O[i,:] = P V and LSE = m + ln l. */
static void oneshot_row(const problem *p, int b, int h, int i, double *s, double *prob,
                        double *o_row, double *lse) {
  double m, l;
  int nvis = prob_row(p, b, h, i, s, prob, &m, &l);
  if (nvis == 0) {
    for (int c = 0; c < p->d; ++c) o_row[c] = 0.0;
    *lse = -INFINITY;
    return;
  }
  int hk = kv_head(p, h);
  for (int c = 0; c < p->d; ++c) {
    double acc = 0.0;
    for (int j = 0; j < p->Sk; ++j)
      acc += prob[j] * elem(p->v, p->in_bf16, kv_index(p, b, j, hk, c));
    o_row[c] = acc;
  }
  *lse = m + log(l);
}

/* The explainer's per-row online loop over key tiles [t_lo, t_hi) of size blk.
 * Produces the normalised row output and its LSE, or (0, -inf). */
static void online_row(const problem *p, int b, int h, int i, int blk, int t_lo, int t_hi,
                       double *s, double *o_row, double *lse) {
  int hk = kv_head(p, h);
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < p->d; ++c) o_row[c] = 0.0;
  for (int t = t_lo; t < t_hi; ++t) {
    int j0 = t * blk;
    int j1 = j0 + blk < p->Sk ? j0 + blk : p->Sk;
    int any = 0;
    double tile_max = -INFINITY;
    for (int j = j0; j < j1; ++j) {
      double sj = score(p, b, h, i, j);
      if (!visible(p, i, j)) sj = -INFINITY;
      else any = 1;
      s[j - j0] = sj;
      if (sj > tile_max) tile_max = sj;
    }
    if (!any) continue; /* fully masked tile: skipped */
    double m2 = m > tile_max ? m : tile_max;
    double alpha = (l != 0.0) ? exp(m - m2) : 0.0;
    double psum = 0.0;
    for (int j = j0; j < j1; ++j) {
      s[j - j0] = exp(s[j - j0] - m2);
      psum += s[j - j0];
    }
    for (int c = 0; c < p->d; ++c) {
      double pv = 0.0;
      for (int j = j0; j < j1; ++j)
        pv += s[j - j0] * elem(p->v, p->in_bf16, kv_index(p, b, j, hk, c));
      o_row[c] = alpha * o_row[c] + pv;
    }
    l = alpha * l + psum;
    m = m2;
  }
  if (l == 0.0) {
    for (int c = 0; c < p->d; ++c) o_row[c] = 0.0;
    *lse = -INFINITY;
    return;
  }
  for (int c = 0; c < p->d; ++c) o_row[c] /= l;
  *lse = m + log(l);
}

#define SETUP_PROBLEM_OPTS(WL, WR, ALIBI, CAP)                                          \
  problem P = {in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, WL, WR, ALIBI, CAP}; \
  int err = check(&P);                                                                   \
  if (err) return err;
#define SETUP_PROBLEM SETUP_PROBLEM_OPTS(-1, -1, NULL, 0.0)

/* Plain definition over all rows. o [B,Sq,Hq,d], lse [B,Hq,Sq]. */
int oracle_attn_fwd_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                        int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                        int window_left, int window_right, const double *alibi,
                        double softcap, double *o, double *lse) {
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  int64_t nrows = (int64_t)B * Hq * Sq;
  #pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
    double *prob = (double *)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
    #pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int b = (int)(r / ((int64_t)Hq * Sq));
      int h = (int)((r / Sq) % Hq);
      int i = (int)(r % Sq);
      oneshot_row(&P, b, h, i, s, prob, o + q_index(&P, b, i, h, 0),
                  lse + ((int64_t)b * Hq + h) * Sq + i);
    }
    free(s);
    free(prob);
  }
  return 0;
}

int oracle_attn_fwd(int in_bf16, const void *q, const void *k, const void *v, int B, int Sq,
                    int Sk, int Hq, int Hkv, int d, int causal, double scale, double *o,
                    double *lse) {
  return oracle_attn_fwd_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1, -1,
                             NULL, 0.0, o, lse);
}

/* Plain definition on selected rows.  rows holds nrows triples (b, h, i);
 * o_rows [nrows, d], lse_rows [nrows]. */
int oracle_attn_rows_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                         int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                         int window_left, int window_right, const double *alibi,
                         double softcap, int nrows, const int *rows, double *o_rows,
                         double *lse_rows) {
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  for (int r = 0; r < nrows; ++r) {
    int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) return 4;
  }
  #pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
    double *prob = (double *)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
    #pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r)
      oneshot_row(&P, rows[3 * r], rows[3 * r + 1], rows[3 * r + 2], s, prob,
                  o_rows + (int64_t)r * d, lse_rows + r);
    free(s);
    free(prob);
  }
  return 0;
}

int oracle_attn_rows(int in_bf16, const void *q, const void *k, const void *v, int B,
                     int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                     int nrows, const int *rows, double *o_rows, double *lse_rows) {
  return oracle_attn_rows_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1,
                              -1, NULL, 0.0, nrows, rows, o_rows, lse_rows);
}

/* The probability row P[b,h,i,:] of the plain definition (zeros if no key is visible). */
int oracle_attn_probs_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                          int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                          int window_left, int window_right, const double *alibi,
                          double softcap, int b, int h, int i, double *prob) {
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) return 4;
  double *s = (double *)malloc(sizeof(double) * (Sk > 0 ? Sk : 1));
  double m, l;
  prob_row(&P, b, h, i, s, prob, &m, &l);
  free(s);
  return 0;
}

int oracle_attn_probs(int in_bf16, const void *q, const void *k, const void *v, int B,
                      int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                      int b, int h, int i, double *prob) {
  return oracle_attn_probs_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1,
                               -1, NULL, 0.0, b, h, i, prob);
}

/* Online (tiled) variant with key tile size blk. */
int oracle_attn_online_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                           int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                           int window_left, int window_right, const double *alibi,
                           double softcap, int blk, double *o, double *lse) {
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  if (blk < 1) return 5;
  int ntiles = (Sk + blk - 1) / blk;
  int64_t nrows = (int64_t)B * Hq * Sq;
  #pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * blk);
    #pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int b = (int)(r / ((int64_t)Hq * Sq));
      int h = (int)((r / Sq) % Hq);
      int i = (int)(r % Sq);
      online_row(&P, b, h, i, blk, 0, ntiles, s, o + q_index(&P, b, i, h, 0),
                 lse + ((int64_t)b * Hq + h) * Sq + i);
    }
    free(s);
  }
  return 0;
}

int oracle_attn_online(int in_bf16, const void *q, const void *k, const void *v, int B,
                       int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                       int blk, double *o, double *lse) {
  return oracle_attn_online_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1,
                                -1, NULL, 0.0, blk, o, lse);
}

/* Split-KV variant: num_splits contiguous tile ranges, each run with the online
 * loop, then the LSE-weighted combine.  o_part [S,B,Hq,Sq,d] and lse_part
 * [S,B,Hq,Sq] receive the per-split results (either may be NULL); o, lse the
 * combined result. */
int oracle_attn_split_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                          int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                          int window_left, int window_right, const double *alibi,
                          double softcap, int blk, int num_splits, double *o_part,
                          double *lse_part, double *o, double *lse) {
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  if (blk < 1) return 5;
  if (num_splits < 1) return 6;
  int ntiles = (Sk + blk - 1) / blk;
  int per_split = (ntiles + num_splits - 1) / num_splits;
  int64_t nrows = (int64_t)B * Hq * Sq;
  #pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * blk);
    double *os = (double *)malloc(sizeof(double) * num_splits * d);
    double *ls = (double *)malloc(sizeof(double) * num_splits);
    #pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
      int b = (int)(r / ((int64_t)Hq * Sq));
      int h = (int)((r / Sq) % Hq);
      int i = (int)(r % Sq);
      for (int sp = 0; sp < num_splits; ++sp) {
        int t_lo = sp * per_split;
        int t_hi = t_lo + per_split < ntiles ? t_lo + per_split : ntiles;
        if (t_lo > t_hi) t_lo = t_hi;
        online_row(&P, b, h, i, blk, t_lo, t_hi, s, os + (int64_t)sp * d, ls + sp);
        int64_t prow = (((int64_t)sp * B + b) * Hq + h) * Sq + i;
        if (o_part)
          memcpy(o_part + prow * d, os + (int64_t)sp * d, sizeof(double) * d);
        if (lse_part) lse_part[prow] = ls[sp];
      }
      /* combine */
      double lmax = -INFINITY;
      for (int sp = 0; sp < num_splits; ++sp)
        if (ls[sp] > lmax) lmax = ls[sp];
      double *orow = o + q_index(&P, b, i, h, 0);
      double *lrow = lse + ((int64_t)b * Hq + h) * Sq + i;
      if (lmax == -INFINITY) {
        for (int c = 0; c < d; ++c) orow[c] = 0.0;
        *lrow = -INFINITY;
        continue;
      }
      double sum = 0.0;
      for (int sp = 0; sp < num_splits; ++sp) sum += exp(ls[sp] - lmax);
      double L = lmax + log(sum);
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int sp = 0; sp < num_splits; ++sp)
          acc += exp(ls[sp] - L) * os[(int64_t)sp * d + c];
        orow[c] = acc;
      }
      *lrow = L;
    }
    free(s);
    free(os);
    free(ls);
  }
  return 0;
}

int oracle_attn_split(int in_bf16, const void *q, const void *k, const void *v, int B,
                      int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                      int blk, int num_splits, double *o_part, double *lse_part, double *o,
                      double *lse) {
  return oracle_attn_split_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1,
                               -1, NULL, 0.0, blk, num_splits, o_part, lse_part, o, lse);
}

/* Backward of the plain definition (see the header).  dout has q's layout and dtype
 * convention.  dq [B,Sq,Hq,d], dk, dv [B,Sk,Hkv,d], dsum [B,Hq,Sq] (D per row).
 * If dq_abs, dk_abs, dv_abs are non-NULL they receive, per element, the sum of the
 * absolute values of the terms that make up dq, dk, dv:
 *   scale * sum_j |dS_j| |k_jc|,  scale * sum_i |dS_ij| |q_ic|,  sum_i P_ij |dO_ic|.
 * units: NULL, or B*Hkv flags; only the (batch, key/value head) units with a non-zero
 * flag are computed (their query heads' dq and dsum rows, their dk and dv), the rest of
 * every output is zero.  Each unit is done in the two steps of the page's table: the
 * full P and dS rows of its query heads (rows in parallel; dq and D on the way), then
 * dV = P^T dO and dK = scale dS^T Q (keys in parallel). */
/* The backward with the sliding window and ALiBi.  Both leave the formulas above as they
 * are: a pair outside the window has P = 0, hence dS = 0, and the ALiBi bias does not
 * depend on q or k, so dQ and dK take dS as it stands.  The soft cap (whose derivative
 * 1 - tanh^2 would scale dS) is not covered: softcap != 0 returns 8. */
int oracle_attn_bwd_ext(int in_bf16, const void *q, const void *k, const void *v, int B,
                        int Sq, int Sk, int Hq, int Hkv, int d, int causal, double scale,
                        int window_left, int window_right, const double *alibi,
                        double softcap, const void *dout, const int *units, double *dq,
                        double *dk, double *dv, double *dsum, double *dq_abs,
                        double *dk_abs, double *dv_abs) {
  if (softcap != 0.0) return 8;
  SETUP_PROBLEM_OPTS(window_left, window_right, alibi, softcap)
  if (!dout || !dq || !dk || !dv || !dsum) return 1;
  const int G = Hq / Hkv;
  const int64_t nq = (int64_t)B * Sq * Hq * d, nkv = (int64_t)B * Sk * Hkv * d;
  for (int64_t x = 0; x < nq; ++x) {
    dq[x] = 0.0;
    if (dq_abs) dq_abs[x] = 0.0;
  }
  for (int64_t x = 0; x < (int64_t)B * Hq * Sq; ++x) dsum[x] = 0.0;
  for (int64_t x = 0; x < nkv; ++x) {
    dk[x] = 0.0;
    dv[x] = 0.0;
    if (dk_abs) dk_abs[x] = 0.0;
    if (dv_abs) dv_abs[x] = 0.0;
  }
  const int64_t nrows = (int64_t)G * Sq;  /* query rows of one unit */
  const int64_t rowlen = Sk > 0 ? Sk : 1;
  double *p_all = (double *)malloc(sizeof(double) * nrows * rowlen);
  double *ds_all = (double *)malloc(sizeof(double) * nrows * rowlen);
  if (!p_all || !ds_all) {
    free(p_all);
    free(ds_all);
    return 5;
  }
  for (int u = 0; u < B * Hkv; ++u) {
    if (units && !units[u]) continue;
    const int b = u / Hkv, hk = u % Hkv;
    /* step 1: P and dS rows; D; dQ = scale sum_j dS_j k_j */
    #pragma omp parallel
    {
      double *s = (double *)malloc(sizeof(double) * rowlen);
      double *o_row = (double *)malloc(sizeof(double) * d);
      #pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        const int h = hk * G + (int)(r / Sq), i = (int)(r % Sq);
        double *prob = p_all + r * rowlen, *ds = ds_all + r * rowlen;
        double lse;
        oneshot_row(&P, b, h, i, s, prob, o_row, &lse);
        /* D = sum_c dO_c O_c */
        double dsum_i = 0.0;
        for (int c = 0; c < d; ++c)
          dsum_i += elem(dout, in_bf16, q_index(&P, b, i, h, c)) * o_row[c];
        dsum[((int64_t)b * Hq + h) * Sq + i] = dsum_i;
        /* dP_j = <dO, v_j>, dS_j = P_j (dP_j - D) */
        for (int j = 0; j < Sk; ++j) {
          if (prob[j] == 0.0) {
            ds[j] = 0.0;
            continue;
          }
          double dp = 0.0;
          for (int c = 0; c < d; ++c)
            dp += elem(dout, in_bf16, q_index(&P, b, i, h, c)) *
                  elem(v, in_bf16, kv_index(&P, b, j, hk, c));
          ds[j] = prob[j] * (dp - dsum_i);
        }
        for (int c = 0; c < d; ++c) {
          double acc = 0.0, acc_abs = 0.0;
          for (int j = 0; j < Sk; ++j) {
            const double kj = elem(k, in_bf16, kv_index(&P, b, j, hk, c));
            acc += ds[j] * kj;
            acc_abs += fabs(ds[j]) * fabs(kj);
          }
          dq[q_index(&P, b, i, h, c)] = scale * acc;
          if (dq_abs) dq_abs[q_index(&P, b, i, h, c)] = scale * acc_abs;
        }
      }
      free(s);
      free(o_row);
    }
    /* step 2: dK_j = scale sum_rows dS_j q,  dV_j = sum_rows P_j dO */
    #pragma omp parallel for schedule(dynamic, 4)
    for (int j = 0; j < Sk; ++j) {
      for (int64_t r = 0; r < nrows; ++r) {
        const int h = hk * G + (int)(r / Sq), i = (int)(r % Sq);
        const double *prob = p_all + r * rowlen, *ds = ds_all + r * rowlen;
        if (prob[j] == 0.0) continue;
        for (int c = 0; c < d; ++c) {
          const int64_t x = kv_index(&P, b, j, hk, c);
          const double qc = elem(q, in_bf16, q_index(&P, b, i, h, c));
          const double doc = elem(dout, in_bf16, q_index(&P, b, i, h, c));
          dk[x] += scale * ds[j] * qc;
          dv[x] += prob[j] * doc;
          if (dk_abs) dk_abs[x] += scale * fabs(ds[j]) * fabs(qc);
          if (dv_abs) dv_abs[x] += prob[j] * fabs(doc);
        }
      }
    }
  }
  free(p_all);
  free(ds_all);
  return 0;
}

int oracle_attn_bwd(int in_bf16, const void *q, const void *k, const void *v, int B, int Sq,
                    int Sk, int Hq, int Hkv, int d, int causal, double scale, const void *dout,
                    const int *units, double *dq, double *dk, double *dv, double *dsum,
                    double *dq_abs, double *dk_abs, double *dv_abs) {
  return oracle_attn_bwd_ext(in_bf16, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, -1, -1,
                             NULL, 0.0, dout, units, dq, dk, dv, dsum, dq_abs, dk_abs,
                             dv_abs);
}

/* ---------------------------------------------------------------------------------
 * FP8 E4M3: decoding, encoding, block quantization, rotation, attention. */

static double e4m3_value(uint8_t c) {
  const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

void oracle_e4m3_decode(const uint8_t *codes, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

/* Nearest finite E4M3 value, ties to the even code (its lowest bit 0); beyond 448 the
 * nearest is 448 (saturation); NaN -> 0x7F.  A search over the 127 non-negative codes. */
static uint8_t e4m3_encode_one(float x) {
  if (isnan(x)) return 0x7F;
  const int neg = signbit(x) != 0;
  const double a = fabs((double)x);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    const double err = fabs(e4m3_value((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(best | (neg ? 0x80 : 0));
}

void oracle_e4m3_encode(const float *x, int64_t n, uint8_t *out) {
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode_one(x[i]);
}

/* In place, each of nrows rows of d floats: the Walsh-Hadamard butterflies in fp32, then
 * the fp32 product with fp32(1/sqrt(d)). */
void oracle_fwht_f32(float *rows, int64_t nrows, int d) {
  const float inv = (float)(1.0 / sqrt((double)d));
  for (int64_t r = 0; r < nrows; ++r) {
    float *y = rows + r * d;
    for (int h = 1; h < d; h *= 2)
      for (int i = 0; i < d; ++i)
        if ((i & h) == 0) {
          const float a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
    for (int i = 0; i < d; ++i) y[i] = y[i] * inv;
  }
}

/* x [B, S, H, d] (bf16 bits if in_bf16, else floats) -> codes [B, S, H, d] and scales
 * [B, H, ceil(S / 128)].  rotate: apply oracle_fwht_f32 to every row first.  d must be a
 * power of two when rotating. */
int oracle_quantize_fp8(int in_bf16, const void *x, int B, int S, int H, int d, int rotate,
                        uint8_t *codes, float *scales) {
  if (!x || !codes || !scales) return 1;
  if (B < 1 || S < 1 || H < 1 || d < 1) return 2;
  if (rotate && (d & (d - 1))) return 3;
  const int nblk = (S + 127) / 128;
  #pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < (int64_t)B * H * nblk; ++u) {
    const int b = (int)(u / ((int64_t)H * nblk)), h = (int)((u / nblk) % H);
    const int blk = (int)(u % nblk);
    const int r0 = blk * 128, r1 = r0 + 128 < S ? r0 + 128 : S;
    float *y = (float *)malloc(sizeof(float) * (size_t)(r1 - r0) * d);
    for (int r = r0; r < r1; ++r)
      for (int c = 0; c < d; ++c) {
        const int64_t idx = (((int64_t)b * S + r) * H + h) * d + c;
        y[(int64_t)(r - r0) * d + c] =
            in_bf16 ? (float)elem(x, 1, idx) : ((const float *)x)[idx];
      }
    if (rotate) oracle_fwht_f32(y, r1 - r0, d);
    float amax = 0.f;
    for (int64_t i = 0; i < (int64_t)(r1 - r0) * d; ++i)
      if (fabsf(y[i]) > amax) amax = fabsf(y[i]);
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[((int64_t)b * H + h) * nblk + blk] = sc;
    for (int r = r0; r < r1; ++r)
      for (int c = 0; c < d; ++c) {
        const int64_t idx = (((int64_t)b * S + r) * H + h) * d + c;
        codes[idx] = e4m3_encode_one(y[(int64_t)(r - r0) * d + c] / sc);
      }
    free(y);
  }
  return 0;
}

/* Dequantized tensor: code * scale of its (b, h, 128-row block), as doubles. */
static double *dequantize(const uint8_t *codes, const float *scales, int B, int S, int H,
                          int d) {
  const int nblk = (S + 127) / 128;
  double *out = (double *)malloc(sizeof(double) * (size_t)B * S * H * d);
  for (int b = 0; b < B; ++b)
    for (int r = 0; r < S; ++r)
      for (int h = 0; h < H; ++h)
        for (int c = 0; c < d; ++c) {
          const int64_t idx = (((int64_t)b * S + r) * H + h) * d + c;
          out[idx] = e4m3_value(codes[idx]) * (double)scales[((int64_t)b * H + h) * nblk + r / 128];
        }
  return out;
}

/* The FP8 forward: the plain definition on the dequantized q, k, v.  o, lse as for
 * oracle_attn_fwd.  If o_abs and inv_l are non-NULL they receive, per row, the sums
 * o_abs[c] = sum_j P_j |v_jc| ([B, Sq, Hq, d]) and 1 / l with l = sum_j exp(s_j - max s)
 * ([B, Hq, Sq], 0 for a row without keys), from which the GPU error bound is derived. */
int oracle_attn_fwd_fp8(const uint8_t *q8, const uint8_t *k8, const uint8_t *v8,
                        const float *q_scale, const float *k_scale, const float *v_scale,
                        int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                        double scale, double *o, double *lse, double *o_abs, double *inv_l) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return 1;
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || d < 1) return 2;
  if (Hq % Hkv) return 3;
  double *q = dequantize(q8, q_scale, B, Sq, Hq, d);
  double *k = dequantize(k8, k_scale, B, Sk, Hkv, d);
  double *v = dequantize(v8, v_scale, B, Sk, Hkv, d);
  int rc = oracle_attn_fwd(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, o, lse);
  if (rc == 0 && o_abs && inv_l) {
    const int in_bf16 = 0;
    SETUP_PROBLEM
    (void)err;
    const int64_t nrows = (int64_t)B * Hq * Sq;
    #pragma omp parallel
    {
      double *srow = (double *)malloc(sizeof(double) * Sk);
      double *prob = (double *)malloc(sizeof(double) * Sk);
      #pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < nrows; ++r) {
        const int b = (int)(r / ((int64_t)Hq * Sq)), h = (int)((r / Sq) % Hq), i = (int)(r % Sq);
        double m, l;
        const int nvis = prob_row(&P, b, h, i, srow, prob, &m, &l);
        inv_l[((int64_t)b * Hq + h) * Sq + i] = nvis ? 1.0 / l : 0.0;
        const int hk = kv_head(&P, h);
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int j = 0; j < Sk; ++j) acc += prob[j] * fabs(v[kv_index(&P, b, j, hk, c)]);
          o_abs[q_index(&P, b, i, h, c)] = acc;
        }
      }
      free(srow);
      free(prob);
    }
  }
  free(q);
  free(k);
  free(v);
  return rc;
}
