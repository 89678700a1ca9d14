/* Runs the C oracle's entry points on small problems, edge cases included, so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer sees every code path touch
 * memory: rows with no visible key (Sq > Sk, causal), one key, splits left empty, the
 * window and ALiBi options, the backward, FP8 quantization with and without the
 * rotation, and the FP8 attention.  It also checks the invariants that tie the paths
 * together (one-shot = online = split within 1e-12) and exits non-zero on a mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn_fwd_ext(int, const void *, const void *, const void *, int, int, int, int, int,
                        int, int, double, int, int, const double *, double, double *, double *);
int oracle_attn_rows_ext(int, const void *, const void *, const void *, int, int, int, int, int,
                         int, int, double, int, int, const double *, double, int, const int *,
                         double *, double *);
int oracle_attn_probs_ext(int, const void *, const void *, const void *, int, int, int, int,
                          int, int, int, double, int, int, const double *, double, int, int,
                          int, double *);
int oracle_attn_online_ext(int, const void *, const void *, const void *, int, int, int, int,
                           int, int, int, double, int, int, const double *, double, int,
                           double *, double *);
int oracle_attn_split_ext(int, const void *, const void *, const void *, int, int, int, int,
                          int, int, int, double, int, int, const double *, double, int, int,
                          double *, double *, double *, double *);
int oracle_attn_bwd_ext(int, const void *, const void *, const void *, int, int, int, int, int,
                        int, int, double, int, int, const double *, double, const void *,
                        const int *, double *, double *, double *, double *, double *, double *,
                        double *);
int oracle_quantize_fp8(int, const void *, int, int, int, int, int, uint8_t *, float *);
int oracle_attn_fwd_fp8(const uint8_t *, const uint8_t *, const uint8_t *, const float *,
                        const float *, const float *, int, int, int, int, int, int, int, double,
                        double *, double *, double *, double *);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(state >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}
static double *random_array(int64_t n) {
  double *a = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) a[i] = uniform();
  return a;
}
static int failures = 0;
static void expect(int cond, const char *what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}
static double maxdiff(const double *a, const double *b, int64_t n) {
  double m = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    if (isinf(a[i]) || isinf(b[i])) {
      if (a[i] != b[i]) return INFINITY;
      continue;
    }
    double e = fabs(a[i] - b[i]);
    if (!(e <= m)) m = e;
  }
  return m;
}

static void forward_case(int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal, int wl,
                         int wr, int alibi) {
  double *q = random_array((int64_t)B * Sq * Hq * d), *k = random_array((int64_t)B * Sk * Hkv * d),
         *v = random_array((int64_t)B * Sk * Hkv * d), *sl = random_array((int64_t)B * Hq);
  const double *slopes = alibi ? sl : NULL;
  int64_t no = (int64_t)B * Sq * Hq * d, nl = (int64_t)B * Hq * Sq;
  double *o = malloc(sizeof(double) * no), *lse = malloc(sizeof(double) * nl);
  double *o2 = malloc(sizeof(double) * no), *lse2 = malloc(sizeof(double) * nl);
  double scale = 1.0 / sqrt((double)d);
  expect(!oracle_attn_fwd_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr, slopes,
                              0.0, o, lse), "fwd");
  for (int blk = 1; blk <= Sk + 1; blk += 3) {
    expect(!oracle_attn_online_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr,
                                   slopes, 0.0, blk, o2, lse2), "online");
    expect(maxdiff(o, o2, no) < 1e-12 && maxdiff(lse, lse2, nl) < 1e-12, "online = one-shot");
  }
  for (int S = 1; S <= 5; ++S) {
    double *op = malloc(sizeof(double) * S * no), *lp = malloc(sizeof(double) * S * nl);
    expect(!oracle_attn_split_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr,
                                  slopes, 0.0, 4, S, op, lp, o2, lse2), "split");
    expect(maxdiff(o, o2, no) < 1e-12 && maxdiff(lse, lse2, nl) < 1e-12, "split = one-shot");
    free(op);
    free(lp);
  }
  int rows[3 * 3] = {0, 0, 0, B - 1, Hq - 1, Sq - 1, 0, Hq - 1, Sq / 2};
  double orow[3 * 128], lrow[3], prob[4096];
  expect(!oracle_attn_rows_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr,
                               slopes, 0.0, 3, rows, orow, lrow), "rows");
  expect(!oracle_attn_probs_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr,
                                slopes, 0.0, B - 1, Hq - 1, Sq - 1, prob), "probs");
  double *dout = random_array(no);
  double *dq = malloc(sizeof(double) * no), *dqa = malloc(sizeof(double) * no);
  int64_t nkv = (int64_t)B * Sk * Hkv * d;
  double *dk = malloc(sizeof(double) * nkv), *dv = malloc(sizeof(double) * nkv);
  double *dka = malloc(sizeof(double) * nkv), *dva = malloc(sizeof(double) * nkv);
  double *dsum = malloc(sizeof(double) * nl);
  expect(!oracle_attn_bwd_ext(0, q, k, v, B, Sq, Sk, Hq, Hkv, d, causal, scale, wl, wr, slopes,
                              0.0, dout, NULL, dq, dk, dv, dsum, dqa, dka, dva), "bwd");
  free(q); free(k); free(v); free(sl); free(o); free(lse); free(o2); free(lse2);
  free(dout); free(dq); free(dqa); free(dk); free(dv); free(dka); free(dva); free(dsum);
}

static void fp8_case(int B, int Sq, int Sk, int H, int d, int causal) {
  int64_t nq = (int64_t)B * Sq * H * d, nk = (int64_t)B * Sk * H * d;
  double *q = random_array(nq), *k = random_array(nk), *v = random_array(nk);
  uint8_t *q8 = malloc(nq), *k8 = malloc(nk), *v8 = malloc(nk);
  float *qs = malloc(sizeof(float) * B * H * ((Sq + 127) / 128));
  float *ks = malloc(sizeof(float) * B * H * ((Sk + 127) / 128));
  float *vs = malloc(sizeof(float) * B * H * ((Sk + 127) / 128));
  expect(!oracle_quantize_fp8(0, q, B, Sq, H, d, 1, q8, qs), "quantize q");
  expect(!oracle_quantize_fp8(0, k, B, Sk, H, d, 1, k8, ks), "quantize k");
  expect(!oracle_quantize_fp8(0, v, B, Sk, H, d, 0, v8, vs), "quantize v");
  double *o = malloc(sizeof(double) * nq), *oa = malloc(sizeof(double) * nq);
  double *lse = malloc(sizeof(double) * B * H * Sq), *il = malloc(sizeof(double) * B * H * Sq);
  expect(!oracle_attn_fwd_fp8(q8, k8, v8, qs, ks, vs, B, Sq, Sk, H, H, d, causal,
                              1.0 / sqrt((double)d), o, lse, oa, il), "fp8 attention");
  free(q); free(k); free(v); free(q8); free(k8); free(v8); free(qs); free(ks); free(vs);
  free(o); free(oa); free(lse); free(il);
}

int main(void) {
  forward_case(2, 9, 9, 4, 2, 8, 1, -1, -1, 0);
  forward_case(1, 13, 5, 2, 1, 16, 1, -1, -1, 0);   /* rows with no visible key */
  forward_case(1, 3, 17, 2, 2, 8, 0, 2, 1, 1);      /* window and ALiBi */
  forward_case(2, 6, 1, 2, 1, 4, 0, -1, -1, 0);     /* one key */
  forward_case(1, 7, 20, 2, 1, 8, 1, 3, 0, 1);      /* keys no query sees */
  fp8_case(1, 130, 200, 2, 64, 1);
  fp8_case(2, 5, 129, 1, 128, 0);
  if (failures) return 1;
  printf("oracle driver: all checks passed\n");
  return 0;
}
