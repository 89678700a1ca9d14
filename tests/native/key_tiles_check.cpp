// Host-side check of the prefill kernel's key-tile range (key_tiles in tiles.h) against
// two independent formulations of which keys a query tile sees: an element-by-element
// visibility scan (small shapes) and per-row visible intervals in 64-bit arithmetic
// (shapes whose windows and positions reach past 2^31).  Prints "all checks passed".
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "tiles.h"

namespace {

constexpr int BM = 128, BN = 64;
int failures = 0;

// Visible keys of query row i: the interval [lo, hi] (empty when lo > hi).  diag = i + Sk -
// Sq; keys j < Sk, j <= diag when causal, diag - wl <= j <= diag + wr (-1: no limit).
void row_interval(int64_t i, int64_t Sq, int64_t Sk, bool causal, int64_t wl, int64_t wr,
                  int64_t* lo, int64_t* hi) {
  const int64_t diag = i + Sk - Sq;
  int64_t a = 0, b = Sk - 1;
  if (causal) b = std::min(b, diag);
  if (wr >= 0) b = std::min(b, diag + wr);
  if (wl >= 0) a = std::max(a, diag - wl);
  *lo = a;
  *hi = b;
}

bool visible(int64_t i, int64_t j, int64_t Sq, int64_t Sk, bool causal, int64_t wl, int64_t wr) {
  const int64_t diag = i + Sk - Sq;
  if (j < 0 || j >= Sk) return false;
  if (causal && j > diag) return false;
  if (wr >= 0 && j > diag + wr) return false;
  if (wl >= 0 && j < diag - wl) return false;
  return true;
}

template <bool CAUSAL, bool WIN>
ff::KeyTiles call(int q0, int Sq, int Sk, int wl, int wr) {
  return ff::key_tiles<BM, BN, CAUSAL, WIN>(q0, Sq, Sk, wl, wr);
}

ff::KeyTiles dispatch(bool causal, bool win, int q0, int Sq, int Sk, int wl, int wr) {
  if (causal) return win ? call<true, true>(q0, Sq, Sk, wl, wr) : call<true, false>(q0, Sq, Sk, -1, -1);
  return win ? call<false, true>(q0, Sq, Sk, wl, wr) : call<false, false>(q0, Sq, Sk, -1, -1);
}

void fail(const char* what, int q0, int Sq, int Sk, bool causal, int wl, int wr, int t,
          const ff::KeyTiles& k) {
  if (++failures <= 20)
    printf("FAIL %s: q0=%d Sq=%d Sk=%d causal=%d wl=%d wr=%d tile=%d -> n_min=%d n_bot=%d "
           "n_mask_lo=%d n_max=%d\n", what, q0, Sq, Sk, (int)causal, wl, wr, t, k.n_min,
           k.n_bot, k.n_mask_lo, k.n_max);
}

// Per tile of query tile q0: whether some row sees a key of it (any) and whether the
// tile holds a (row, key) pair that must be masked, key positions >= Sk included (mask).
// The interval form: a row's visible keys are [lo, hi], so tile [t0, t0 + BN) has a
// visible key iff the intervals meet, and every key of it is visible iff [t0, t0 + BN)
// lies inside [lo, hi].
void tiles_by_intervals(int q0, int Sq, int Sk, bool causal, int wl, int wr, int64_t t_lo,
                        int64_t t_hi, std::vector<char>& any, std::vector<char>& mask) {
  const int64_t rows_end = std::min<int64_t>((int64_t)q0 + BM, Sq);
  any.assign(t_hi - t_lo, 0);
  mask.assign(t_hi - t_lo, 0);
  for (int64_t i = q0; i < rows_end; ++i) {
    int64_t lo, hi;
    row_interval(i, Sq, Sk, causal, wl, wr, &lo, &hi);
    for (int64_t t = t_lo; t < t_hi; ++t) {
      const int64_t a = t * BN, b = a + BN - 1;
      if (lo <= hi && a <= hi && b >= lo) any[t - t_lo] = 1;
      if (!(lo <= a && b <= hi)) mask[t - t_lo] = 1;
    }
  }
}

void check_shape(bool causal, bool win, int Sq, int Sk, int wl, int wr, bool brute) {
  if (!win) wl = wr = -1;
  const int nb_total = (Sk + BN - 1) / BN;
  const int num_m = (Sq + BM - 1) / BM;
  for (int m = 0; m < num_m; ++m) {
    const int q0 = m * BM;
    const ff::KeyTiles k = dispatch(causal, win, q0, Sq, Sk, wl, wr);
    std::vector<char> any, mask;
    tiles_by_intervals(q0, Sq, Sk, causal, wl, wr, 0, nb_total, any, mask);
    if (brute) {  // the element scan must agree with the interval form
      const int rows_end = std::min(q0 + BM, Sq);
      for (int t = 0; t < nb_total; ++t) {
        bool a = false, msk = false;
        for (int i = q0; i < rows_end; ++i)
          for (int j = t * BN; j < t * BN + BN; ++j) {
            const bool v = visible(i, j, Sq, Sk, causal, wl, wr);
            a = a || v;
            msk = msk || !v;
          }
        if (a != (bool)any[t] || msk != (bool)mask[t]) fail("scan vs intervals", q0, Sq, Sk, causal, wl, wr, t, k);
      }
    }
    int first = -1, last = -1;
    for (int t = 0; t < nb_total; ++t)
      if (any[t]) {
        if (first < 0) first = t;
        last = t;
      }
    if (first < 0) {
      if (k.n_max > k.n_min) fail("visits tiles although no key is visible", q0, Sq, Sk, causal, wl, wr, -1, k);
      continue;
    }
    // the range is exactly the tiles from the first to the last with a visible key
    if (k.n_min != first) fail("n_min", q0, Sq, Sk, causal, wl, wr, first, k);
    if (k.n_max != last + 1) fail("n_max", q0, Sq, Sk, causal, wl, wr, last, k);
    if (k.n_bot < k.n_min || k.n_bot > k.n_max) fail("n_bot outside range", q0, Sq, Sk, causal, wl, wr, -1, k);
    for (int t = k.n_min; t < k.n_max; ++t)
      if (mask[t] && !(t >= k.n_mask_lo || t < k.n_bot))
        fail("tile needing a mask runs unmasked", q0, Sq, Sk, causal, wl, wr, t, k);
  }
}

// Shapes whose positions need 64 bits in the window arithmetic: only a few query tiles
// and the tiles around each row interval are examined.
void check_large(bool causal, int Sq, int Sk, int wl, int wr) {
  const int num_m = (Sq + BM - 1) / BM;
  const int ms[4] = {0, num_m / 2, num_m - 2, num_m - 1};
  for (int m : ms) {
    if (m < 0) continue;
    const int q0 = m * BM;
    const ff::KeyTiles k = dispatch(causal, true, q0, Sq, Sk, wl, wr);
    // visible span of the whole query tile
    int64_t lo_all = INT64_MAX, hi_all = INT64_MIN;
    const int64_t rows_end = std::min<int64_t>((int64_t)q0 + BM, Sq);
    for (int64_t i = q0; i < rows_end; ++i) {
      int64_t lo, hi;
      row_interval(i, Sq, Sk, causal, wl, wr, &lo, &hi);
      if (lo > hi) continue;
      lo_all = std::min(lo_all, lo);
      hi_all = std::max(hi_all, hi);
    }
    if (lo_all > hi_all) {
      if (k.n_max > k.n_min) fail("large: visits tiles although no key is visible", q0, Sq, Sk, causal, wl, wr, -1, k);
      continue;
    }
    if (k.n_min != lo_all / BN) fail("large: n_min", q0, Sq, Sk, causal, wl, wr, -1, k);
    if (k.n_max != hi_all / BN + 1) fail("large: n_max", q0, Sq, Sk, causal, wl, wr, -1, k);
    // masks near both ends of the range
    const int64_t n_lo = k.n_min, n_hi = k.n_max;
    for (int64_t base : {n_lo, std::max(n_lo, n_hi - 4)}) {
      const int64_t e = std::min(n_hi, base + 4);
      std::vector<char> any, mask;
      tiles_by_intervals(q0, Sq, Sk, causal, wl, wr, base, e, any, mask);
      for (int64_t t = base; t < e; ++t)
        if (mask[t - base] && !(t >= k.n_mask_lo || t < k.n_bot))
          fail("large: tile needing a mask runs unmasked", q0, Sq, Sk, causal, wl, wr, (int)t, k);
    }
  }
}

}  // namespace

int main() {
  uint64_t state = 0x9E3779B97F4A7C15ull;
  auto rnd = [&](int n) {  // xorshift64*, uniform on [0, n)
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (int)(((state * 0x2545F4914F6CDD1Dull) >> 33) % (uint64_t)n);
  };
  int shapes = 0;
  // edge sizes around the tile sizes, then random ones
  const int edge[] = {1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 255, 256, 257, 300};
  for (int causal = 0; causal < 2; ++causal)
    for (int Sq : edge)
      for (int Sk : edge) {
        check_shape(causal, false, Sq, Sk, -1, -1, true);
        ++shapes;
      }
  for (int it = 0; it < 3000; ++it) {
    const bool causal = rnd(2), win = rnd(4) != 0;
    const int Sq = 1 + rnd(420), Sk = 1 + rnd(420);
    const int wl = rnd(3) == 0 ? -1 : rnd(300), wr = rnd(3) == 0 ? -1 : rnd(300);
    check_shape(causal, win, Sq, Sk, wl, wr, it < 1500);
    ++shapes;
  }
  // long sequences and windows (positions and limits past 2^31 in the window sums)
  const int big = 2000000000;
  const int large[][4] = {{4096, big, big, big}, {big / 4, big, 0, big}, {300, big, 5, 7},
                          {big, big, big, 0}, {100000, 300000, 70000, 65}, {4096, 4096, big, -1}};
  for (auto& c : large)
    for (int causal = 0; causal < 2; ++causal) {
      check_large(causal, c[0], c[1], c[2], c[3]);
      ++shapes;
    }
  if (failures) {
    printf("%d failures over %d shapes\n", failures, shapes);
    return 1;
  }
  printf("%d shapes: all checks passed\n", shapes);
  return 0;
}
