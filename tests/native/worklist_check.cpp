// Host-side check of the kernels' work lists (worklist.h).  For many shapes (unit counts,
// ranks, subs) and both dispatch modes (plain, snake), the workgroup -> item map must:
//   - be a permutation of the list (xcd_remap, work_index), also for totals that are not a
//     multiple of 8;
//   - decode every entry to a distinct (unit slot, rank, sub), idle exactly when the unit
//     slot lies past the unit count;
//   - put workgroup w (which runs on XCD w mod 8) on a unit slot of that XCD, x, x + 8, ...;
//   - in plain mode, hand each XCD its items in non-decreasing rank (heaviest first), and
//     exactly in the order of nested loops over rank, then the XCD's unit slots, then sub,
//     so the query heads of one kv head run next to each other;
//   - in snake mode, give each round of C workgroups of an XCD the same items as plain mode,
//     in reverse order every other round.
// Prints "all checks passed".
#include <stdio.h>

#include <vector>

#include "worklist.h"

namespace {

int failures = 0;

void fail(const char* what, int U, int R, int G, int snake, int w) {
  if (failures++ < 20)
    printf("FAIL %s: units %d ranks %d subs %d snake %d workgroup %d\n", what, U, R, G, snake, w);
}

void check_remap(int total) {
  std::vector<int> seen(total, 0);
  for (int w = 0; w < total; ++w) {
    const int idx = ff::xcd_remap(w, total);
    if (idx < 0 || idx >= total || seen[idx]++) fail("xcd_remap permutation", total, 0, 0, 0, w);
  }
}

void check_list(int U, int R, int G, int snake) {
  const int u_per = (U + ff::kXcds - 1) / ff::kXcds;
  const int total = ff::kXcds * u_per * R * G;
  std::vector<int> seen_idx(total, 0), seen_item(total, 0);
  std::vector<int> last_rank(ff::kXcds, -1), pos(ff::kXcds, 0);
  for (int w = 0; w < total; ++w) {
    const int idx = ff::work_index(w, total, snake);
    if (idx < 0 || idx >= total || seen_idx[idx]++) {
      fail("work_index permutation", U, R, G, snake, w);
      continue;
    }
    const ff::UnitItem it = ff::unit_item(idx, u_per, R, G);
    if (it.unit < 0 || it.unit >= ff::kXcds * u_per || it.rank < 0 || it.rank >= R ||
        it.sub < 0 || it.sub >= G) {
      fail("item range", U, R, G, snake, w);
      continue;
    }
    const int key = (it.unit * R + it.rank) * G + it.sub;
    if (seen_item[key]++) fail("item decoded twice", U, R, G, snake, w);
    if (it.unit % ff::kXcds != w % ff::kXcds) fail("unit slot of another XCD", U, R, G, snake, w);
    if (!snake) {
      const int x = w % ff::kXcds;
      if (it.rank < last_rank[x]) fail("rank order within an XCD", U, R, G, snake, w);
      last_rank[x] = it.rank;
      // the pos[x]-th item of XCD x in nested-loop order (rank, unit slot, sub)
      int n = pos[x]++, want_rank = -1, want_unit = -1, want_sub = -1;
      for (int r = 0; r < R && want_rank < 0; ++r)
        for (int s = 0; s < u_per && want_rank < 0; ++s)
          for (int g = 0; g < G; ++g)
            if (n-- == 0) {
              want_rank = r, want_unit = x + ff::kXcds * s, want_sub = g;
              break;
            }
      if (it.rank != want_rank || it.unit != want_unit || it.sub != want_sub)
        fail("nested order within an XCD", U, R, G, snake, w);
    } else {
      // the same round of the plain order, mirrored in odd rounds
      const int k = w / ff::kXcds, round = k / snake, j = k - round * snake;
      const int len = total / ff::kXcds;
      const int m = len - round * snake < snake ? len - round * snake : snake;
      const int kp = (round & 1) ? round * snake + (m - 1 - j) : k;
      if (idx != ff::work_index(w % ff::kXcds + ff::kXcds * kp, total, 0))
        fail("snake round", U, R, G, snake, w);
    }
  }
  // every item of every unit slot appears once; idle slots are exactly those >= U
  int real = 0;
  for (int u = 0; u < ff::kXcds * u_per; ++u)
    for (int r = 0; r < R; ++r)
      for (int g = 0; g < G; ++g)
        if (seen_item[(u * R + r) * G + g] != 1) fail("item missing", U, R, G, snake, u);
        else if (u < U) ++real;
  if (real != U * R * G) fail("real item count", U, R, G, snake, -1);
}

}  // namespace

int main() {
  for (int total = 1; total <= 300; ++total) check_remap(total);
  const int subs[] = {1, 2, 4, 8};
  for (int U = 1; U <= 41; ++U)
    for (int R = 1; R <= 34; R += (R < 5 ? 1 : 7))
      for (int G : subs) {
        check_list(U, R, G, 0);
        for (int C : {1, 3, 32})  // CUs per XCD in snake mode
          check_list(U, R, G, C);
      }
  // the workloads' shapes: causal_prefill (64 units, 32 tiles, G 1), long_causal_gqa
  // (8 units, 128 tiles, G 4), the backward's key blocks (64 units, 32 blocks)
  check_list(64, 32, 1, 0);
  check_list(8, 128, 4, 0);
  check_list(16, 40, 1, 32);
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("all checks passed\n");
  return 0;
}
