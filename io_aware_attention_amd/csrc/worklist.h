// Work lists of the tiled kernels (the bf16 and FP8 forward, both backward kernels): which
// item workgroup w owns.  Plain integer arithmetic, callable from the kernels and from host
// code (a host-side unit test checks that every list is a permutation with the order
// described below).
//
// Items are (unit, rank, sub): a unit is one (batch, kv head); rank orders a unit's items
// by work (the forward and dQ kernels: query tile, heaviest first when causal; dK/dV: key
// block, the heaviest first when causal); sub is the query head of the unit (the forward
// and dQ kernels, G per unit) or unused (1).  Each of the 8 XCDs holds u_per =
// ceil(units / 8) unit slots, XCD x the units x, x + 8, x + 16, ... (slots past the last
// unit are idle), so that the kv heads of one sequence spread over the XCDs and sequences
// of different length load them evenly; inside an XCD the order is rank, then unit, then
// sub, so every XCD starts its heaviest items first.  The list has 8 u_per ranks subs
// entries.
#pragma once
#include <hip/hip_runtime.h>

namespace ff {

constexpr int kXcds = 8;

// The hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Give each XCD one
// contiguous run of the work list, so that the workgroups sharing a key/value head also
// share that XCD's L2.
__host__ __device__ __forceinline__ int xcd_remap(int w, int total) {
  const int x = w % kXcds, k = w / kXcds;
  const int q = total / kXcds, r = total % kXcds;
  return x * q + (x < r ? x : r) + k;
}

// Work item of workgroup w.  A grid that is resident all at once gets no second round in
// which short items could fill in behind long ones, and the dispatcher gives the c-th
// workgroup of an XCD to CU c mod C, again and again.  With the work list heaviest
// first, CU 0 would then collect the longest item of every round.  For such grids
// (snake = C) every other round runs backwards, so a CU's long item of one round is
// followed by a short one of the next.
__host__ __device__ __forceinline__ int work_index(int w, int total, int snake) {
  if (!snake) return xcd_remap(w, total);
  const int x = w % kXcds, k = w / kXcds;
  const int q = total / kXcds, r = total % kXcds;
  const int len = q + (x < r);
  const int round = k / snake, j = k - round * snake;
  const int left = len - round * snake;
  const int m = left < snake ? left : snake;  // items in this round
  const int kk = (round & 1) ? round * snake + (m - 1 - j) : k;
  return x * q + (x < r ? x : r) + kk;
}

struct UnitItem {
  int unit;  // (batch, kv head) unit, batch-major; >= the unit count for an idle slot
  int rank;  // 0 = the unit's heaviest item
  int sub;   // query head of the unit (0 .. subs - 1)
};

// Entry idx of the work list above.
__host__ __device__ __forceinline__ UnitItem unit_item(int idx, int u_per, int ranks, int subs) {
  const int grp = u_per * subs * ranks;  // entries per XCD
  const int x = idx / grp;
  const int r0 = idx - x * grp;
  const int rank = r0 / (u_per * subs);
  const int rest = r0 - rank * u_per * subs;
  return UnitItem{(rest / subs) * kXcds + x, rank, rest % subs};
}

}  // namespace ff
