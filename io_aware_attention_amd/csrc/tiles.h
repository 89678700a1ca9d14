// Key-tile range of one query tile of the prefill kernel: which 64-key tiles its
// workgroup visits and which of them need the element mask.  Plain integer arithmetic on
// wave-uniform values, callable from the kernel and from host code (the host-side unit
// test checks it against a brute-force visibility scan).
//
// The walk-through of the forward kernel ("03 · 前向 CUDA kernel", §5 on masking) clips
// the key loop at the causal diagonal, so tiles above it are never visited, and runs the
// few tiles that straddle the diagonal or the key tail as masked steps before an
// unmasked main loop.  The v2 code walk-through adds the window limits, which clip the
// range at both ends (its n_block_min / n_block_max).  With diag = i + Sk - Sq, key j is
// visible to query i iff j < Sk, and (causal) j <= diag, and (window) diag - wl <= j <=
// diag + wr, a limit of -1 meaning none.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ff {

struct KeyTiles {
  int n_min;      // first tile that holds a key some row of the query tile sees
  int n_bot;      // tiles [n_min, n_bot) hold keys left of the last row's window: masked
  int n_mask_lo;  // tiles [n_mask_lo, n_max) straddle the diagonal, right limit or key tail
  int n_max;      // one past the last tile with a visible key (n_max <= n_min: none)
};

// Query rows q0 .. min(q0 + BM, Sq) - 1 against Sk keys in tiles of BN.  Every tile that
// holds a key none of the rows sees, or a key position >= Sk, lies in [n_min, n_bot) or
// [n_mask_lo, n_max); the kernel masks those tiles element by element and no other.
template <int BM, int BN, bool CAUSAL, bool WIN>
__host__ __device__ __forceinline__ KeyTiles key_tiles(int q0, int Sq, int Sk, int wl, int wr) {
  static_assert(BN > 0 && (BN & (BN - 1)) == 0, "BN must be a power of two");
  constexpr int LB = __builtin_ctz(BN);
  KeyTiles r;
  const int nb_total = (Sk + BN - 1) / BN;
  r.n_max = nb_total;
  const int last_q = (q0 + BM < Sq ? q0 + BM : Sq) - 1;
  if (CAUSAL) {
    const int lim = last_q + Sk - Sq;  // diagonal of the last row
    r.n_max = lim < 0 ? 0 : ((lim / BN + 1) < r.n_max ? lim / BN + 1 : r.n_max);
  }
  r.n_mask_lo = (Sk % BN) ? nb_total - 1 : nb_total;  // the key tail
  if (CAUSAL) {
    const int first = q0 + Sk - Sq + 1;  // first key the first row does not see
    const int tm = first <= 0 ? 0 : first / BN;
    r.n_mask_lo = tm < r.n_mask_lo ? tm : r.n_mask_lo;
  }
  r.n_min = 0;
  r.n_bot = 0;
  if (WIN) {
    // 64-bit positions (a window may reach past 2^31); tile numbers by shifts of
    // non-negative values, which stay scalar
    if (wr >= 0) {
      const int64_t lim = (int64_t)last_q + Sk - Sq + wr;  // right limit of the last row
      const int64_t nm = lim < 0 ? 0 : (lim >> LB) + 1;
      r.n_max = nm < r.n_max ? (int)nm : r.n_max;
      const int64_t first = (int64_t)q0 + Sk - Sq + wr + 1;  // first key row q0 misses
      const int64_t tm = first <= 0 ? 0 : first >> LB;
      r.n_mask_lo = tm < r.n_mask_lo ? (int)tm : r.n_mask_lo;
    }
    if (wl >= 0) {
      const int64_t lo_first = (int64_t)q0 + Sk - Sq - wl;     // left limit of row q0
      const int64_t lo_last = (int64_t)last_q + Sk - Sq - wl;  // left limit of the last row
      r.n_min = lo_first <= 0 ? 0 : (int)(lo_first >> LB);
      const int64_t nb = lo_last <= 0 ? 0 : (lo_last + BN - 1) >> LB;
      r.n_bot = (int)(nb < r.n_max ? nb : r.n_max);
      r.n_bot = r.n_bot > r.n_min ? r.n_bot : r.n_min;
    }
  }
  return r;
}

}  // namespace ff
