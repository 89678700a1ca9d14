// attn_kvcache_append: new keys and values written into a key/value cache.
#pragma once
#include "device.h"

namespace ff {

// Writes new keys and values into a key/value cache laid out as for the CACHE split
// kernel: row t of batch b goes to logical position cache_seqlens[b] + t ("03 forward
// CUDA kernel", section 8: new tokens are appended to the cache in place before the
// attention reads it).  Positions past the cache's capacity are dropped.  One thread per
// 16-byte chunk of a (batch, new row, kv head) row, K and V both.
struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int* seqlens;
  const int* block_table;
  int B, S_new, Hkv, num_blocks, page, max_blocks;
  int64_t chunks;  // B * S_new * Hkv * D / 8
};

template <int D>
__global__ __launch_bounds__(256) void attn_kvcache_append(AppendParams p) {
  constexpr int CPR = D / 8;  // 16-byte chunks per head row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.chunks) return;
  const int c = (int)(i % CPR);
  int64_t r = i / CPR;
  const int h = (int)(r % p.Hkv);
  r /= p.Hkv;
  const int t = (int)(r % p.S_new);
  const int b = (int)(r / p.S_new);
  const int cap = p.max_blocks * p.page;
  int n0 = p.seqlens[b];
  n0 = n0 < 0 ? 0 : (n0 > cap ? cap : n0);
  const int pos = n0 + t;  // cap + S_new fits in an int (host check)
  if (pos >= cap) return;
  const int pg = pos / p.page;
  int blk = p.block_table ? p.block_table[(int64_t)b * p.max_blocks + pg] : b;
  blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
  const int64_t dst = (((int64_t)blk * p.page + (pos - pg * p.page)) * p.Hkv + h) * D + 8 * c;
  const int64_t src = (((int64_t)b * p.S_new + t) * p.Hkv + h) * D + 8 * c;
  st16(p.k_cache + dst, ld16(p.k_new + src));
  st16(p.v_cache + dst, ld16(p.v_new + src));
}

}  // namespace ff
