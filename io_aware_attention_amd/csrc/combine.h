// attn_splitkv_combine: the LSE-weighted combine of the split-KV partials ("03 forward
// CUDA kernel", section 7.3): with L = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - L) O_s.
// Splits with LSE_s = -inf weigh nothing; when every split is empty the row gets O = 0
// and LSE = -inf.
#pragma once
#include "device.h"

namespace ff {

struct CombineParams {
  const float* o_accum;
  const float* lse_accum;
  float* o;
  float* lse;
  int B, Sq, Hq, num_splits;
  int rows;  // B * Hq * Sq
};

// One wavefront per (batch, head, query) row; lanes cover the head dimension.  Lane l
// loads the LSE of splits l and l + 64 (the host allows at most 128 splits), so every
// LSE load is in flight at once; the maximum and the sum are wavefront reductions, and
// the weight of split s is read from its lane.  The partial outputs are read four splits
// at a time.
template <int D>
__global__ __launch_bounds__(256) void attn_splitkv_combine(CombineParams p) {
  constexpr int DPL = D / 64;  // dcols per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= p.rows) return;
  const int64_t split_stride = (int64_t)p.rows;
  const int S = p.num_splits;
  const float la = lane < S ? p.lse_accum[lane * split_stride + row] : -INFINITY;
  const float lb = lane + 64 < S ? p.lse_accum[(lane + 64) * split_stride + row] : -INFINITY;
  float M = vmax(la, lb);
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) M = vmax(M, __shfl_xor(M, x));
  const int i = row % p.Sq;
  const int bh = row / p.Sq;
  const int h = bh % p.Hq, b = bh / p.Hq;
  float* orow = p.o + (((int64_t)b * p.Sq + i) * p.Hq + h) * D + lane * DPL;
  if (M == -INFINITY) {  // every split empty: no visible key
#pragma unroll
    for (int c = 0; c < DPL; ++c) orow[c] = 0.f;
    if (lane == 0) p.lse[row] = -INFINITY;
    return;
  }
  // exp2 of -inf is 0: empty splits weigh nothing
  float sum = fast_exp2((la - M) * kLog2e) + fast_exp2((lb - M) * kLog2e);
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) sum += __shfl_xor(sum, x);
  const float L = M + fast_log2(sum) * kLn2;
  const float wa = fast_exp2((la - L) * kLog2e);
  const float wb = fast_exp2((lb - L) * kLog2e);
  auto weight = [&](int s) {  // s is wave-uniform
    const float w = s < 64 ? wa : wb;
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s & 63));
  };
  const float* src = p.o_accum + (int64_t)row * D + lane * DPL;
  const int64_t sstep = split_stride * D;
  float acc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = 0.f;
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float v[4][DPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < DPL; ++c) v[u][c] = src[(s + u) * sstep + c];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = weight(s + u);
#pragma unroll
      for (int c = 0; c < DPL; ++c) acc[c] += w * v[u][c];
    }
  }
  for (; s < S; ++s) {
    const float w = weight(s);
#pragma unroll
    for (int c = 0; c < DPL; ++c) acc[c] += w * src[s * sstep + c];
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c) orow[c] = acc[c];
  if (lane == 0) p.lse[row] = L;
}

}  // namespace ff
