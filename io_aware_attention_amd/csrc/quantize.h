// attn_quantize_fp8: the block quantizer of the FP8 forward ("FlashAttention 1, 2, 3"
// explainer, FlashAttention-3 precision section: a scale per block, and an orthogonal
// transform of Q and K that keeps QK^T).
//
// Format: OCP FP8 E4M3 (bias 7, subnormals, max 448), the format of
// v_mfma_f32_32x32x64_f8f6f4 and v_cvt_pk_fp8_f32 on gfx950.  A tensor [B, S, H, d] is
// held as codes of the same shape plus one fp32 scale per (b, h, block of 128 rows),
// [B, H, ceil(S / 128)]: element = code * scale.
//
// One workgroup per (b, h, 128-row block), 4 wavefronts x 32 rows.  Each lane holds
// d / 64 consecutive elements of every row it owns.  The optional rotation is the
// Walsh-Hadamard butterfly (distance 1 inside a lane at d = 128, the others across
// lanes), in fp32, then the product with fp32(1/sqrt(d)).  Then scale = amax / 448 over
// the block and code = RNE(x / scale) (IEEE division, the conversion instruction rounds
// to nearest even).
#pragma once
#include "device.h"

namespace ff {

struct QuantParams {
  const uint16_t* x;  // bf16 [B, S, H, d]
  uint8_t* codes;     // e4m3 [B, S, H, d]
  float* scales;      // [B, H, nblk]
  int B, S, H, nblk, rotate;
};

template <int D>
__global__ __launch_bounds__(256) void attn_quantize_fp8(QuantParams p) {
  constexpr int E = D / 64;    // elements per lane per row
  constexpr int RPW = 32;      // rows per wavefront
  // head innermost: consecutive workgroups read the heads of the same 128 rows, one
  // contiguous region of 128 * H * D * 2 bytes, instead of 256-byte pieces of rows
  // H * D * 2 bytes apart
  const int u = blockIdx.x;
  const int h = u % p.H;
  const int blk = (u / p.H) % p.nblk;
  const int b = u / (p.nblk * p.H);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blk * 128 + wave * RPW;
  __shared__ float wmax[4];

  // All 32 row loads are issued before any is used (rows past S read row 0 and are
  // zeroed afterwards): a load under a condition became a branch with its own wait,
  // which serialised 32 memory latencies per wavefront.
  uint32_t raw[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = r0 + r < p.S ? r0 + r : 0;
    const int64_t off = (((int64_t)b * p.S + row) * p.H + h) * D + E * lane;
    if constexpr (E == 2) raw[r] = *reinterpret_cast<const uint32_t*>(p.x + off);
    else raw[r] = p.x[off];
  }
  float y[RPW][E];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const uint32_t w = r0 + r < p.S ? raw[r] : 0u;
    float v[E];
    if constexpr (E == 2) {
      v[0] = __uint_as_float(w << 16);
      v[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      v[0] = __uint_as_float(w << 16);
    }
    if (p.rotate) {
      // butterflies of distance 1, 2, ..., D/2 over element index E * lane + k
      if constexpr (E == 2) {
        const float a = v[0], c = v[1];
        v[0] = a + c;
        v[1] = a - c;
      }
#pragma unroll
      for (int m = 1; m < 64; m *= 2) {  // distance E * m: partner lane lane ^ m
#pragma unroll
        for (int k = 0; k < E; ++k) {
          const float o = __shfl_xor(v[k], m);
          v[k] = (lane & m) ? o - v[k] : v[k] + o;
        }
      }
      constexpr float inv = D == 128 ? 0.08838834764831845f : 0.125f;  // fp32(1/sqrt(D))
#pragma unroll
      for (int k = 0; k < E; ++k) v[k] = v[k] * inv;
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
      y[r][k] = v[k];
      amax = vmax(amax, __builtin_fabsf(v[k]));
    }
  }
  // block maximum: wave reduction, then across the four waves
#pragma unroll
  for (int m = 32; m >= 1; m /= 2) amax = vmax(amax, __shfl_xor(amax, m));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = vmax(vmax(wmax[0], wmax[1]), vmax(wmax[2], wmax[3]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  if (threadIdx.x == 0) p.scales[((int64_t)b * p.H + h) * p.nblk + blk] = sc;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = r0 + r;
    if (row >= p.S) break;
    const int64_t off = (((int64_t)b * p.S + row) * p.H + h) * D + E * lane;
    if constexpr (E == 2) {
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[r][0] / sc, y[r][1] / sc, 0, false);
      *reinterpret_cast<uint16_t*>(p.codes + off) = (uint16_t)w;
    } else {
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[r][0] / sc, 0.f, 0, false);
      p.codes[off] = (uint8_t)w;
    }
  }
}

}  // namespace ff
