// attn_fwd_prefill: the fused forward kernel for gfx950.
//
// One workgroup (4 wavefronts, 256 threads) owns one (query tile of BM = 128
// rows, batch, query head): the Q tile stays in registers while key/value
// tiles of BN = 64 rows stream through double-buffered LDS, highest tile
// first ("03 forward CUDA kernel", sections 2-5; the walk-through's
// compute_attn_1rowblock description).  Each wavefront owns 32 query rows and
// never merges with the others (the explainer's FA2 split-Q section).
//
// Data movement.  K and V tiles go from HBM straight into LDS with buffer
// loads (no register staging); the buffer descriptor of each tile ends at key
// Sk, so rows past the key tail read as zero.  Both tiles are stored
// row-major with the 16-byte chunks of each row XOR-swizzled, so that the
// 128-bit reads of K (GEMM0) and the transposing reads of V (GEMM1,
// ds_read_b64_tr_b16) each touch every LDS bank the minimum number of times.
//
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form:
//   GEMM0  S^T (keys x queries) = K . Q^T      A = K rows from LDS, B = Q^T in VGPRs
//   GEMM1  O^T (dcols x queries) += V^T . P^T  A = V^T via LDS transpose reads, B = P^T
// The GEMM0 output leaves every lane with 32 scores of ONE query, so the row
// max needs a single cross-lane step (lanes l and l^32) and the row sum none
// until the epilogue.  The key rows fed to GEMM0 are permuted (bits 2 and 3
// of the row index swapped) so that the score registers already are the
// GEMM1 B operand: eight consecutive keys per lane, no shuffles.
//
// Softmax runs in base 2 with the scale folded into one FMA (e^x = 2^(x log2 e))
// and the state (m, l, o) of the explainer's online-softmax section, the
// normalisation deferred to the epilogue (FA2).  The reference point m is
// raised only when a tile's maximum exceeds it by more than kRescaleSlack
// (base-2 units); numerator and denominator always share it, so the result is
// the same up to rounding (the explainer's rescaling-invariance argument) while
// the O rescale is skipped for almost every tile.
#pragma once
#include "device.h"

namespace ff {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv, G;  // G = Hq / Hkv
  int num_m;                  // query tiles per (batch, head)
  int total;                  // num_m * B * Hq workgroups
  float scale_log2;           // scale * log2(e)
};

// Exponents stay within 2^kRescaleSlack of the stored reference point.
constexpr float kRescaleSlack = 8.0f;

// The hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Give
// each XCD one contiguous run of the work list so the workgroups sharing a
// key/value head also share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  constexpr int kXcd = 8;
  const int x = w % kXcd, k = w / kXcd;
  const int q = total / kXcd, r = total % kXcd;
  return x * q + (x < r ? x : r) + k;
}

template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct PrefillTraits {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int kThreads = 256;
  static constexpr int ROWB = D * 2;               // bytes per K/V row in LDS
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;           // bytes per K or V tile
  static constexpr int kLds = 2 * 2 * TILE;        // K and V, double buffered
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte bank line
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tile
  // swizzle keys: physical chunk = logical chunk ^ key(row)
  static __device__ __forceinline__ int kkey(int r) { return (r / RPB) % CPR; }
  static __device__ __forceinline__ int vkey(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_prefill(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource builtins exist for the device target only
  using T = PrefillTraits<D>;
  constexpr int BM = T::BM, BN = T::BN, ROWB = T::ROWB, CPR = T::CPR, TILE = T::TILE;
  constexpr int LOADS = T::LOADS;
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds];

  // ---- which (batch, head, query tile) this workgroup owns
  const int idx = xcd_remap(blockIdx.x, p.total);
  const int hg = idx % p.G;
  const int t1 = idx / p.G;
  const int mi = t1 % p.num_m;
  const int t2 = t1 / p.num_m;
  const int hk = t2 % p.Hkv;
  const int b = t2 / p.Hkv;
  const int h = hk * p.G + hg;
  const int mblk = CAUSAL ? p.num_m - 1 - mi : mi;  // heaviest causal tiles first
  const int q0 = mblk * BM;
  const int Sq = p.Sq, Sk = p.Sk;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query column of this lane in both products
  const int H = lane >> 5;   // which half of the wave
  const int qrow = q0 + wave * 32 + n;

  // ---- key-tile range (causal clipping: never visit tiles above the diagonal)
  const int nb_total = (Sk + BN - 1) / BN;
  int n_max = nb_total;
  const int last_q = (q0 + BM < Sq ? q0 + BM : Sq) - 1;
  if (CAUSAL) {
    const int lim = last_q + Sk - Sq;
    n_max = lim < 0 ? 0 : ((lim / BN + 1) < n_max ? lim / BN + 1 : n_max);
  }
  // Tiles [n_mask_lo, n_max) need an element mask (key tail or causal diagonal).
  int n_mask_lo = (Sk % BN) ? nb_total - 1 : nb_total;
  if (CAUSAL) {
    const int first = q0 + Sk - Sq + 1;
    const int tm = first <= 0 ? 0 : first / BN;
    n_mask_lo = tm < n_mask_lo ? tm : n_mask_lo;
  }

  const int64_t q_stride = (int64_t)p.Hq * D;    // elements between query positions
  const int kv_row_bytes = p.Hkv * D * 2;        // bytes between key positions
  const float c2 = p.scale_log2;

  if (n_max <= 0) {  // no visible key for any row of this tile
    if (qrow < Sq) {
      float* orow = p.o + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = H * 4; c < D; c += 8) st16f(orow + c, z);
      if (H == 0) p.lse[((int64_t)b * p.Hq + h) * Sq + qrow] = -INFINITY;
    }
    return;
  }

  // ---- Q^T fragments (GEMM0 B operand): Q[qrow][16c + 8H .. +7]
  u32x4 qf[D / 16];
  {
    const uint16_t* qp = p.q + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D + 8 * H;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (qrow < Sq) qf[c] = ld16(qp + 16 * c);
      else qf[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- direct HBM -> LDS loads.  Wave w, load k fills the 1 KiB LDS block
  // LOADS*w + k: lane i writes chunk slot 64*(LOADS*w + k) + i, i.e. row slot/CPR,
  // physical chunk slot%CPR, which holds logical chunk (physical ^ key(row)).
  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)b * Sk * p.Hkv + hk) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)b * Sk * p.Hkv + hk) * D * 2;
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int k = 0; k < LOADS; ++k) {
    const int slot = 64 * (LOADS * wave + k) + lane;
    const int r = slot / CPR, ph = slot % CPR;
    koff[k] = r * kv_row_bytes + 16 * (ph ^ T::kkey(r));
    voff[k] = r * kv_row_bytes + 16 * (ph ^ T::vkey(r));
  }
  auto issue_loads = [&](int t, int buf) {
    const int rows_left = Sk - t * BN;  // > 0 for every visited tile
    const uint32_t bytes = (uint32_t)rows_left * (uint32_t)kv_row_bytes;
    const int64_t toff = (int64_t)t * BN * kv_row_bytes;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + toff), 0, (int)bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + toff), 0, (int)bytes, 0x00020000);
    char* kl = smem + buf * 2 * TILE + 1024 * LOADS * wave;
    char* vl = kl + TILE;
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(kl + 1024 * k), 16, koff[k], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(vl + 1024 * k), 16, voff[k], 0, 0, 0);
    }
  };

  // ---- LDS read addresses
  // GEMM0 A operand: K row 32kb + prow (prow = n with bits 2 and 3 swapped),
  // logical chunk 2c + H.
  const int prow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
  int ka[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) ka[c] = prow * ROWB + 16 * ((2 * c + H) ^ T::kkey(prow));
  // GEMM1 A operand through ds_read_b64_tr_b16: in each 16-lane group g = lane/16,
  // source lane s points at key row R + 8(g/2) + s/4 and dcols 32db + 16(g%2) + 4(s%4);
  // the group then holds, per lane, one dcol over four consecutive keys.
  const int g = lane >> 4, s = lane & 15;
  const int vrow = 8 * (g >> 1) + (s >> 2);
  int va[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    va[db] = vrow * ROWB + 16 * ((4 * db + 2 * (g & 1) + ((s & 3) >> 1)) ^ T::vkey(vrow)) +
             8 * (s & 1);

  // ---- online-softmax state: this lane's query row, its half of the keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // reference point, scale*log2(e) units
  float l_run = 0.f;        // running sum over this lane's keys

  auto tile = [&](int t, int buf, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* kl = smem + buf * 2 * TILE;
    const char* vl = kl + TILE;
    // GEMM0: S^T for key blocks kb = 0, 1 (32 keys each)
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kl + ka[c] + kb * 32 * ROWB);
        sc[kb] = mfma32(a, qf[c], sc[kb]);
      }
    }
    // mask: element 4j+i of block kb is key t*BN + 32 kb + 16(j>>1) + 8H + 4(j&1) + i
    if constexpr (MASKED) {
      const int lim = CAUSAL ? qrow + Sk - Sq : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t * BN + 32 * kb + 16 * (j >> 1) + 8 * H + 4 * (j & 1) + i;
            if (key >= Sk || key > lim) sc[kb][4 * j + i] = -INFINITY;
          }
    }
    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = vmax(mx, sc[kb][e]);
    mx = max_xor32(mx) * c2;
    const bool raise = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform: some row raises m
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;  // 0 when m_run = -inf
      m_run = raise ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(sc[kb][e], c2, -m_use));
        sc[kb][e] = pe;
        ls += pe;
      }
    l_run += ls;
    // P^T fragments (GEMM1 B operand): elements 8c'..8c'+7 of block kb
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        pf[kb][cp] = pack8(sc[kb][8 * cp + 0], sc[kb][8 * cp + 1], sc[kb][8 * cp + 2],
                           sc[kb][8 * cp + 3], sc[kb][8 * cp + 4], sc[kb][8 * cp + 5],
                           sc[kb][8 * cp + 6], sc[kb][8 * cp + 7]);
    // GEMM1: O^T += V^T . P^T, V^T fragments by two transposing reads
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
          const char* base = vl + va[db] + (32 * kb + 16 * cp) * ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + 4 * ROWB));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
          oacc[db] = mfma32(a, pf[kb][cp], oacc[db]);
        }
  };

  // ---- main loop: tiles n_max-1 down to 0, masked suffix first
  int t = n_max - 1;
  if ((t + 1) * BN > Sk) {
    // key tail: rows past Sk must read as zeros even if the loads leave them alone
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < 2 * TILE / 16; i += T::kThreads) st16(smem + 16 * i, z);
    __syncthreads();
  }
  issue_loads(t, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile is in LDS
  __syncthreads();
  int buf = 0;
  for (; t >= 0 && t >= n_mask_lo; --t) {
    if (t > 0) issue_loads(t - 1, buf ^ 1);
    tile(t, buf, MaskTag<true>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    buf ^= 1;
  }
  for (; t >= 0; --t) {
    if (t > 0) issue_loads(t - 1, buf ^ 1);
    tile(t, buf, MaskTag<false>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: O = o / l, LSE = (m + log2 l) ln 2
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < Sq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = p.o + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 val = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                           oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
        st16f(orow + 32 * db + 8 * j + 4 * H, val);
      }
    if (H == 0)
      p.lse[((int64_t)b * p.Hq + h) * Sq + qrow] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
#endif
}

}  // namespace ff
