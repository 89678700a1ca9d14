// attn_fwd_prefill: the fused forward kernel for gfx950.
//
// One workgroup (4 wavefronts, 256 threads) owns one (query tile of BM = 128
// rows, batch, query head): the Q tile stays in registers while key/value
// tiles of BN = 64 rows stream through double-buffered LDS, highest tile
// first ("03 forward CUDA kernel", sections 2-5; the walk-through's
// compute_attn_1rowblock description).  Each wavefront owns 32 query rows and
// never merges with the others (the explainer's FA2 split-Q section).
//
// Both products run on v_mfma_f32_32x32x16_bf16 in transposed form:
//   GEMM0  S^T (keys x queries) = K . Q^T      A = K rows from LDS, B = Q^T in VGPRs
//   GEMM1  O^T (dcols x queries) += V^T . P^T  A = V^T rows from LDS, B = P^T in VGPRs
// The GEMM0 output leaves every lane with 32 scores of ONE query, so the row
// max needs a single cross-lane step (lanes l and l^32) and the row sum none
// until the epilogue.  The key rows fed to GEMM0 are permuted (bits 2 and 3
// of the row index swapped) so that the score registers are already the
// GEMM1 B operand: eight consecutive keys per lane, no shuffles.  V is
// transposed on its way into LDS so GEMM1's A operand is one 128-bit LDS read.
//
// Softmax runs in base 2 with the scale folded into one FMA (e^x = 2^(x log2 e));
// the state (m, l, o) follows the explainer's online-softmax section with the
// normalisation deferred to the epilogue (FA2).
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

template <int D>
struct PrefillTraits {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int kThreads = 256;
  static constexpr int KS = D * 2 + 16;            // K row stride in LDS, bytes
  static constexpr int VS = BN * 2 + 16;           // V^T row stride in LDS, bytes
  static constexpr int KBUF = BN * KS;
  static constexpr int VBUF = D * VS;
  static constexpr int kLds = 2 * (KBUF + VBUF);   // double buffered
  static constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
  static constexpr int KPT = BN * CPR / kThreads;  // K chunks per thread
  static constexpr int VKB = KPT;                  // V keys per thread block (x 8 dcols)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_prefill(FwdParams p) {
  using T = PrefillTraits<D>;
  constexpr int BM = T::BM, BN = T::BN, KS = T::KS, VS = T::VS;
  constexpr int CPR = T::CPR, KPT = T::KPT, VKB = T::VKB;
  __shared__ __attribute__((aligned(16))) char smem[T::kLds];

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

  const int64_t q_stride = (int64_t)p.Hq * D;   // elements between query positions
  const int64_t kv_stride = (int64_t)p.Hkv * D; // elements between key positions
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

  const uint16_t* kbase = p.k + (int64_t)b * Sk * kv_stride + (int64_t)hk * D;
  const uint16_t* vbase = p.v + (int64_t)b * Sk * kv_stride + (int64_t)hk * D;

  // K tile: thread chunk c = tid + 256 i -> row c / CPR, 16-byte column c % CPR.
  // V tile: thread block of VKB keys x 8 dcols: dcol group tid % CPR, key group tid / CPR.
  const int v_cg = tid % CPR;
  const int v_kg = tid / CPR;
  u32x4 kreg[KPT], vreg[VKB];

  auto load_kv = [&](int t, bool partial) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + T::kThreads * i;
      const int j = t * BN + c / CPR;
      if (!partial || j < Sk) kreg[i] = ld16(kbase + (int64_t)j * kv_stride + (c % CPR) * 8);
      else kreg[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < VKB; ++r) {
      const int j = t * BN + v_kg * VKB + r;
      if (!partial || j < Sk) vreg[r] = ld16(vbase + (int64_t)j * kv_stride + v_cg * 8);
      else vreg[r] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto store_kv = [&](int buf) {
    char* kb = smem + buf * (T::KBUF + T::VBUF);
    char* vb = kb + T::KBUF;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + T::kThreads * i;
      st16(kb + (c / CPR) * KS + (c % CPR) * 16, kreg[i]);
    }
    // transpose VKB keys x 8 dcols into V^T rows (one row per dcol)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      char* dst = vb + (v_cg * 8 + c) * VS + v_kg * VKB * 2;
      const int dw = c >> 1;
      if constexpr (VKB == 4) {
        u32x2 val;
        if (c & 1) {
          val[0] = hi_hi(vreg[0][dw], vreg[1][dw]);
          val[1] = hi_hi(vreg[2][dw], vreg[3][dw]);
        } else {
          val[0] = lo_lo(vreg[0][dw], vreg[1][dw]);
          val[1] = lo_lo(vreg[2][dw], vreg[3][dw]);
        }
        *reinterpret_cast<u32x2*>(dst) = val;
      } else {
        static_assert(VKB == 2, "V block is 2 or 4 keys");
        *reinterpret_cast<uint32_t*>(dst) =
            (c & 1) ? hi_hi(vreg[0][dw], vreg[1][dw]) : lo_lo(vreg[0][dw], vreg[1][dw]);
      }
    }
  };

  // ---- online-softmax state: this lane's query row, its half of the keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of scale*log2(e)*s
  float l_run = 0.f;        // running sum over this lane's keys

  // GEMM0 A-operand row for this lane: bits 2 and 3 of n swapped.
  const int prow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);

  auto tile = [&](int t, int buf, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* kb = smem + buf * (T::KBUF + T::VBUF);
    const char* vb = kb + T::KBUF;
    // GEMM0: S^T for key blocks kb = 0, 1 (32 keys each)
    f32x16 s[2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk) {
      s[kbk] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + (32 * kbk + prow) * KS + (16 * c + 8 * H) * 2);
        s[kbk] = mfma32(a, qf[c], s[kbk]);
      }
    }
    // mask: element 4j+i of block kbk is key t*BN + 32 kbk + 16(j>>1) + 8H + 4(j&1) + i
    if constexpr (MASKED) {
      const int lim = CAUSAL ? qrow + Sk - Sq : 0x7fffffff;
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t * BN + 32 * kbk + 16 * (j >> 1) + 8 * H + 4 * (j & 1) + i;
            if (key >= Sk || key > lim) s[kbk][4 * j + i] = -INFINITY;
          }
    }
    // online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = vmax(mx, s[kbk][e]);
    mx = max_xor32(mx);
    const float m_new = vmax(m_run, mx * c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float ls = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(s[kbk][e], c2, -m_use));
        s[kbk][e] = pe;
        ls += pe;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    // P^T fragments (GEMM1 B operand): elements 8c'..8c'+7 of block kbk
    u32x4 pf[2][2];
#pragma unroll
    for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        pf[kbk][cp] = pack8(s[kbk][8 * cp + 0], s[kbk][8 * cp + 1], s[kbk][8 * cp + 2],
                            s[kbk][8 * cp + 3], s[kbk][8 * cp + 4], s[kbk][8 * cp + 5],
                            s[kbk][8 * cp + 6], s[kbk][8 * cp + 7]);
    // GEMM1: O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
        for (int cp = 0; cp < 2; ++cp) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(vb + (32 * db + n) * VS + (32 * kbk + 16 * cp + 8 * H) * 2);
          oacc[db] = mfma32(a, pf[kbk][cp], oacc[db]);
        }
  };

  // ---- main loop: tiles n_max-1 down to 0, masked suffix first
  int t = n_max - 1;
  load_kv(t, (t + 1) * BN > Sk);
  store_kv(0);
  __syncthreads();
  int buf = 0;
  for (; t >= 0 && t >= n_mask_lo; --t) {
    if (t > 0) load_kv(t - 1, false);
    tile(t, buf, MaskTag<true>{});
    if (t > 0) store_kv(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  for (; t >= 0; --t) {
    if (t > 0) load_kv(t - 1, false);
    tile(t, buf, MaskTag<false>{});
    if (t > 0) store_kv(buf ^ 1);
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
}

}  // namespace ff
