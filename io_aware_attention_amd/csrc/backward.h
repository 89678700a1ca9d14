// attn_bwd: the backward pass of the fused attention forward, for gfx950.
//
// It follows the "FlashAttention 1, 2, 3" explainer's backward sections: P is not
// stored but recomputed from the saved LSE, P = exp(scale * q.k - LSE); with the row
// scalar D = sum_c dO_c O_c,
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Masked pairs have P = dS = 0.  Two kernels, in this order, both deterministic (no
// atomics):
//   attn_bwd_dq    one workgroup per 128-query tile, key/value tiles streamed
//                  through LDS: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T; its
//                  prologue also computes D and the base-2 LSE of its rows and
//                  stores them in the workspace
//   attn_bwd_dkdv  one workgroup per 128 keys of a key/value head, query tiles of
//                  every query head of the group (and their D, LSE) streamed through
//                  LDS: S = Q K^T, dV^T += dO^T P, dP = dO V^T, dK^T += Q^T dS
// The products use v_mfma_f32_32x32x16_bf16; P and dS are rounded to bf16 (RNE) as
// MFMA operands, everything else stays fp32.  The dQ kernel is the forward kernel's
// mirror image (key rows permuted so that scores are the next product's B operand);
// the dK/dV kernel is the same with the roles of queries and keys exchanged.
#pragma once
#include "device.h"
#include "prefill.h"
#include "worklist.h"

namespace ff {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* o;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* dsum;  // [B, Hq, sq_pad]  D per row
  float* lse2;  // [B, Hq, sq_pad]  LSE * log2(e); +inf for rows with no visible key
  int B, Sq, Sk, Hq, Hkv, G;
  int sq_pad;        // Sq rounded up to 64: 256-byte aligned rows for the loads into LDS
  int num_m;         // 128-query tiles per (batch, head)
  int num_n;         // 128-key blocks per (batch, kv head)
  int u_per;         // (batch, kv head) unit slots per XCD: ceil(B * Hkv / 8)
  float scale;       // softmax scale: enters dQ and dK
  float scale_log2;  // scale * log2(e)
  // Variants (VAR of both kernels): window limits (-1 = none), key j visible to query i
  // iff diag - wl <= j <= diag + wr with diag = i + Sk - Sq; ALiBi slope of (batch b,
  // query head h) at alibi[b * alibi_bstride + h], bias -slope |diag - j|.
  int wl, wr;
  const float* alibi;
  int alibi_bstride;
};

// Shared geometry of the two main kernels: 4 wavefronts of 32 rows, tiles of T rows
// of the streamed tensors, row-major in LDS with the 16-byte chunks of each row
// XOR-swizzled by swz(row).  The same swizzle serves the 128-bit row reads and the
// transposing reads.
template <int D, int TROWS>
struct BwdTraits {
  static constexpr int kThreads = 256;
  static constexpr int ROWB = D * 2;                      // bytes per row in LDS
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int TILE = TROWS * ROWB;               // bytes per streamed tile
  static constexpr int RPB = 256 / ROWB;                  // rows per 256-byte line
  static constexpr int LOADS = TROWS * CPR / kThreads;    // 16-byte loads per thread per tile
  // LDS banks span 256-byte lines.  The 128-bit row reads take 16 lanes (16 rows, one
  // logical chunk) at a time and the transposing reads 32 lanes (4 rows x 4 chunks of
  // an aligned group of four) at a time, so the XOR key must be one-to-one over the
  // lines of 16 rows and must differ in bits 2 and up across 4 consecutive rows: the
  // key of line u swaps the 2-bit fields of u (one bit of u at d = 64, where a line
  // holds two rows and the key has three bits).
  static __device__ __forceinline__ int swz(int r) {
    constexpr int L = 4 / RPB;  // lines per 4 rows
    const int u = r / RPB;
    return ((u % L) << 2) | ((u / L) % 4);
  }
  static_assert(D == 64 || D == 128, "head dimension");
};

#if defined(__HIP_DEVICE_COMPILE__)
// 128-bit LDS read at byte address a.
__device__ __forceinline__ u32x4 lds_b128(uint32_t a) {
  return *reinterpret_cast<const u32x4*>((const __attribute__((address_space(3))) char*)(uintptr_t)a);
}
#endif

// The transposing reads of one MFMA A operand: rows R + {0..3} (lo) and R + {4..7}
// (hi) of a tile, through precomputed per-lane addresses; R is a multiple of 16, so
// the swizzle of row R + r equals that of r and R enters as an immediate offset.
template <int OFF>
__device__ __forceinline__ u32x4 tr_operand(uint32_t base, uint32_t a_lo, uint32_t a_hi) {
  const u32x2 lo = ds_read_tr16_b64<OFF>(base + a_lo);
  const u32x2 hi = ds_read_tr16_b64<OFF>(base + a_hi);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Direct HBM -> LDS loads of one tile.  Wave w, load j fills the 1 KiB LDS block
// LOADS*w + j: lane i writes chunk slot 64*(LOADS*w + j) + i, i.e. row slot/CPR,
// physical chunk slot%CPR, which holds logical chunk (physical ^ swz(row)).  Rows at
// or past `rows` are out of the descriptor's range and land as zeros.
template <int LOADS>
__device__ __forceinline__ void tile_load(const char* base, int rows, int row_bytes,
                                          const int* off, uint32_t lds, int wave) {
  const i32x4 rd = buffer_desc(base, rows > 0 ? (uint32_t)rows * (uint32_t)row_bytes : 0u);
  const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds + 1024 * LOADS * wave);
#pragma unroll
  for (int j = 0; j < LOADS; ++j) buffer_load_lds16(rd, off[j], l0 + 1024 * j);
}

// Per-lane addresses shared by both kernels (lane = 32 H + n, 16-lane group g, s).
template <int D, int TROWS>
struct BwdAddr {
  using T = BwdTraits<D, TROWS>;
  int row[D / 16];    // row read: tile row prow(n) (bits 2, 3 of n swapped), logical chunk 2c + H
  int tlo[D / 32];    // transposing read, rows 8(g/2) + s/4, dcols 32db + 16(g%2) + 4(s%4)
  int thi[D / 32];    // the same four rows further down
  __device__ __forceinline__ BwdAddr(int lane) {
    const int n = lane & 31, H = lane >> 5;
    const int prow = (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) row[c] = prow * T::ROWB + 16 * ((2 * c + H) ^ T::swz(prow));
    const int g = lane >> 4, s = lane & 15;
    const int vrow = 8 * (g >> 1) + (s >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = 4 * db + 2 * (g & 1) + ((s & 3) >> 1);
      tlo[db] = vrow * T::ROWB + 16 * (chunk ^ T::swz(vrow)) + 8 * (s & 1);
      thi[db] = (vrow + 4) * T::ROWB + 16 * (chunk ^ T::swz(vrow + 4)) + 8 * (s & 1);
    }
  }
};

// Score element e (accumulator index 4j + i) of a 32x32 product whose A rows were
// read through prow: it belongs to row 16(j>>1) + 8H + 4(j&1) + i of the 32-row block.
__device__ __forceinline__ constexpr int perm_row(int e) {
  return 16 * ((e >> 2) >> 1) + 4 * ((e >> 2) & 1) + (e & 3);
}

// ---------------------------------------------------------------------------
// attn_bwd_dq: one workgroup per (128-query tile, batch, query head).  VAR: the window
// (and ALiBi) of the forward's variants; the key-tile range is clipped at both ends and
// tiles below n_bot get the left-edge element mask, as in the forward kernel.
template <int D, bool CAUSAL, int VAR>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist for the device target only
  constexpr bool WIN = VAR & kVarWindow, ALIBI = VAR & kVarAlibi;
  static_assert(VAR == 0 || WIN, "variant kernels include the window");
  constexpr int BM = 128, BN = 64;
  using T = BwdTraits<D, BN>;
  constexpr int ROWB = T::ROWB, CPR = T::CPR, TILE = T::TILE, LOADS = T::LOADS;
  // K tiles 0/1, V tiles 2/3 (before the first tile: the query tile's dO and Q rows),
  // then D of the tile's 128 rows
  constexpr int D_OFF = 4 * TILE;
  static_assert(BM * ROWB <= 2 * TILE, "dO and Q rows fit two tile buffers each");
  __shared__ __attribute__((aligned(1024))) char smem[D_OFF + BM * 4];

  // Work list of worklist.h, as the forward kernel's: rank = query tile (heaviest first
  // when causal), sub = query head of the unit.
  const int total = kXcds * p.u_per * p.G * p.num_m;
  const UnitItem item = unit_item(xcd_remap(blockIdx.x, total), p.u_per, p.num_m, p.G);
  const int unit = item.unit, mi = item.rank;
  if (unit >= p.B * p.Hkv) return;  // an idle unit slot
  const int b = unit / p.Hkv, hk = unit % p.Hkv, h = hk * p.G + item.sub;
  const int mblk = CAUSAL ? p.num_m - 1 - mi : mi;  // heaviest causal tiles first
  const int q0 = mblk * BM;
  const int Sq = p.Sq, Sk = p.Sk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31, H = lane >> 5;
  const int qrow = q0 + wave * 32 + n;

  // key tiles [0, n_max); tiles from n_mask need an element mask
  const int nb_total = (Sk + BN - 1) / BN;
  int n_max = nb_total;
  if (CAUSAL) {
    const int lim = (q0 + BM < Sq ? q0 + BM : Sq) - 1 + Sk - Sq;
    n_max = lim < 0 ? 0 : ((lim / BN + 1) < n_max ? lim / BN + 1 : n_max);
  }
  int n_mask = (Sk % BN) ? nb_total - 1 : nb_total;
  if (CAUSAL) {
    const int first = q0 + Sk - Sq + 1;
    const int tm = first <= 0 ? 0 : first / BN;
    n_mask = tm < n_mask ? tm : n_mask;
  }
  // Window: key tiles [n_min, n_max) hold keys some row of the tile sees; tiles below
  // n_bot hold keys left of the last row's window and need the element mask too.  The
  // range starts at an even tile, since the buffer parity is t & 1; a tile added that way
  // lies left of every row's window, below n_bot, so it is masked out entirely.
  int n_min = 0, n_bot = 0;
  if constexpr (WIN) {
    constexpr int LB = 6;  // log2(BN)
    static_assert((1 << LB) == BN, "BN");
    const int last_q = (q0 + BM < Sq ? q0 + BM : Sq) - 1;
    if (p.wr >= 0) {
      const int64_t lim = (int64_t)last_q + Sk - Sq + p.wr;
      const int64_t nm = lim < 0 ? 0 : (lim >> LB) + 1;
      n_max = nm < n_max ? (int)nm : n_max;
      const int64_t first = (int64_t)q0 + Sk - Sq + p.wr + 1;
      const int64_t tm = first <= 0 ? 0 : first >> LB;
      n_mask = tm < n_mask ? (int)tm : n_mask;
    }
    if (p.wl >= 0) {
      const int64_t lo_first = (int64_t)q0 + Sk - Sq - p.wl;
      const int64_t lo_last = (int64_t)last_q + Sk - Sq - p.wl;
      n_min = lo_first <= 0 ? 0 : (int)((lo_first >> LB) < nb_total ? lo_first >> LB : nb_total);
      const int64_t nb = lo_last <= 0 ? 0 : (lo_last + BN - 1) >> LB;
      n_bot = (int)(nb < n_max ? nb : n_max);
      n_bot = n_bot > n_min ? n_bot : n_min;
      n_min &= ~1;
    }
  }

  const int64_t q_stride = (int64_t)p.Hq * D;
  const int kv_row_bytes = p.Hkv * D * 2;
  float* dq_row = p.dq + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D;

  // Resident dO^T and Q^T fragments [qrow][16c + 8H .. +7], and the row scalars
  // D = sum_c dO_c O_c and L2 = LSE log2(e) (+inf for a row with no visible key).  They go
  // to the workspace for the dK/dV kernel, which runs next.  Every row below Sq is
  // written, also in tiles that see no key, since that kernel multiplies P = 0 by
  // (dP - D).  All loads read whole rows: dO and Q go to LDS (four 256-byte rows per load
  // instruction at d = 128) and the fragments are read from there; O (fp32, needed for D
  // only) goes to registers 8 lanes per row, one 128-byte line per row and instruction.
  // Loaded straight into the fragment layout, each instruction read 32-byte pieces of
  // 32 rows.  Rows past Sq read as zeros.
  const uint32_t smem_addr = lds_addr(smem);
  const int rows_q = Sq - q0 < BM ? Sq - q0 : BM;  // rows of the tile below Sq (>= 1)
  const int q_row_bytes = p.Hq * D * 2;
  const int64_t qtile = (((int64_t)b * Sq + q0) * p.Hq + h) * D;  // element offset of row q0
  {
    constexpr int QL = BM * CPR / T::kThreads;  // 16-byte loads per thread per tensor
    int qoff[QL];
#pragma unroll
    for (int j = 0; j < QL; ++j) {
      const int slot = 64 * (QL * wave + j) + lane;
      const int r = slot / CPR, ph = slot % CPR;
      qoff[j] = r * q_row_bytes + 16 * (ph ^ T::swz(r));
    }
    tile_load<QL>(reinterpret_cast<const char*>(p.dout + qtile), rows_q, q_row_bytes, qoff,
                  smem_addr, wave);
    tile_load<QL>(reinterpret_cast<const char*>(p.q + qtile), rows_q, q_row_bytes, qoff,
                  smem_addr + 2 * TILE, wave);
  }
  // O: pass ps covers rows 32 ps + tid / 8; load j of a lane holds the row's 16-byte chunk
  // 8 j + tid % 8 (dcols 4 (8 j + tid % 8) .. + 3)
  constexpr int OJ = D / 32;  // loads per row and lane
  f32x4 ov[4][OJ];
  {
    const auto od = __builtin_amdgcn_make_buffer_rsrc((void*)(p.o + qtile), (short)0,
                                                      rows_q * (p.Hq * D * 4), 0x00020000);
#pragma unroll
    for (int ps = 0; ps < 4; ++ps)
#pragma unroll
      for (int j = 0; j < OJ; ++j) {
        const int r = 32 * ps + (tid >> 3), c = 8 * j + (tid & 7);
        ov[ps][j] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       od, r * (p.Hq * D * 4) + 16 * c, 0, 0));
      }
  }
  const bool in = qrow < Sq;
  float L2 = INFINITY;
  if (in) {
    const float l = p.lse[((int64_t)b * p.Hq + h) * Sq + qrow];
    L2 = l == -INFINITY ? INFINITY : l * kLog2e;
  }
  wait_vmem();
  __syncthreads();  // every wavefront's dO and Q rows have landed
  // D of rows 32 ps + tid / 8: this lane's 4 OJ products, then the 8 lanes of the row
  {
    float* dsh = reinterpret_cast<float*>(smem + D_OFF);
#pragma unroll
    for (int ps = 0; ps < 4; ++ps) {
      const int r = 32 * ps + (tid >> 3);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < OJ; ++j) {
        const int c = 8 * j + (tid & 7);  // dcols 4c .. 4c + 3: bf16 chunk c / 2, half c % 2
        const u32x2 d2 = *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(
            (uintptr_t)(smem_addr + r * ROWB + 16 * ((c >> 1) ^ T::swz(r)) + 8 * (c & 1)));
        const f32x4& o = ov[ps][j];
        acc += __uint_as_float(d2[0] << 16) * o[0];
        acc += __uint_as_float(d2[0] & 0xffff0000u) * o[1];
        acc += __uint_as_float(d2[1] << 16) * o[2];
        acc += __uint_as_float(d2[1] & 0xffff0000u) * o[3];
      }
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if ((tid & 7) == 0) {
        dsh[r] = acc;
        if (r < rows_q) p.dsum[((int64_t)b * p.Hq + h) * p.sq_pad + q0 + r] = acc;
      }
    }
  }
  // the fragments: row qrow - q0, logical chunk 2c + H
  u32x4 of[D / 16], qf[D / 16];
  {
    const int rq = 32 * wave + n;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const uint32_t a = smem_addr + rq * ROWB + 16 * ((2 * c + H) ^ T::swz(rq));
      of[c] = lds_b128(a);
      qf[c] = lds_b128(a + 2 * TILE);
    }
  }
  __syncthreads();  // D complete; every wavefront is past its reads of the dO and Q rows
  const float Dr = reinterpret_cast<const float*>(smem + D_OFF)[32 * wave + n];
  if (in && H == 0) p.lse2[((int64_t)b * p.Hq + h) * p.sq_pad + qrow] = L2;
  if (n_max <= n_min) {  // no visible key for any row of this tile: dQ = 0
    if (qrow < Sq) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = H * 4; c < D; c += 8) st16f(dq_row + c, z);
    }
    return;
  }

  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)b * Sk * p.Hkv + hk) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)b * Sk * p.Hkv + hk) * D * 2;
  int loff[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int slot = 64 * (LOADS * wave + j) + lane;
    const int r = slot / CPR, ph = slot % CPR;
    loff[j] = r * kv_row_bytes + 16 * (ph ^ T::swz(r));
  }
  auto issue = [&](int t) {
    const int rows = Sk - t * BN;
    const int64_t toff = (int64_t)t * BN * kv_row_bytes;
    tile_load<LOADS>(kbase + toff, rows, kv_row_bytes, loff, smem_addr + (t & 1) * TILE, wave);
    tile_load<LOADS>(vbase + toff, rows, kv_row_bytes, loff, smem_addr + (2 + (t & 1)) * TILE, wave);
  };
  const BwdAddr<D, BN> ad(lane);

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqacc[i] = f32x16{};
  const float c2 = p.scale_log2;
  int last_key = CAUSAL && qrow + Sk - Sq < Sk - 1 ? qrow + Sk - Sq : Sk - 1;
  int first_key = 0;  // window: keys below are invisible to this row
  const int diag = qrow + Sk - Sq;
  if constexpr (WIN) {
    if (p.wr >= 0 && (int64_t)diag + p.wr < last_key) last_key = (int)((int64_t)diag + p.wr);
    if (p.wl >= 0 && (int64_t)diag - p.wl > 0) first_key = (int)((int64_t)diag - p.wl);
  }
  // ALiBi slope of this head in base-2 units
  const float slope2 = ALIBI ? p.alibi[(int64_t)b * p.alibi_bstride + h] * kLog2e : 0.f;

  // one key tile; PAR = t % 2 selects its K and V buffers at compile time, so every LDS
  // access is a per-lane offset plus an immediate
  const uint32_t lds0 = lds_addr(smem);
  auto step = [&](auto PARC, int t) {
    constexpr uint32_t PAR = decltype(PARC)::value;
    constexpr uint32_t K_OFF = PAR * TILE, V_OFF = (2 + PAR) * TILE;
    if (t + 1 < n_max) issue(t + 1);  // into the other buffers, free since the last barrier
    // per 32-key block kb: S^T = K Q^T and dP^T = V dO^T, dS^T = P^T (dP^T - D) with
    // P^T = 2^(s c2 - L2) (masked keys give 0), then dQ^T += K^T dS^T through transposing
    // reads of the K tile
    const bool masked = t >= n_mask || (WIN && t < n_bot);
    static_for<2>([&](auto KB) {
      constexpr int kb = decltype(KB)::value;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = mfma32(lds_b128(lds0 + K_OFF + kb * 32 * ROWB + ad.row[c]), qf[c], s);
        dp = mfma32(lds_b128(lds0 + V_OFF + kb * 32 * ROWB + ad.row[c]), of[c], dp);
      }
      float pr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = __builtin_fmaf(s[e], c2, -L2);
        if constexpr (ALIBI) {  // key t BN + 32 kb + 8 H + perm_row(e)
          const int key = t * BN + 32 * kb + 8 * H + perm_row(e);
          x = __builtin_fmaf(-slope2, __builtin_fabsf((float)(diag - key)), x);
        }
        pr[e] = fast_exp2(x);
      }
      if (masked) {
        const int vis = last_key - t * BN - 8 * H - 32 * kb;  // key offsets <= vis are visible
        const int vlo = first_key - t * BN - 8 * H - 32 * kb;  // and >= vlo (window)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (perm_row(e) > vis || (WIN && perm_row(e) < vlo)) pr[e] = 0.f;
      }
      float ds[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) ds[e] = pr[e] * (dp[e] - Dr);
      u32x4 dsf[2];
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        dsf[cp] = pack8(ds[8 * cp], ds[8 * cp + 1], ds[8 * cp + 2], ds[8 * cp + 3],
                        ds[8 * cp + 4], ds[8 * cp + 5], ds[8 * cp + 6], ds[8 * cp + 7]);
      static_for<2>([&](auto CP) {
        constexpr int cp = decltype(CP)::value;
        constexpr int off = (32 * kb + 16 * cp) * ROWB;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dqacc[db] = mfma32(tr_operand<off>(lds0 + K_OFF, ad.tlo[db], ad.thi[db]), dsf[cp], dqacc[db]);
      });
    });
    wait_vmem();
    __syncthreads();
  };

  issue(n_min);
  wait_vmem();
  __syncthreads();
  int t = n_min;
  for (; t + 1 < n_max; t += 2) {
    step(std::integral_constant<uint32_t, 0>{}, t);
    step(std::integral_constant<uint32_t, 1>{}, t + 1);
  }
  if (t < n_max) step(std::integral_constant<uint32_t, 0>{}, t);

  // dQ = scale * dQ^T: element 4j + i of block db is dcol 32db + 8j + 4H + i.  The rows
  // leave through LDS as in the forward kernel (each wavefront stages its 32 rows in the
  // tile buffers, 16-byte chunks XOR-swizzled by row) and are stored whole, with the
  // non-temporal hint.
  {
    const float sc = p.scale;
    constexpr int CH = D / 4, OROWB = D * 4, RPI = 64 / CH;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    wait_vmem();
    __syncthreads();  // every wavefront is past its last read of the tiles
    const uint32_t ost = lds0 + wave * 32 * OROWB;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 val = {dqacc[db][4 * j] * sc, dqacc[db][4 * j + 1] * sc,
                           dqacc[db][4 * j + 2] * sc, dqacc[db][4 * j + 3] * sc};
        const int c = 8 * db + 2 * j + H;
        *reinterpret_cast<lds_f32x4*>((uintptr_t)(ost + n * OROWB + 16 * (c ^ (n & 7)))) = val;
      }
    wave_lds_sync();
    const int rr = lane / CH, cc = lane % CH;
    const int row0 = q0 + 32 * wave;
    float* obase = p.dq + ((int64_t)b * Sq + row0) * q_stride + (int64_t)h * D + 4 * cc;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + rr;
      const f32x4 val =
          *reinterpret_cast<const lds_f32x4*>((uintptr_t)(ost + r * OROWB + 16 * (cc ^ (r & 7))));
      if (row0 + r < Sq) st16f_nt(obase + (int64_t)r * q_stride, val);
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// attn_bwd_dkdv: one workgroup of 8 wavefronts per (128 keys, batch, key/value head);
// its query tiles (64 rows) are those of every query head of the group.  Each tile goes
// through two phases:
//   1. wavefront w takes query block qb = w / 4 and key block kb = w % 4 (32 x 32):
//      S = Q K^T, dP = dO V^T (K and V fragments of the block resident), P and
//      dS = P (dP - D); P and dS go to LDS as bf16, [key][query];
//   2. wavefront w takes key block kb = w % 4 and half dh = w / 4 of the head
//      dimension: dV^T += dO^T P and dK^T += Q^T dS over the tile's 64 queries, dO^T
//      and Q^T through transposing reads, P and dS read back from LDS.
// Splitting the accumulators over two wavefronts keeps each at 32 keys x d/2, so two
// wavefronts fit on a SIMD.  Each tile costs two workgroup barriers: the one at its
// start also orders the previous tile's phase 2 before this tile's phase 1, so P and
// dS need one buffer each.
// VAR: the window (and ALiBi): the query-tile range is clipped at both ends and the
// element mask covers both edges of each key's window.
template <int D, bool CAUSAL, int VAR>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool WIN = VAR & kVarWindow, ALIBI = VAR & kVarAlibi;
  static_assert(VAR == 0 || WIN, "variant kernels include the window");
  constexpr int BK = 128, BQ = 64, NT = 512;
  constexpr int ROWB = D * 2, CPR = D / 8, TILE = BQ * ROWB;
  constexpr int LOADS = BQ * CPR / NT;          // 16-byte loads per thread per tile
  constexpr int PROWB = BQ * 2;                 // bytes per key row of the P / dS buffers
  constexpr int PBUF = BK * PROWB;              // the P or the dS buffer
  constexpr int DH = D / 64;                    // 32-dcol blocks per half of d
  using T = BwdTraits<D, BQ>;
  // Q tiles 0/1, dO tiles 2/3, P, dS, then L2 and D slots 0/1 (1 KiB each: the 64
  // values use the first 256 bytes, the rest of the load lands as zeros), then the
  // staging area of the block's V rows.  The block's K rows are staged in the P and dS
  // buffers, which the first tile's phase 1 writes only after a workgroup barrier.
  constexpr int KV_OFF = 4 * TILE;                        // K rows (in P and dS)
  constexpr int VV_OFF = 4 * TILE + 2 * PBUF + 4 * 1024;  // V rows
  static_assert(BK * ROWB <= 2 * PBUF, "K rows fit the P and dS buffers");
  __shared__ __attribute__((aligned(1024))) char smem[VV_OFF + BK * ROWB];

  // Work list of worklist.h: rank = key block (ascending: the heaviest first when
  // causal), one item per unit and rank.
  const int total = kXcds * p.u_per * p.num_n;
  const UnitItem item = unit_item(xcd_remap(blockIdx.x, total), p.u_per, p.num_n, 1);
  const int unit = item.unit, nb = item.rank;
  if (unit >= p.B * p.Hkv) return;  // an idle unit slot
  const int b = unit / p.Hkv, hk = unit % p.Hkv;
  const int k0 = nb * BK;
  const int Sq = p.Sq, Sk = p.Sk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31, H = lane >> 5;
  const int kb = wave & 3;       // key block of both phases
  const int qb = wave >> 2;      // phase 1: query block
  const int dh = wave >> 2;      // phase 2: half of the head dimension
  const int key = k0 + 32 * kb + n;

  // query tiles [qt_lo, qt_hi) of each head; tiles below qt_mask need the mask of the
  // right edge (key <= q + Sk - Sq + r: r = 0 when causal, else the window's wr) and
  // tiles from qt_lmask that of the left edge (key >= q + Sk - Sq - wl)
  const int num_qt = (Sq + BQ - 1) / BQ;
  int qt_lo = 0, qt_hi = num_qt, qt_mask = 0, qt_lmask = num_qt;
  int64_t r_edge = -1;  // -1: no right edge
  if (CAUSAL) r_edge = 0;
  else if (WIN && p.wr >= 0) r_edge = p.wr;
  if (r_edge >= 0) {
    const int64_t first_q = (int64_t)k0 - (Sk - Sq) - r_edge;  // first query seeing key k0
    qt_lo = first_q <= 0 ? 0 : (int)(first_q / BQ < num_qt ? first_q / BQ : num_qt);
    const int64_t q_full = (int64_t)k0 + BK - 1 - (Sk - Sq) - r_edge;  // from here all keys
    qt_mask = q_full <= 0 ? 0 : (int)((q_full + BQ - 1) / BQ < num_qt ? (q_full + BQ - 1) / BQ : num_qt);
  }
  if (WIN && p.wl >= 0) {
    const int64_t last_q = (int64_t)k0 + BK - 1 - (Sk - Sq) + p.wl;  // last query seeing a key
    qt_hi = last_q < 0 ? 0 : (int)(last_q / BQ + 1 < num_qt ? last_q / BQ + 1 : num_qt);
    const int64_t qa = (int64_t)k0 - (Sk - Sq) + p.wl + 1;  // from here key k0 is left out
    qt_lmask = qa <= 0 ? 0 : (int)(qa / BQ < num_qt ? qa / BQ : num_qt);
  }
  const int per_head = qt_hi > qt_lo ? qt_hi - qt_lo : 0;
  const int items = per_head * p.G;

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const int q_row_bytes = p.Hq * D * 2;

  f32x16 dkacc[DH], dvacc[DH];
#pragma unroll
  for (int i = 0; i < DH; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  if (items > 0) {
    u32x4 kf[D / 16], vf[D / 16];  // read from LDS once the block's rows have landed (below)
    int loff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int slot = 64 * (LOADS * wave + j) + lane;
      const int r = slot / CPR, ph = slot % CPR;
      loff[j] = r * q_row_bytes + 16 * (ph ^ T::swz(r));
    }
    const uint32_t smem_addr = lds_addr(smem);
    const uint32_t s_base = smem_addr + 4 * TILE + 2 * PBUF;  // L2 0/1, then D 0/1
    // item it: head h = hk*G + it / per_head, query tile qt_lo + it % per_head
    auto issue = [&](int it) {
      const int h = hk * p.G + it / per_head;
      const int q0 = (qt_lo + it % per_head) * BQ;
      const int64_t qoff = (((int64_t)b * Sq + q0) * p.Hq + h) * D * 2;
      const int rows = Sq - q0;
      const uint32_t par = it & 1;
      tile_load<LOADS>(reinterpret_cast<const char*>(p.q) + qoff, rows, q_row_bytes, loff,
                       smem_addr + par * TILE, wave);
      tile_load<LOADS>(reinterpret_cast<const char*>(p.dout) + qoff, rows, q_row_bytes, loff,
                       smem_addr + (2 + par) * TILE, wave);
      if (wave < 2) {  // wave 0: L2, wave 1: D, 64 floats each
        const float* src = (wave == 0 ? p.lse2 : p.dsum) + ((int64_t)b * p.Hq + h) * p.sq_pad + q0;
        const int nv = rows < BQ ? rows : BQ;
        const i32x4 rd = buffer_desc(src, (uint32_t)nv * 4u);
        const uint32_t dst = s_base + (2 * wave + par) * 1024;
        buffer_load_lds16(rd, 16 * lane, __builtin_amdgcn_readfirstlane(dst));
      }
    };
    // Per-lane LDS offsets, fixed for the whole loop; the tile parity is a compile-time
    // constant in each copy of the loop body, so every LDS access is one of these plus an
    // immediate.
    const BwdAddr<D, BQ> ad(lane);
    int arow[D / 16];  // phase 1 A operand: row read of query block qb, chunk 2c + H
#pragma unroll
    for (int c = 0; c < D / 16; ++c) arow[c] = ad.row[c] + qb * 32 * ROWB;
    // transposing-read offsets of this wavefront's dcol blocks dh*DH + j (the layout of
    // BwdAddr::tlo / thi)
    int tlo[DH], thi[DH];
    {
      const int g = lane >> 4, s = lane & 15;
      const int vrow = 8 * (g >> 1) + (s >> 2);
#pragma unroll
      for (int j = 0; j < DH; ++j) {
        const int chunk = 4 * (dh * DH + j) + 2 * (g & 1) + ((s & 3) >> 1);
        tlo[j] = vrow * ROWB + 16 * (chunk ^ T::swz(vrow)) + 8 * (s & 1);
        thi[j] = (vrow + 4) * ROWB + 16 * (chunk ^ T::swz(vrow + 4)) + 8 * (s & 1);
      }
    }
    // P / dS buffers: row = key in the block (128 bytes: 64 queries, two rows per
    // 256-byte bank line, bit 0 of the row picking the half), 16-byte chunk c of row r
    // stored at chunk c ^ key(r), key(r) = ((r / 2) % 8) ^ 4 (r % 2).  Phase 1 writes and
    // phase 2 reads both have lane (n, H) on row n, chunk c0 + H.  The hardware serves a
    // 128-bit write eight consecutive lanes at a time and a 128-bit read in four groups
    // of 16 lanes (lane bit 5 and the parity of lane bits 2-4 fixed), each group needing
    // distinct bank slots; measured on these exact access patterns, this key gives no bank
    // conflicts for either, where (r / 2) % 8 cost 8 conflict cycles per write.
    auto pchunk = [](int r, int c) {
      const int key = ((r >> 1) & 7) ^ ((r & 1) << 2);
      return r * PROWB + 16 * (c ^ key);
    };
    const int prow = 32 * kb + n;
    int pwr[2], prd[4];  // phase 1 writes (queries 32qb + 16half + 8H ..), phase 2 reads
#pragma unroll
    for (int half = 0; half < 2; ++half) pwr[half] = pchunk(prow, 4 * qb + H + 2 * half);
#pragma unroll
    for (int cq = 0; cq < 4; ++cq) prd[cq] = pchunk(prow, 2 * cq + H);
    const int srow = 4 * (32 * qb + 8 * H);  // L2 / D of queries 32qb + 8H ..
    const float c2 = p.scale_log2;
    const uint32_t lds0 = lds_addr(smem);
    constexpr uint32_t P_OFF = 4 * TILE, DS_OFF = 4 * TILE + PBUF, S_OFF = 4 * TILE + 2 * PBUF;
    auto st_lds = [](uint32_t a, u32x4 v) {
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)a) = v;
    };

    // one tile: PAR is the parity of item it (LDS buffers of its Q, dO, L2 and D)
    auto step = [&](auto PARC, int it) {
      constexpr uint32_t PAR = decltype(PARC)::value;
      constexpr uint32_t Q_OFF = PAR * TILE, O_OFF = (2 + PAR) * TILE;
      constexpr uint32_t L2_OFF = S_OFF + PAR * 1024, DD_OFF = S_OFF + (2 + PAR) * 1024;
      wait_vmem();
      __syncthreads();  // tile it in LDS; phase 2 of tile it-1 done everywhere
      if (it + 1 < items) issue(it + 1);
      const int qt = qt_lo + it % per_head;
      const bool masked = (r_edge >= 0 && qt < qt_mask) || (WIN && qt >= qt_lmask);
      // ALiBi slope of this item's query head in base-2 units
      const float slope2 =
          ALIBI ? p.alibi[(int64_t)b * p.alibi_bstride + hk * p.G + it / per_head] * kLog2e : 0.f;

      // ---- phase 1: S, dP of (qb, kb); P, dS -> LDS.  Lane (key n, H) holds queries
      // 32 qb + 8H + {0..7} (elements 0..7) and + 16 (elements 8..15).
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) sacc = mfma32(lds_b128(lds0 + Q_OFF + arow[c]), kf[c], sacc);
      float pr[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // elements 4w .. 4w+3: queries 16(w/2) + 4(w%2) + ..
        const u32x4 l2 = lds_b128(lds0 + L2_OFF + srow + 4 * (16 * (w >> 1) + 4 * (w & 1)));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          float y = __builtin_fmaf(sacc[4 * w + x], c2, -__uint_as_float(l2[x]));
          if constexpr (ALIBI) {  // query qt BQ + 32 qb + 8 H + perm_row(e)
            const int e = 4 * w + x;
            const int diag = qt * BQ + 32 * qb + 8 * H + perm_row(e) + Sk - Sq;
            y = __builtin_fmaf(-slope2, __builtin_fabsf((float)(diag - key)), y);
          }
          pr[4 * w + x] = fast_exp2(y);
        }
      }
      if (masked) {
        // key <= q + Sk - Sq + r  <=>  query offset in the tile >= key - (Sk - Sq) - r - q0;
        // key >= q + Sk - Sq - wl  <=>  query offset <= key - (Sk - Sq) + wl - q0
        const int64_t base = (int64_t)key - (Sk - Sq) - qt * BQ - 8 * H - 32 * qb;
        // element offsets lie in [0, 23]: bounds clamped to [-1, 32] compare as int
        const int64_t need = r_edge >= 0 ? base - r_edge : -1;
        const int64_t lim = WIN && p.wl >= 0 ? base + p.wl : 32;
        const int need_c = (int)(need < -1 ? -1 : (need > 32 ? 32 : need));
        const int lim_c = (int)(lim < -1 ? -1 : (lim > 32 ? 32 : lim));
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (perm_row(e) < need_c || perm_row(e) > lim_c) pr[e] = 0.f;
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        st_lds(lds0 + P_OFF + pwr[half],
               pack8(pr[8 * half], pr[8 * half + 1], pr[8 * half + 2], pr[8 * half + 3],
                     pr[8 * half + 4], pr[8 * half + 5], pr[8 * half + 6], pr[8 * half + 7]));
      f32x16 dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) dpacc = mfma32(lds_b128(lds0 + O_OFF + arow[c]), vf[c], dpacc);
      float ds[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x4 dd = lds_b128(lds0 + DD_OFF + srow + 4 * (16 * (w >> 1) + 4 * (w & 1)));
#pragma unroll
        for (int x = 0; x < 4; ++x)
          ds[4 * w + x] = pr[4 * w + x] * (dpacc[4 * w + x] - __uint_as_float(dd[x]));
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
        st_lds(lds0 + DS_OFF + pwr[half],
               pack8(ds[8 * half], ds[8 * half + 1], ds[8 * half + 2], ds[8 * half + 3],
                     ds[8 * half + 4], ds[8 * half + 5], ds[8 * half + 6], ds[8 * half + 7]));
      __syncthreads();  // P and dS of the whole tile written

      // ---- phase 2: dV^T += dO^T P, dK^T += Q^T dS for key block kb, dcols of half dh,
      // over the tile's four 16-query chunks
      static_for<4>([&](auto CQ) {
        constexpr int cq = decltype(CQ)::value;
        constexpr int rowoff = 16 * cq * ROWB;
        const u32x4 pb = lds_b128(lds0 + P_OFF + prd[cq]);
        const u32x4 sb = lds_b128(lds0 + DS_OFF + prd[cq]);
#pragma unroll
        for (int j = 0; j < DH; ++j) {
          dvacc[j] = mfma32(tr_operand<rowoff>(lds0 + O_OFF, tlo[j], thi[j]), pb, dvacc[j]);
          dkacc[j] = mfma32(tr_operand<rowoff>(lds0 + Q_OFF, tlo[j], thi[j]), sb, dkacc[j]);
        }
      });
    };

    // Resident K and V fragments of key block kb (B operands of S = Q K^T, dP = dO V^T).
    // The block's 128 K and V rows go to LDS as whole rows (four rows of 256 bytes per
    // load instruction at d = 128, in flight with tile 0's loads; rows past Sk land as
    // zeros), and each lane reads its fragments from there: loaded straight into the
    // fragment layout, every instruction read 32-byte pieces of 32 rows.
    {
      constexpr int KVL = BK * CPR / NT;  // 16-byte loads per thread per tensor
      const int kv_row_bytes = (int)kv_stride * 2;
      int koff[KVL];
#pragma unroll
      for (int j = 0; j < KVL; ++j) {
        const int slot = 64 * (KVL * wave + j) + lane;
        const int r = slot / CPR, ph = slot % CPR;
        koff[j] = r * kv_row_bytes + 16 * (ph ^ T::swz(r));
      }
      const int64_t boff = (((int64_t)b * Sk + k0) * kv_stride + (int64_t)hk * D) * 2;
      tile_load<KVL>(reinterpret_cast<const char*>(p.k) + boff, Sk - k0, kv_row_bytes, koff,
                     smem_addr + KV_OFF, wave);
      tile_load<KVL>(reinterpret_cast<const char*>(p.v) + boff, Sk - k0, kv_row_bytes, koff,
                     smem_addr + VV_OFF, wave);
      issue(0);
      wait_vmem();
      __syncthreads();  // every wavefront's rows have landed
      // row 32 kb + n, logical chunk 2c + H; the first step's barrier orders these reads
      // before phase 1 rewrites the K rows' area
      const int kr = 32 * kb + n;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const int a = kr * ROWB + 16 * ((2 * c + H) ^ T::swz(kr));
        kf[c] = lds_b128(smem_addr + KV_OFF + a);
        vf[c] = lds_b128(smem_addr + VV_OFF + a);
      }
    }
    int it = 0;
    for (; it + 1 < items; it += 2) {
      step(std::integral_constant<uint32_t, 0>{}, it);
      step(std::integral_constant<uint32_t, 1>{}, it + 1);
    }
    if (it < items) step(std::integral_constant<uint32_t, 0>{}, it);
  }

  // dK = scale * dK^T, dV = dV^T: element 4j + i of block jb is dcol
  // 32 (dh DH + jb) + 8j + 4H + i.  Each wavefront's 32 key rows of its half of d leave
  // through LDS (dK, then dV, in the Q/dO tile buffers), 16-byte chunks XOR-swizzled by
  // row, and are stored as whole half rows (128-byte lines) with the non-temporal hint.
  {
    const float sc = p.scale;
    constexpr int HD = D / 2, HCH = HD / 4, HROWB = HD * 4, RPI = 64 / HCH;
    static_assert(8 * 32 * HROWB <= 4 * TILE, "staging fits the tile buffers");
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    wait_vmem();
    __syncthreads();  // every wavefront is past its last read of the tiles
    const uint32_t ost = lds_addr(smem) + wave * 32 * HROWB;
    const int rr = lane / HCH, cc = lane % HCH;
    const int krow0 = k0 + 32 * kb;
    static_for<2>([&](auto KV) {
      constexpr int kv = decltype(KV)::value;  // 0: dK, 1: dV
#pragma unroll
      for (int jb = 0; jb < DH; ++jb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& a = kv == 0 ? dkacc[jb] : dvacc[jb];
          const float f = kv == 0 ? sc : 1.f;
          const f32x4 val = {a[4 * j] * f, a[4 * j + 1] * f, a[4 * j + 2] * f, a[4 * j + 3] * f};
          const int c = 8 * jb + 2 * j + H;
          *reinterpret_cast<lds_f32x4*>((uintptr_t)(ost + n * HROWB + 16 * (c ^ (n & 7)))) = val;
        }
      wave_lds_sync();
      float* base = (kv == 0 ? p.dk : p.dv) + ((int64_t)b * Sk + krow0) * kv_stride +
                    (int64_t)hk * D + dh * HD + 4 * cc;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = RPI * i + rr;
        const f32x4 val = *reinterpret_cast<const lds_f32x4*>(
            (uintptr_t)(ost + r * HROWB + 16 * (cc ^ (r & 7))));
        if (krow0 + r < Sk) st16f_nt(base + (int64_t)r * kv_stride, val);
      }
      wave_lds_sync();  // dV's rows overwrite dK's
    });
  }
#endif
}

}  // namespace ff
