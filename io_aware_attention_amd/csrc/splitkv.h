// attn_fwd_splitkv: the split-KV forward pass for short query blocks (decode),
// whose partials attn_splitkv_combine (combine.h) merges ("03 forward CUDA
// kernel", section 7; the walk-through's split-KV kernel and grid description).
//
// A workgroup owns one (block of 16 folded query rows, batch, key/value head,
// split).  The Hq/Hkv query heads that share a key/value head are folded into
// the row dimension (row R -> query position R / G, head hk*G + R % G), so one
// key/value stream serves the whole group (forward-kernel page section 7.4).
// The split's key range is dealt to the 4 wavefronts in 32-key steps; each
// wavefront keeps its own online-softmax state for the 16 rows and the four
// states are merged through LDS at the end, exactly like the split combine.
//
// Products use v_mfma_f32_16x16x32_bf16:
//   S^T (16 keys x 16 rows) = K . Q^T   A = K rows from LDS
//   O^T (16 dcols x 16 rows) += V^T . P^T, 32 keys per instruction
// The key rows of the two 16-key blocks are interleaved so that each lane's
// eight scores are eight consecutive keys, which makes them the P^T operand
// as they stand.  K and V are loaded as whole rows (16 lanes per 256-byte row, so
// every load instruction reads full cache lines) and go through per-wavefront LDS
// areas row by row, as loaded; GEMM0's K fragments come out with 128-bit reads and
// GEMM1's V^T fragments with transposing reads.
//
// Variants (VAR != 0, cache kernels only; the walk-through's Is_local, Has_alibi,
// Is_softcap): with diag = i + Sk - Sq for query i, the window keeps keys
// diag - wl <= j <= diag + wr (-1: no limit) and narrows the keys the splits share;
// ALiBi adds -slope |diag - j| and the soft cap maps s to c tanh(s scale / c), both
// applied to the scores in base-2 units before the row maximum.
#pragma once
#include "device.h"

namespace ff {

struct SplitParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_accum;
  float* lse_accum;
  float* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv, G;
  int rows;         // Sq * G folded rows per key/value head
  int num_mb;       // ceil(rows / 16)
  int num_splits;
  int split_keys;   // keys per split (a multiple of the split block)
  int causal;
  float scale_log2;
  // Key/value cache (the CACHE kernel): k and v hold num_blocks blocks of `page` key
  // positions, [num_blocks, page, Hkv, d].  Logical position t of batch b lives in block
  // block_table[b * max_blocks + t / page] (block b when block_table is NULL), row
  // t % page; batch b's keys are positions leftpad[b] .. kv_seqlens[b] + new_keys - 1.
  // Each split takes an equal share of its batch's keys.  Sk is unused.
  const int* kv_seqlens;
  const int* leftpad;
  const int* block_table;
  int num_blocks, page, max_blocks, new_keys;
  // Variants: window limits (-1 = none); ALiBi slope of (batch b, query head h) at
  // alibi[b * alibi_bstride + h]; soft-cap constants cap_k = 2 scale log2(e) / c and
  // cap2 = c log2(e).
  int wl, wr;
  const float* alibi;
  int alibi_bstride;
  float cap_k, cap2;
};

template <int D>
struct SplitTraits {
  static constexpr int BMD = 16;                  // folded rows per workgroup
  static constexpr int TK = 32;                   // keys per wavefront step
  static constexpr int kWaves = 4;
  // V rows in a wavefront's LDS area: key row r of the step at RS p(r) bytes, p(r) = r
  // with its bits 2 and 3 exchanged, RS = the row's bytes + 32.  The 32-byte pad moves
  // consecutive slots 32 bytes along the 256-byte bank line (RS / 32 is odd), and the
  // exchange puts the eight rows that one half-wavefront's transposing read touches
  // (rows j and 8 + j, j < 4, of its two 16-lane groups; + 4 for the second read) on
  // eight consecutive slots: 32 lanes x 8 bytes then cover the line once.  A 128-bit row
  // write by 8 consecutive lanes is 128 contiguous bytes.  Row r + i (i < 4) of a 4-row
  // group is slot p(r) + i, and the second read's rows are slot + 8, so every address
  // is one per-lane base plus an immediate.
  static constexpr int RS = 2 * D + 32;
  static constexpr int WV = TK * RS;               // V area per wavefront
  // K rows in a wavefront's LDS area, unpadded, the 16-byte chunks of row r XOR-swizzled
  // by kswz(r).  A 128-bit read serves 16 lanes per cycle, and the 16 lanes of a GEMM0
  // fragment read touch rows {0..3, 8..11, 16..19, 24..27} (+ 4 kb) at one logical
  // chunk: the swizzle puts them on 16 distinct 16-byte slots of the 256-byte bank line.
  // A row write (16 lanes, one row's chunks, d = 128; two rows at d = 64) is a
  // permutation of whole lines, conflict-free as well.
  static constexpr int RSK = 2 * D;
  static constexpr int WK = TK * RSK;              // K area per wavefront
  static __device__ __forceinline__ int kswz(int r) {
    return D == 128 ? (r + 4 * (r >> 4)) & 15 : ((r >> 1) & 1) | (((r >> 3) & 3) << 1);
  }
  static constexpr int KB = TK * D / 8 / 64;       // 16-byte K loads per lane per step
  static __device__ __forceinline__ int slot(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
  }
  static constexpr int VB = TK * D / 8 / 4 / 64;  // 4-key x 8-dcol V blocks per lane
  // The merge's partial O rows, padded by 4 floats: at D floats a row is a multiple of
  // the 256-byte bank line, and the 16 rows one write instruction spreads over would
  // all start on the same bank.
  static constexpr int CD = D + 4;
  static constexpr int kCombine = kWaves * (2 * BMD + BMD * CD) * 4;
  static constexpr int kLds =
      kWaves * (WV + WK) > kCombine ? kWaves * (WV + WK) : kCombine;
};

template <int D, bool CACHE, int VAR>
__global__ __launch_bounds__(256, 2) void attn_fwd_splitkv(SplitParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist for the device target only
  constexpr bool WIN = VAR & kVarWindow, ALIBI = VAR & kVarAlibi, CAP = VAR & kVarSoftcap;
  constexpr bool LOGIT = ALIBI || CAP;  // scores become base-2 logits before the row max
  static_assert(VAR == 0 || CACHE, "variants are built for the cache kernel");
  using T = SplitTraits<D>;
  constexpr int TK = T::TK, VB = T::VB, NW = T::kWaves;
  __shared__ __attribute__((aligned(16))) char smem[T::kLds];

  int u = blockIdx.x;
  const int s = u % p.num_splits;
  u /= p.num_splits;
  const int mb = u % p.num_mb;
  u /= p.num_mb;
  const int hk = u % p.Hkv;
  const int b = u / p.Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int nr = lane & 15;   // row of this lane in the B operand and the outputs
  const int g4 = lane >> 4;   // which 16-lane group

  const int G = p.G, Sq = p.Sq;
  int Sk = p.Sk;
  int lp = 0;  // first key position (cache left padding)
  if constexpr (CACHE) {
    // clamped so that no access leaves the cache, whatever the device arrays hold
    const int cap = p.max_blocks * p.page;
    int64_t n = (int64_t)p.kv_seqlens[b] + p.new_keys;
    Sk = n < 0 ? 0 : (n > cap ? cap : (int)n);
    if (p.leftpad) {
      const int a = p.leftpad[b];
      lp = a < 0 ? 0 : (a > Sk ? Sk : a);
    }
  }
  const int R = mb * 16 + nr;
  const bool row_ok = R < p.rows;
  const int qi = R / G;
  const int qh = hk * G + R % G;

  // key range of this split, clipped by the causal limit of the block's last row
  const int r_last = (mb * 16 + 16 < p.rows ? mb * 16 + 16 : p.rows) - 1;
  const int i_first = (mb * 16) / G;
  int k_first = lp, k_end = Sk;  // keys some row of the block may see
  int mask_below = lp;           // steps starting below this need the element mask
  if constexpr (WIN) {
    const int64_t off = (int64_t)Sk - Sq;
    if (p.wr >= 0) {
      const int64_t e = (int64_t)(r_last / G) + off + p.wr + 1;
      k_end = e < k_end ? (e < 0 ? 0 : (int)e) : k_end;
    }
    if (p.wl >= 0) {
      const int64_t f = (int64_t)i_first + off - p.wl;
      const int64_t fl = (int64_t)(r_last / G) + off - p.wl;
      k_first = f > k_first ? (int)(f < Sk ? f : Sk) : k_first;
      mask_below = fl > mask_below ? (int)(fl < Sk ? fl : Sk) : mask_below;
    }
  }
  int j_lo, j_hi;
  if constexpr (CACHE) {
    // equal shares of whole 128-key blocks from the step holding the first key
    const int base0 = k_first & ~(TK - 1);
    int per = (k_end - base0 + p.num_splits - 1) / p.num_splits;
    per = per < 0 ? 0 : per;
    const int chunk = (per + NW * TK - 1) / (NW * TK) * (NW * TK);
    j_lo = base0 + s * chunk;
    j_hi = j_lo + chunk < k_end ? j_lo + chunk : k_end;
  } else {
    j_lo = s * p.split_keys;
    j_hi = j_lo + p.split_keys < Sk ? j_lo + p.split_keys : Sk;
  }
  if (p.causal) {
    const int lim = r_last / G + Sk - Sq + 1;
    j_hi = lim < j_hi ? lim : j_hi;
  }
  // steps whose keys all lie below this bound need no element mask
  int nomask_end = p.causal ? (i_first + Sk - Sq + 1 < Sk ? i_first + Sk - Sq + 1 : Sk) : Sk;
  int row_lim = p.causal ? qi + Sk - Sq : 0x7fffffff;
  int row_lo = lp;  // keys below are invisible to this lane's row
  if constexpr (WIN) {
    const int64_t diag = (int64_t)qi + Sk - Sq;
    if (p.wr >= 0) {
      const int64_t ne = (int64_t)i_first + Sk - Sq + p.wr + 1;
      nomask_end = ne < nomask_end ? (ne < 0 ? 0 : (int)ne) : nomask_end;
      const int64_t rl = diag + p.wr;
      row_lim = rl < row_lim ? (rl < -1 ? -1 : (int)rl) : row_lim;
    }
    if (p.wl >= 0) {
      const int64_t lo = diag - p.wl;
      row_lo = lo > row_lo ? (int)lo : row_lo;
    }
  }

  const int64_t q_stride = (int64_t)p.Hq * D;
  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const float c2 = p.scale_log2;
  // ALiBi slope of this lane's row (its query head) in base-2 units
  const float slope2 = ALIBI ? p.alibi[(int64_t)b * p.alibi_bstride + qh] * kLog2e : 0.f;
  const int diag_row = qi + Sk - Sq;

  // Q^T fragments: Q[row][32c + 8 g4 .. +7]
  u32x4 qf[D / 32];
  {
    const uint16_t* qp = p.q + ((int64_t)b * Sq + qi) * q_stride + (int64_t)qh * D + 8 * g4;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      if (row_ok) qf[c] = ld16(qp + 32 * c);
      else qf[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // row 0 of this batch (dense) or of the cache (CACHE) for this key/value head
  const int64_t brow = CACHE ? 0 : (int64_t)b * Sk;
  const uint16_t* kbase = p.k + brow * kv_stride + (int64_t)hk * D;
  const uint16_t* vbase = p.v + brow * kv_stride + (int64_t)hk * D;
  const uint32_t wv = lds_addr(smem) + wave * T::WV;
  const uint32_t wk = lds_addr(smem) + NW * T::WV + wave * T::WK;
  // V addresses (the layout in SplitTraits).  Writes: row 4 kg + r, 16-byte chunk cg of
  // this lane's loads at vw[bi] + RS r.  Reads: GEMM1's A operand for dcols 16 db ..
  // + 15 is two ds_read_b64_tr_b16.  In each 16-lane group g4, source lane nr addresses
  // key row 8 g4 + nr / 4 (+ 4 for the second read) at dcols 16 db + 4 (nr % 4) .. + 3,
  // so result lane nr holds dcol 16 db + nr over keys 8 g4 .. + 3 (+ 4 .. + 7): the A
  // fragment V^T[16 db + nr][8 g4 .. + 7].
  int vw[VB];
#pragma unroll
  for (int bi = 0; bi < VB; ++bi) {
    const int blk = lane + 64 * bi;
    const int cg = blk % (D / 8), kg = blk / (D / 8);
    vw[bi] = T::slot(4 * kg) * T::RS + 16 * cg;
  }
  const int vr = T::slot(8 * g4 + (nr >> 2)) * T::RS + 8 * (nr & 3);

  f32x4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // K row read by this lane for key block kb: 8*(nr/4) + 4*kb + nr%4
  const int krow0 = 8 * (nr >> 2) + (nr & 3);

  // Software pipeline: each wavefront's loads of its next 32-key step are in
  // flight while the current step is computed (two register sets, swapped by
  // unrolling the loop twice).
  // Every key and value is read once, so the loads carry the non-temporal hint.  With
  // whole-row loads it pays on a dense and a paged cache alike (paged_decode 190.8 ->
  // 172.0 us); while K was read as 64-byte pieces of 16 rows per instruction, the hint
  // cost the paged cache 13% and was left off there.
  constexpr int kv_policy = kLoadStreaming;
  // Loads go through buffer descriptors that cover rows j0 .. min(j0 + TK, Sk) - 1
  // of this key/value head, so rows past Sk read as zero without a branch.  A cache
  // step (32 aligned keys) lies inside one block, since blocks hold a multiple of 32
  // positions; V rows before the first key read as zero too (an offset of nrec is out
  // of range), because the product with a zero probability must not meet stale data.
  const int kv_row_bytes = p.Hkv * D * 2;
  auto load_kv = [&](int j0, u32x4 (&kreg)[T::KB], u32x4 (&vreg)[VB][4]) {
    const int rows = Sk - j0 < TK ? Sk - j0 : TK;
    const int nrec = rows > 0 ? rows * kv_row_bytes : 0;
    int64_t row0 = j0;
    if constexpr (CACHE) {
      const int pg = j0 / p.page;
      int blk = p.block_table ? p.block_table[(int64_t)b * p.max_blocks + pg] : b;
      blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);
      row0 = (int64_t)blk * p.page + (j0 - pg * p.page);
    }
    const int lo = lp - j0;  // rows below this are left padding
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + row0 * kv_stride), (short)0, nrec, 0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + row0 * kv_stride), (short)0, nrec, 0x00020000);
    // K: load i covers rows (lane + 64 i) / (D / 8), whole rows across lanes; rows
    // before the left padding are loaded as they are (their scores are masked)
#pragma unroll
    for (int i = 0; i < T::KB; ++i) {
      const int blk = lane + 64 * i;
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rk, (blk / (D / 8)) * kv_row_bytes + 16 * (blk % (D / 8)), 0, kv_policy);
    }
#pragma unroll
    for (int bi = 0; bi < VB; ++bi) {
      const int blk = lane + 64 * bi;
      const int cg = blk % (D / 8), kg = blk / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int off = (4 * kg + r) * kv_row_bytes + 16 * cg;
        if (CACHE && 4 * kg + r < lo) off = nrec;
        vreg[bi][r] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kv_policy);
      }
    }
  };
  auto compute = [&](int j0, const u32x4 (&kreg)[T::KB], const u32x4 (&vreg)[VB][4]) {
    typedef __attribute__((address_space(3))) char lds_char;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    // K and V rows into this wavefront's LDS areas, as loaded
#pragma unroll
    for (int i = 0; i < T::KB; ++i) {
      const int blk = lane + 64 * i;
      const int r = blk / (D / 8);
      *reinterpret_cast<lds_u32x4*>((lds_char*)(uintptr_t)(
          wk + r * T::RSK + 16 * ((blk % (D / 8)) ^ T::kswz(r)))) = kreg[i];
    }
#pragma unroll
    for (int bi = 0; bi < VB; ++bi) {
      lds_char* row0 = (lds_char*)(uintptr_t)(wv + vw[bi]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<lds_u32x4*>(row0 + T::RS * r) = vreg[bi][r];
    }
    wave_lds_sync();
    // S^T = K . Q^T for the two 16-key blocks; lane element i is key j0 + 8 g4 + 4 kb + i.
    // A operand: K[krow0 + 4 kb][32 c + 8 g4 .. + 7]
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const int r = krow0 + 4 * kb;
        const u32x4 ka = *reinterpret_cast<const lds_u32x4*>((const lds_char*)(uintptr_t)(
            wk + r * T::RSK + 16 * ((4 * c + g4) ^ T::kswz(r))));
        sc[kb] = mfma16(ka, qf[c], sc[kb]);
      }
    }
    if constexpr (LOGIT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x;
          if constexpr (CAP) x = softcap2(sc[kb][i], p.cap_k, p.cap2);
          else x = sc[kb][i] * c2;
          if constexpr (ALIBI) {
            const int key = j0 + 8 * g4 + 4 * kb + i;
            x = __builtin_fmaf(-slope2, __builtin_fabsf((float)(diag_row - key)), x);
          }
          sc[kb][i] = x;
        }
    }
    if (j0 + TK > nomask_end || (CACHE && j0 < mask_below)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = j0 + 8 * g4 + 4 * kb + i;
          if (key >= Sk || key > row_lim || (CACHE && key < row_lo)) sc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = vmax(mx, sc[kb][i]);
    mx = vmax(mx, __shfl_xor(mx, 16));
    mx = vmax(mx, __shfl_xor(mx, 32));
    const float m_new = vmax(m_run, LOGIT ? mx : mx * c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float ls = -0.f;  // -0: the first add folds away
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = fast_exp2(__builtin_fmaf(sc[kb][i], LOGIT ? 1.f : c2, -m_use));
        sc[kb][i] = pe;
        ls += pe;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
    const u32x4 pf = pack8(sc[0][0], sc[0][1], sc[0][2], sc[0][3], sc[1][0], sc[1][1],
                           sc[1][2], sc[1][3]);
    // O^T += V^T . P^T; A operand: V^T[16 db + nr][8 g4 .. +7]
    static_for<D / 16>([&](auto DB) {
      constexpr int db = decltype(DB)::value;
      const u32x2 lo = ds_read_tr16_b64<32 * db>(wv + vr);
      const u32x2 hi = ds_read_tr16_b64<32 * db + 8 * T::RS>(wv + vr);
      oacc[db] = mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, oacc[db]);
    });
    wave_lds_sync();
  };
  // The prefetch is unconditional (a conditional one would make the compiler wait
  // for it before the current step): past the split's end it re-reads the current
  // step's rows, which the cache still holds.
  u32x4 kA[T::KB], vA[VB][4], kB[T::KB], vB[VB][4];
  int j0 = j_lo + wave * TK;
  if (j0 < j_hi) {
    load_kv(j0, kA, vA);
    while (true) {
      int j1 = j0 + NW * TK;
      load_kv(j1 < j_hi ? j1 : j0, kB, vB);
      compute(j0, kA, vA);
      if (j1 >= j_hi) break;
      j0 = j1;
      j1 = j0 + NW * TK;
      load_kv(j1 < j_hi ? j1 : j0, kA, vA);
      compute(j0, kB, vB);
      if (j1 >= j_hi) break;
      j0 = j1;
    }
  }

  // ---- merge the four wavefront states (same algebra as the split combine)
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  __syncthreads();
  float* cm = reinterpret_cast<float*>(smem);
  float* cl = cm + NW * 16;
  float* co = cl + NW * 16;
  if (g4 == 0) {
    cm[wave * 16 + nr] = m_run;
    cl[wave * 16 + nr] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    st16f(co + (wave * 16 + nr) * T::CD + 16 * db + 4 * g4, oacc[db]);
  __syncthreads();

  constexpr int DPT = D / 16;  // dcols per thread in the merge
  const int row = tid >> 4;
  const int dc0 = (tid & 15) * DPT;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = vmax(M, cm[w * 16 + row]);
  float wgt[NW];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wgt[w] = (M == -INFINITY) ? 0.f : fast_exp2(cm[w * 16 + row] - M);
    L += cl[w * 16 + row] * wgt[w];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float out[DPT];
#pragma unroll
  for (int c = 0; c < DPT; ++c) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc += co[(w * 16 + row) * T::CD + dc0 + c] * wgt[w];
    out[c] = acc * inv;
  }
  const float lse_val = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;

  const int Ro = mb * 16 + row;
  if (Ro < p.rows) {
    const int i = Ro / G, h = hk * G + Ro % G;
    float* dst;
    float* ldst;
    if (p.num_splits == 1) {
      dst = p.o + ((int64_t)b * Sq + i) * q_stride + (int64_t)h * D + dc0;
      ldst = p.lse + ((int64_t)b * p.Hq + h) * Sq + i;
    } else {
      const int64_t prow = (((int64_t)s * p.B + b) * p.Hq + h) * Sq + i;
      dst = p.o_accum + prow * D + dc0;
      ldst = p.lse_accum + prow;
    }
#pragma unroll
    for (int c = 0; c < DPT; c += 4) st16f(dst + c, f32x4{out[c], out[c + 1], out[c + 2], out[c + 3]});
    if ((tid & 15) == 0) *ldst = lse_val;
  }
#endif
}

}  // namespace ff
