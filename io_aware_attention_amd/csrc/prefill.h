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
//
// Variants (VAR != 0; the walk-through's Is_local, Has_alibi, Is_softcap).  With
// diag = i + Sk - Sq, key j is visible to query i iff diag - wl <= j <= diag + wr
// (-1: no limit), on top of the causal limit.  The window clips the key-tile range at
// both ends (the walk-through's n_block_min / n_block_max), so tiles are masked at the
// top (right edge, visited first) and at the bottom (left edge, visited last).  With
// ALiBi or the soft cap, each score is turned into its base-2 logit before the row
// maximum: the cap c log2(e) tanh(s scale / c), then the bias -slope |diag - j| log2(e).
#pragma once
#include <utility>

#include "device.h"
#include "tiles.h"
#include "worklist.h"

namespace ff {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv, G;  // G = Hq / Hkv
  int num_m;                  // query tiles per (batch, head)
  int total;                  // 8 * u_per * G * num_m workgroups
  int u_per;                  // (batch, kv head) unit slots per XCD: ceil(B * Hkv / 8)
  int snake;                  // CUs per XCD when the whole grid is resident at once, else 0
  float scale_log2;           // scale * log2(e)
  // Variable-length batches: when cu_q is set, q/o are [total_q, Hq, d], k/v are
  // [total_k, Hkv, d], sequence b owns rows cu_q[b] .. cu_q[b+1]-1 (keys: cu_k), Sq is
  // the longest query sequence, and lse is [Hq, total_q].
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // Variants: window limits (-1 = none); ALiBi slope of (batch b, head h) at
  // alibi[b * alibi_bstride + h]; soft-cap constants cap_k = 2 scale log2(e) / c and
  // cap2 = c log2(e).
  int wl, wr;
  const float* alibi;
  int alibi_bstride;
  float cap_k, cap2;
};

// Rows [start, start + len) of sequence b under prefix sums cu (clamped to [0, total],
// so that malformed sums cannot send any access out of the tensor).
__device__ __forceinline__ void seq_range(const int* cu, int b, int total, int* start, int* len) {
  int a = cu[b], e = cu[b + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
  *start = a;
  *len = e - a;
}

// Exponents stay within 2^kRescaleSlack of the stored reference point.
constexpr float kRescaleSlack = 8.0f;

template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};

// The two transposing reads of GEMM1 fragment i = (kb, db, cp): keys
// 32kb + 16cp + {0..3, 4..7} of the V tile, dcols 32db + lane's column.
template <int I, int D, int ROWB>
__device__ __forceinline__ void gemm1_read(uint32_t vbase, const int* va, u32x2& lo, u32x2& hi) {
  constexpr int NG1 = (D / 32) * 4;  // key block major: (kb, db, cp)
  constexpr int kb = I / (NG1 / 2), db = (I % (NG1 / 2)) / 2, cp = I % 2;
  constexpr int off = (32 * kb + 16 * cp) * ROWB;
  const uint32_t a = vbase + va[db];
  lo = ds_read_tr16_b64<off>(a);
  hi = ds_read_tr16_b64<off + 4 * ROWB>(a);
}

template <int D>
struct PrefillTraits {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int kThreads = 256;
  static constexpr int ROWB = D * 2;               // bytes per K/V row in LDS
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;           // bytes per K or V tile
  static constexpr int QTILE = BM * ROWB;          // bytes of the query tile
  // K and V, double buffered each; the query tile is loaded into V's second buffer and
  // the QTILE - TILE bytes after it, before that buffer's first V tile
  static constexpr int kLds = 3 * TILE + QTILE;
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte bank line
  static constexpr int LOADS = BN * CPR / kThreads;  // 16-byte loads per thread per tile
  static constexpr int QLOADS = BM * CPR / kThreads;  // the same for the query tile
  // swizzle keys: physical chunk = logical chunk ^ key(row)
  static __device__ __forceinline__ int kkey(int r) { return (r / RPB) % CPR; }
  static __device__ __forceinline__ int vkey(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

// Occupancy: two workgroups per CU at d = 128 (256 VGPRs); three at d = 64, where the
// kernel fits the 168 VGPRs that three waves per SIMD allow (32 KiB of LDS each).  A
// third slot per CU shortens the second, partly filled round of workgroups that grids
// slightly above 512 leave (2 x 5000 x 8 at d = 64: 640 workgroups).
template <int D, bool CAUSAL, int VAR>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void attn_fwd_prefill(FwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource builtins exist for the device target only
  constexpr bool WIN = VAR & kVarWindow, ALIBI = VAR & kVarAlibi, CAP = VAR & kVarSoftcap;
  constexpr bool LOGIT = ALIBI || CAP;  // scores become base-2 logits before the row max
  using T = PrefillTraits<D>;
  constexpr int BM = T::BM, BN = T::BN, ROWB = T::ROWB, CPR = T::CPR, TILE = T::TILE;
  constexpr int LOADS = T::LOADS;
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds];

  // ---- which (batch, head, query tile) this workgroup owns (the work list of
  // worklist.h: rank = query tile, heaviest first when causal; sub = query head)
  const UnitItem item = unit_item(work_index(blockIdx.x, p.total, p.snake), p.u_per, p.num_m, p.G);
  const int unit = item.unit, mi = item.rank, hg = item.sub;
  if (unit >= p.B * p.Hkv) return;
  const int hk = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const int h = hk * p.G + hg;
  const int mblk = CAUSAL ? p.num_m - 1 - mi : mi;  // heaviest causal tiles first
  const int q0 = mblk * BM;
  // this sequence's rows: q rows q_start .. q_start + Sq - 1, k/v rows k_start ..
  int q_start, Sq, k_start, Sk;
  int64_t lse_base;  // LSE index of the sequence's row 0 for this head
  if (p.cu_q) {
    seq_range(p.cu_q, b, p.total_q, &q_start, &Sq);
    seq_range(p.cu_k, b, p.total_k, &k_start, &Sk);
    lse_base = (int64_t)h * p.total_q + q_start;
  } else {
    q_start = b * p.Sq;
    Sq = p.Sq;
    k_start = b * p.Sk;
    Sk = p.Sk;
    lse_base = ((int64_t)b * p.Hq + h) * Sq;
  }
  if (q0 >= Sq) return;  // past the end of a shorter sequence

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query column of this lane in both products
  const int H = lane >> 5;   // which half of the wave
  const int qrow = q0 + wave * 32 + n;

  // ---- key-tile range (causal clipping: never visit tiles above the diagonal)
  const KeyTiles kt = key_tiles<BM, BN, CAUSAL, WIN>(q0, Sq, Sk, p.wl, p.wr);
  const int n_max = kt.n_max, n_mask_lo = kt.n_mask_lo, n_min = kt.n_min, n_bot = kt.n_bot;

  const int64_t q_stride = (int64_t)p.Hq * D;    // elements between query positions
  const int kv_row_bytes = p.Hkv * D * 2;        // bytes between key positions
  const float c2 = p.scale_log2;

  if (n_max <= n_min) {  // no visible key for any row of this tile
    if (qrow < Sq) {
      float* orow = p.o + ((int64_t)q_start + qrow) * q_stride + (int64_t)h * D;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = H * 4; c < D; c += 8) st16f(orow + c, z);
      if (H == 0) p.lse[lse_base + qrow] = -INFINITY;
    }
    return;
  }

  // ---- the query tile, straight into LDS like the K/V tiles below: whole rows per load
  // instruction (loading the Q^T fragments into registers directly takes 32 rows in
  // 32-byte pieces per instruction, four times the cache-line requests).  Rows past Sq
  // read as zeros.  Its loads stay in flight with the first K and V tiles'; each wave
  // reads its fragments once they have all landed.
  const uint32_t smem_addr = lds_addr(smem);
  const uint32_t qlds = smem_addr + 3 * TILE;
  u32x4 qf[D / 16];  // Q^T fragments (GEMM0 B operand), read from LDS before the first tile
  {
    const int q_row_bytes = p.Hq * D * 2;
    const int rows = Sq - q0 < BM ? Sq - q0 : BM;
    const char* qbase =
        reinterpret_cast<const char*>(p.q) + (((int64_t)q_start + q0) * p.Hq + h) * D * 2;
    const i32x4 qd = buffer_desc(qbase, (uint32_t)rows * (uint32_t)q_row_bytes);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(qlds + 1024 * T::QLOADS * wave);
#pragma unroll
    for (int k = 0; k < T::QLOADS; ++k) {
      const int slot = 64 * (T::QLOADS * wave + k) + lane;
      const int r = slot / CPR, ph = slot % CPR;
      buffer_load_lds16(qd, r * q_row_bytes + 16 * (ph ^ T::kkey(r)), l0 + 1024 * k);
    }
  }

  // ---- direct HBM -> LDS loads.  Wave w, load k fills the 1 KiB LDS block
  // LOADS*w + k: lane i writes chunk slot 64*(LOADS*w + k) + i, i.e. row slot/CPR,
  // physical chunk slot%CPR, which holds logical chunk (physical ^ key(row)).
  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)k_start * p.Hkv + hk) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)k_start * p.Hkv + hk) * D * 2;
  int koff[LOADS], voff[LOADS];
#pragma unroll
  for (int k = 0; k < LOADS; ++k) {
    const int slot = 64 * (LOADS * wave + k) + lane;
    const int r = slot / CPR, ph = slot % CPR;
    koff[k] = r * kv_row_bytes + 16 * (ph ^ T::kkey(r));
    voff[k] = r * kv_row_bytes + 16 * (ph ^ T::vkey(r));
  }
  // LDS: K tiles in buffers 0/1, V tiles in buffers 2/3.  Tiles are visited from
  // t = n_max - 1 down; tile t uses parity (n_max - 1 - t) & 1, so that the parity of
  // each step of the twice-unrolled key loop is a compile-time constant.
  auto par = [&](int t) { return (n_max - 1 - t) & 1; };
  auto kbuf = [&](int t) { return smem_addr + par(t) * TILE; };
  auto vbuf = [&](int t) { return smem_addr + (2 + par(t)) * TILE; };
  // Loads of tile t of K (or V) into its buffer.  A tile index below the range (below 0,
  // or below the window's first tile) gets an empty descriptor: every lane reads as out of
  // range, and the buffer is not read later.
  const int n_lo = WIN ? __builtin_amdgcn_readfirstlane(n_min) : 0;  // wave-uniform
  auto issue = [&](const char* base, const int* off, int t, uint32_t lds) {
    const int rows_left = t >= n_lo ? Sk - t * BN : 0;
    const uint32_t bytes = (uint32_t)rows_left * (uint32_t)kv_row_bytes;
    const int64_t toff = t >= n_lo ? (int64_t)t * BN * kv_row_bytes : 0;
    const i32x4 rd = buffer_desc(base + toff, bytes);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds + 1024 * LOADS * wave);
#pragma unroll
    for (int k = 0; k < LOADS; ++k) buffer_load_lds16(rd, off[k], l0 + 1024 * k);
  };
  auto issue_k = [&](int t) { issue(kbase, koff, t, kbuf(t)); };
  auto issue_v = [&](int t) { issue(vbase, voff, t, vbuf(t)); };

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

  // GEMM0: S^T for key blocks kb = 0, 1 (32 keys each) of the K tile at `kl`.
  auto gemm0 = [&](uint32_t kl, f32x16* sc) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(
            (const __attribute__((address_space(3))) char*)(uintptr_t)(kl + ka[c] + kb * 32 * ROWB));
        sc[kb] = mfma32(a, qf[c], sc[kb]);
      }
  };
  // Score element e (block e / 16, accumulator index e % 16 = 4j + i) of tile t is
  // key t*BN + 8H + key_off(e), key_off(e) = 32(e / 16) + 16(j >> 1) + 4(j & 1) + i.
  // The key is visible to row qrow iff it is below Sk and (causal) at most
  // qrow + Sk - Sq, that is iff key_off(e) <= vis_lim(t): one bound per tile against compile-time offsets.
  auto key_off = [](int e) {
    const int j = (e & 15) >> 2, i = e & 3;
    return 32 * (e >> 4) + 16 * (j >> 1) + 4 * (j & 1) + i;
  };
  int last_key = CAUSAL && qrow + Sk - Sq < Sk - 1 ? qrow + Sk - Sq : Sk - 1;
  int first_key = 0;  // window: keys below are invisible to this row
  if constexpr (WIN) {
    const int64_t diag = (int64_t)qrow + Sk - Sq;
    if (p.wr >= 0 && diag + p.wr < last_key) last_key = (int)(diag + p.wr);
    if (p.wl >= 0 && diag - p.wl > 0) first_key = (int)(diag - p.wl);
  }
  auto vis_lim = [&](int t) { return last_key - t * BN - 8 * H; };
  auto vis_lo = [&](int t) { return first_key - t * BN - 8 * H; };
  // The window's bottom tiles: key_off(e) < vis_lo(t) is invisible as well.
  auto mask = [&](f32x16* sc, int t) {
    const int vl = vis_lim(t);
    const int vlo = vis_lo(t);
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (key_off(e) > vl || (WIN && key_off(e) < vlo)) sc[e >> 4][e & 15] = -INFINITY;
  };
  // Variants: score -> base-2 logit (soft cap, then ALiBi bias).  rb = diag - (first key
  // of this lane's half of tile t), so key_off(e) is at distance rb - key_off(e).
  const float slope2 = ALIBI ? p.alibi[(int64_t)b * p.alibi_bstride + h] * kLog2e : 0.f;
  auto rbase = [&](int t) { return (float)(qrow + Sk - Sq - t * BN - 8 * H); };
  auto logit = [&](float s, int e, float rb) {
    float x;
    if constexpr (CAP) x = softcap2(s, p.cap_k, p.cap2);
    else x = s * c2;
    if constexpr (ALIBI) x = __builtin_fmaf(-slope2, __builtin_fabsf(rb - (float)key_off(e)), x);
    return x;
  };
  // Row maximum of a score tile in scale*log2(e) units (both wave halves).
  auto rowmax = [&](const f32x16* sc) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = vmax(mx, sc[kb][e]);
    return LOGIT ? max_xor32(mx) : max_xor32(mx) * c2;
  };
  const float cexp = LOGIT ? 1.f : c2;  // exponent factor of the stored scores
  // ---- software-pipelined key loop, tiles n_max-1 down to 0.  While tile t's
  // softmax and PV product run, tile t-1's QK^T product is issued (K streams one
  // tile ahead of V) and its row maximum is taken in the shadow of tile t's PV
  // product.  Masked tiles (key tail, causal diagonal) are the first ones visited.
  int t = n_max - 1;
  if ((t + 1) * BN > Sk) {
    // key tail: rows past Sk must read as zeros even if the loads leave them alone
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE / 16; i += T::kThreads) {
      st16(smem + 16 * i, z);  // parity 0: the first tile visited
      st16(smem + 2 * TILE + 16 * i, z);
    }
    __syncthreads();
  }
  issue_k(t);
  issue_v(t);
  issue_k(t - 1);
  // Masked steps: those whose next tile needs the element mask, rounded up to even.
  const int n_next = n_max - 1 - n_min;  // steps that have a next tile
  int n_masked = n_next - (n_mask_lo > n_min ? n_mask_lo - n_min : 0);
  n_masked = n_masked < 0 ? 0 : (n_masked > n_next ? n_next : n_masked);
  // On the causal diagonal the first tile visited can lie wholly right of every row of a
  // wavefront (the lower half of the query tile, when the tile edges line up).  Such a
  // wavefront skips that tile's products and exponentials; it still takes part in the
  // step's loads and barriers, and its state stays (m, l, o) = (-inf, 0, 0).  Only the
  // first pair of masked steps, which the loop below peels, can take this path.
  bool skip_first = false;
  if constexpr (CAUSAL) {
    const int w_rows_end = q0 + 32 * __builtin_amdgcn_readfirstlane(wave) + 32;  // wave-uniform
    const int w_last_row = (w_rows_end < Sq ? w_rows_end : Sq) - 1;
    skip_first = n_masked > 0 && t - n_min >= 2 && w_last_row + Sk - Sq < t * BN;
  }
  wait_vmem();  // this wave's share of the query tile and of the first tiles in LDS
  __syncthreads();
  // ---- Q^T fragments: Q[qrow][16c + 8H .. +7], logical chunk 2c + H of the tile's row
  // qrow - q0 (bank-conflict free, as the K rows)
  {
    const int rq = 32 * wave + n;
    const uint32_t qa = qlds + rq * ROWB;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[c] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          (uintptr_t)(qa + 16 * ((2 * c + H) ^ T::kkey(rq))));
  }
  // Scores of two consecutive tiles: in a step of parity P, S[P] holds tile t's and
  // S[P ^ 1] receives tile t-1's; the roles swap every step, so nothing is copied.
  f32x16 S[2][2];
  float mx = -INFINITY;
  if (!skip_first) {
    gemm0(kbuf(t), S[0]);
    if constexpr (LOGIT) {
      const float rb = rbase(t);
#pragma unroll
      for (int e = 0; e < 32; ++e) S[0][e >> 4][e & 15] = logit(S[0][e >> 4][e & 15], e, rb);
    }
    if (t >= n_mask_lo || t < n_bot) mask(S[0], t);
    mx = rowmax(S[0]);
  }
  // Every wave has read K of the first tile and its Q fragments before the first step
  // refills their buffers (the query tile lies in V's second buffer).
  __syncthreads();

  // One step (parity P): softmax + PV of tile t; QK^T, mask and row max of tile t-1
  // if HAS_NEXT.
  // The instruction order is fixed by hand: each group holds one MFMA, the LDS read
  // two MFMAs ahead, and a share of the softmax VALU work, and sched_barrier(0)
  // keeps the compiler from regrouping them (left alone it clusters the MFMAs and
  // issues every LDS read just before its use).
  constexpr int NG0 = 2 * (D / 16);  // GEMM0 MFMAs: (c, kb), kb fastest
  constexpr int NG1 = 4 * (D / 32);  // GEMM1 MFMAs: (kb, db, cp)
  auto step = [&](auto par_tag, int t, auto has_next_tag, auto mask_next_tag,
                  auto skip_tag) {
    constexpr int P = decltype(par_tag)::value;
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    constexpr bool MASK_NEXT = decltype(mask_next_tag)::value;
    constexpr bool SKIP = decltype(skip_tag)::value;  // no visible key of tile t here
    f32x16(&sc)[2] = S[P];
    f32x16(&sn)[2] = S[P ^ 1];
    // reference point for tile t: raise it (and rescale o, l) only past the slack
    const bool raise = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;  // 0 when m_run = -inf
      m_run = raise ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    if constexpr (HAS_NEXT) {
      issue(vbase, voff, t - 1, smem_addr + (2 + (P ^ 1)) * TILE);
      issue(kbase, koff, t - 2, smem_addr + P * TILE);
    }
    __builtin_amdgcn_sched_barrier(0);

    // -- block A: QK^T of tile t-1 interleaved with p = 2^(s c - m) of tile t.  It runs
    // at raised wave priority and block B at the base one: when the two wavefronts of a
    // SIMD compete, the one in the vector-heavy block issues first and the other's
    // products fill the matrix pipe (causal_prefill +2.5%, long_causal_gqa +3.2%; the
    // opposite assignment gained nothing).
    __builtin_amdgcn_s_setprio(1);
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    u32x4 kr[3];
    const uint32_t kl = smem_addr + (P ^ 1) * TILE;  // K of tile t-1
    auto kread = [&](int i) {
      const int c = i >> 1, kb = i & 1;
      return *reinterpret_cast<const u32x4*>(
          (const __attribute__((address_space(3))) char*)(uintptr_t)(kl + ka[c] + kb * 32 * ROWB));
    };
    if constexpr (HAS_NEXT) {
      kr[0] = kread(0);
      kr[1] = kread(1);
    }
    // partial row sums start at -0, the exact additive identity, so the first add of
    // each folds away (0 + x cannot be folded under IEEE rules: -0 + 0 = +0)
    float lsum[4] = {-0.f, -0.f, -0.f, -0.f};
    u32x4 pf[2][2];
    static_for<NG0>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (HAS_NEXT) {
        if constexpr (i + 2 < NG0) kr[(i + 2) % 3] = kread(i + 2);
        sn[i & 1] = mfma32(kr[i % 3], qf[i >> 1], sn[i & 1]);
      }
      constexpr int EPG = 32 / NG0;  // score elements per group
      if constexpr (!SKIP) {
#pragma unroll
        for (int q = 0; q < EPG; ++q) {
          const int e = i * EPG + q;  // 0..31: block e / 16, element e % 16
          const float x = fast_exp2(__builtin_fmaf(sc[e >> 4][e & 15], cexp, -m_use));
          sc[e >> 4][e & 15] = x;
          lsum[q & 3] += x;
        }
      }
      if constexpr (!SKIP && ((i + 1) * EPG) % 8 == 0) {  // eight more probabilities: pack them
        constexpr int e0 = (i + 1) * EPG - 8;
        const f32x16& b = sc[e0 >> 4];
        constexpr int o = e0 & 15;
        pf[e0 >> 4][o >> 3] = pack8(b[o], b[o + 1], b[o + 2], b[o + 3], b[o + 4], b[o + 5], b[o + 6], b[o + 7]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (!SKIP) l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);

    // -- block B: PV of tile t interleaved with mask and row max of tile t-1
    __builtin_amdgcn_s_setprio(0);
    const uint32_t vl = smem_addr + (2 + P) * TILE;  // V of tile t
    u32x2 flo[3], fhi[3];
    if constexpr (!SKIP) {
      gemm1_read<0, D, ROWB>(vl, va, flo[0], fhi[0]);
      gemm1_read<1, D, ROWB>(vl, va, flo[1], fhi[1]);
    }
    const int vln = vis_lim(t - 1);
    const int vlon = vis_lo(t - 1);
    const float rbn = LOGIT ? rbase(t - 1) : 0.f;
    float mxn = -INFINITY;
    static_for<NG1>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (!SKIP) {
        if constexpr (i + 2 < NG1)
          gemm1_read<i + 2, D, ROWB>(vl, va, flo[(i + 2) % 3], fhi[(i + 2) % 3]);
        const u32x4 a = {flo[i % 3][0], flo[i % 3][1], fhi[i % 3][0], fhi[i % 3][1]};
        constexpr int kb = i / (NG1 / 2), db = (i % (NG1 / 2)) / 2, cp = i % 2;
        oacc[db] = mfma32(a, pf[kb][cp], oacc[db]);
      }
      if constexpr (HAS_NEXT) {
        constexpr int EPG = 32 / NG1;
#pragma unroll
        for (int q = 0; q < EPG; ++q) {
          const int e = i * EPG + q;
          if constexpr (LOGIT) sn[e >> 4][e & 15] = logit(sn[e >> 4][e & 15], e, rbn);
          if constexpr (MASK_NEXT) {
            if (key_off(e) > vln || (WIN && key_off(e) < vlon)) sn[e >> 4][e & 15] = -INFINITY;
          }
          mxn = vmax(mxn, sn[e >> 4][e & 15]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (HAS_NEXT) {
      mx = LOGIT ? max_xor32(mxn) : max_xor32(mxn) * c2;
      wait_vmem();
      __syncthreads();
    }
  };
  // The loop runs in pairs of steps (parity 0, then 1).  Masked tiles (key tail,
  // causal diagonal, window right edge) are the first ones visited: steps t with
  // t - 1 >= n_mask_lo mask the next tile, and their number is rounded up to even
  // (masking a tile that needs none changes nothing), so every pair loop starts at
  // parity 0 and the mask code stays out of the main loop.  The window's left-edge tiles
  // (below n_bot) come last, again in masked pairs.
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  using Yes = MaskTag<true>;
  using No = MaskTag<false>;
  int pair = 0;
  if (n_masked > 0 && t - n_min >= 2) {  // the first masked pair, peeled
    if (skip_first) step(Par0{}, t, Yes{}, Yes{}, Yes{});
    else step(Par0{}, t, Yes{}, Yes{}, No{});
    step(Par1{}, t - 1, Yes{}, Yes{}, No{});
    pair = 1;
    t -= 2;
  }
  for (; pair < (n_masked + 1) / 2 && t - n_min >= 2; ++pair, t -= 2) {
    step(Par0{}, t, Yes{}, Yes{}, No{});
    step(Par1{}, t - 1, Yes{}, Yes{}, No{});
  }
  for (; t - 2 >= n_bot; t -= 2) {  // both next tiles lie at or above n_bot
    step(Par0{}, t, Yes{}, No{}, No{});
    step(Par1{}, t - 1, Yes{}, No{}, No{});
  }
  if constexpr (WIN) {
    for (; t - n_min >= 2; t -= 2) {
      step(Par0{}, t, Yes{}, Yes{}, No{});
      step(Par1{}, t - 1, Yes{}, Yes{}, No{});
    }
  }
  if (t - n_min == 1) {
    step(Par0{}, n_min + 1, Yes{}, Yes{}, No{});
    step(Par1{}, n_min, No{}, No{}, No{});
  } else {
    step(Par0{}, n_min, No{}, No{}, No{});
  }

  // ---- epilogue: O = o / l, LSE = (m + log2 l) ln 2.  The rows leave through LDS: each
  // wavefront stages its 32 normalised O rows in its own quarter of the tile buffers (all
  // free once every wave is past its last step), the 16-byte chunks XOR-swizzled by row,
  // and then stores whole rows, two (d = 128) or four (d = 64) per instruction, where
  // storing from the product's layout writes 32 rows in 32-byte pieces per instruction.
  // Both LDS passes are free of bank conflicts.  The row stores carry the non-temporal
  // hint: written once, O then streams through L2 without displacing the K/V tiles the
  // other workgroups are reading (causal_prefill 274 -> 265 us, its memory latencies
  // shorter in every phase of a workgroup).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int CH = D / 4;     // 16-byte chunks per O row
  constexpr int OROWB = D * 4;  // bytes per O row
  constexpr int RPI = 64 / CH;  // rows per store instruction
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  __syncthreads();
  const uint32_t ost = smem_addr + wave * 32 * OROWB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 val = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                         oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
      const int c = 8 * db + 2 * j + H;  // dcols 32 db + 8 j + 4 H .. + 3
      *reinterpret_cast<lds_f32x4*>((uintptr_t)(ost + n * OROWB + 16 * (c ^ (n & 7)))) = val;
    }
  wave_lds_sync();
  const int rr = lane / CH, cc = lane % CH;
  const int row0 = q0 + 32 * wave;
  float* obase = p.o + ((int64_t)q_start + row0) * q_stride + (int64_t)h * D + 4 * cc;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + rr;
    const f32x4 val =
        *reinterpret_cast<const lds_f32x4*>((uintptr_t)(ost + r * OROWB + 16 * (cc ^ (r & 7))));
    if (row0 + r < Sq) st16f_nt(obase + (int64_t)r * q_stride, val);
  }
  if (qrow < Sq && H == 0)
    p.lse[lse_base + qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
#endif
}

}  // namespace ff
