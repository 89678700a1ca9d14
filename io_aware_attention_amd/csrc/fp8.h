// FP8 forward for gfx950: the fused attention kernel on the fp8 matrix cores
// ("FlashAttention 1, 2, 3" explainer, FlashAttention-3 precision section: FP8 inputs
// with a scale per block, the scales carried into the computation, softmax statistics
// in fp32).  Its inputs come from attn_quantize_fp8 (quantize.h): OCP E4M3 codes of
// the tensor's shape plus one fp32 scale per (b, h, block of 128 rows).
//
// attn_fwd_fp8: the prefill kernel's structure (one workgroup per 128-query tile,
// 64-key tiles through double-buffered LDS by direct buffer loads, software-pipelined
// key loop) with both products on v_mfma_f32_32x32x64_f8f6f4:
//   GEMM0  S^T = K . Q^T     A = K rows from LDS (32 bytes per lane), B = Q^T in VGPRs
//   GEMM1  O^T += V^T . P^T  A = V^T by ds_read_b64_tr_b8 on row-major V, B = P^T (fp8)
// Both operands of a product take their 32 k-slots per lane in the same order, so the
// instruction's internal k order does not matter.  Lane (query n, half H) receives the
// scores of keys 32 kb + 8 j + 4 H + i (element 16 kb + 4 j + i); its 32 probabilities
// are the B operand of the PV product as they stand, and the transposing V reads fetch
// exactly those keys (the source lane of each byte addresses the key row that the byte
// must hold).
//
// Scales: the Q tile's scale sq and the key tile's sk (tile t lies in scale block t / 2)
// fold into the exponent factor of the tile, c2_t = scale log2(e) sq sk_t.  V's block
// scale sv_t folds into the probabilities before rounding them to fp8:
// p~ = 2^(s c2_t - m + log2(sv_t / sv_max)) <= p <= 2^8 (the lazy reference point), and
// the row sum takes p = p~ sv_max / sv_t; the epilogue multiplies O by sv_max.
#pragma once
#include <utility>

#include "device.h"
#include "prefill.h"
#include "worklist.h"

namespace ff {

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* q_scale;  // [B, Hq, nqb]
  const float* k_scale;  // [B, Hkv, nkb]
  const float* v_scale;  // [B, Hkv, nkb]
  float* o;
  float* lse;
  int B, Sq, Sk, Hq, Hkv, G;
  int num_m, total, u_per;
  int nqb, nkb;
  float scale_log2;
};

template <int D>
struct Fp8Traits {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int kThreads = 256;
  static constexpr int ROWB = D;                   // bytes per K/V row in LDS
  static constexpr int CPR = D / 16;               // 16-byte chunks per row
  static constexpr int TILE = BN * ROWB;
  static constexpr int kLds = 4 * TILE;
  static constexpr int RPB = 256 / ROWB;           // rows per 256-byte bank line
  static constexpr int LOADS = BN * CPR / kThreads;
  // swizzle: physical chunk = logical chunk ^ key(row); rows 16 apart share a key.  Banks
  // span 256-byte lines (RPB rows); a 128-bit read serves 16 lanes (16 consecutive rows,
  // one logical chunk), a transposing read 32 lanes (rows {0..3, 8..11} + 4H of a 16-row
  // group, two adjacent chunks).  The key of line u must be one-to-one for the first and
  // spread the rows 0, 2, 8, 10 (lines 0, 1, 4, 5) over distinct chunk pairs for the second:
  // at d = 128 it is u with bits 0 and 1 swapped; at d = 64 (four rows a line) u itself.
  static __device__ __forceinline__ int key(int r) {
    const int u = (r / RPB) % CPR;
    return CPR == 8 ? ((u & 4) | ((u & 1) << 1) | ((u >> 1) & 1)) : u;
  }
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32 bytes of one fp8 MFMA operand, as two 16-byte halves.
struct Frag32 {
  u32x4 lo, hi;
};

__device__ __forceinline__ u32x4 lds_ld16(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)a);
}

// D(32x32) += A(32x64) * B(64x32) in fp8 E4M3.  Lane l supplies 32 bytes of row l%32
// of A and of column l%32 of B, over the same 32 k-slots.
__device__ __forceinline__ f32x16 mfma32_fp8(const Frag32& fa, const Frag32& fb, f32x16 c) {
  const i32x8 a = {(int)fa.lo[0], (int)fa.lo[1], (int)fa.lo[2], (int)fa.lo[3],
                   (int)fa.hi[0], (int)fa.hi[1], (int)fa.hi[2], (int)fa.hi[3]};
  const i32x8 b = {(int)fb.lo[0], (int)fb.lo[1], (int)fb.lo[2], (int)fb.lo[3],
                   (int)fb.hi[0], (int)fb.hi[1], (int)fb.hi[2], (int)fb.hi[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Wait states after fp8 32x32x64 MFMAs before plain vector instructions (or spills)
// read their results.  The compiler's count for this instruction was measured short: a
// copy of the last two accumulator registers, 19 wait states after the MFMA issued, read
// stale values.  Every place that reads these accumulators with vector instructions (the
// scores after QK^T, the O rescale, the epilogue) first passes through this drain, 96
// cycles, more than the instruction's 64.  The accumulators are in/out operands, so no
// read of them can be scheduled above it.
#define FF_FP8_DRAIN_NOPS                                                               \
  "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"               \
  "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
__device__ __forceinline__ void fp8_mfma_drain(f32x16& a, f32x16& b) {
  asm volatile(FF_FP8_DRAIN_NOPS : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void fp8_mfma_drain(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile(FF_FP8_DRAIN_NOPS : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
// The same instruction also reads its 32-byte A and B operands later than the compiler
// assumes: taking the sources as free right after the issue, it may write other values
// into them at once (a pipelined version of this kernel wrote a row maximum into the
// probability registers one instruction after the last PV product, and its last 32 dcols
// came out wrong).  So the operands of the last product of a block are kept live, as
// inputs of the statement below, through 64 more wait states.
#define FF_FP8_HOLD_NOPS "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
__device__ __forceinline__ void fp8_mfma_hold(const Frag32& a, const Frag32& b) {
  asm volatile(FF_FP8_HOLD_NOPS ::"v"(a.lo), "v"(a.hi), "v"(b.lo), "v"(b.hi));
}
// The result drain of two accumulators that also keeps the A operand of the last product
// (its B operand is a Q fragment, never written) live until it ends.
__device__ __forceinline__ void fp8_mfma_drain_hold(f32x16& a, f32x16& b, const Frag32& s) {
  asm volatile(FF_FP8_DRAIN_NOPS : "+v"(a), "+v"(b) : "v"(s.lo), "v"(s.hi));
}

template <int N>
__device__ __forceinline__ void fp8_mfma_drain(f32x16 (&acc)[N]) {
  static_assert(N == 2 || N == 4, "two or four accumulators");
  if constexpr (N == 2) fp8_mfma_drain(acc[0], acc[1]);
  else fp8_mfma_drain(acc[0], acc[1], acc[2], acc[3]);
}

// ds_read_b64_tr_b8 at LDS byte address a + OFF.  Within each group of 16 lanes, result
// lane i, byte j is byte (i & 7) of the 8 bytes that lane 2j + (i >> 3) addressed.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr8_b64(uint32_t a) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(uintptr_t)(a + OFF));
  return __builtin_bit_cast(u32x2, r);
}

// Four fp32 values to four E4M3 bytes (round to nearest even), a in the lowest byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 3) void attn_fwd_fp8(Fp8Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Fp8Traits<D>;
  constexpr int BM = T::BM, BN = T::BN, ROWB = T::ROWB, CPR = T::CPR, TILE = T::TILE;
  constexpr int LOADS = T::LOADS;
  constexpr int NC = D / 64;  // 64-wide slices of d (GEMM0 k steps)
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds];

  // ---- work item, in the order of the bf16 prefill kernel (units round-robin over XCDs,
  // heaviest query tiles first)
  const UnitItem item = unit_item(xcd_remap(blockIdx.x, p.total), p.u_per, p.num_m, p.G);
  const int unit = item.unit, mi = item.rank, hg = item.sub;
  if (unit >= p.B * p.Hkv) return;
  const int hk = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const int h = hk * p.G + hg;
  const int mblk = CAUSAL ? p.num_m - 1 - mi : mi;
  const int q0 = mblk * BM;
  const int Sq = p.Sq, Sk = p.Sk;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int H = lane >> 5;
  const int qrow = q0 + wave * 32 + n;

  const int nb_total = (Sk + BN - 1) / BN;
  int n_max = nb_total;
  const int last_q = (q0 + BM < Sq ? q0 + BM : Sq) - 1;
  if (CAUSAL) {
    const int lim = last_q + Sk - Sq;
    n_max = lim < 0 ? 0 : ((lim / BN + 1) < n_max ? lim / BN + 1 : n_max);
  }
  int n_mask_lo = (Sk % BN) ? nb_total - 1 : nb_total;
  if (CAUSAL) {
    const int first = q0 + Sk - Sq + 1;
    const int tm = first <= 0 ? 0 : first / BN;
    n_mask_lo = tm < n_mask_lo ? tm : n_mask_lo;
  }

  const int64_t q_stride = (int64_t)p.Hq * D;
  const int kv_row_bytes = p.Hkv * D;
  const int64_t lse_base = ((int64_t)b * p.Hq + h) * Sq;
  if (n_max <= 0) {
    if (qrow < Sq) {
      float* orow = p.o + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = H * 4; c < D; c += 8) st16f(orow + c, z);
      if (H == 0) p.lse[lse_base + qrow] = -INFINITY;
    }
    return;
  }

  // ---- scales: the Q tile's; the largest V block scale of this kv head
  const float* ks = p.k_scale + ((int64_t)b * p.Hkv + hk) * p.nkb;
  const float* vs = p.v_scale + ((int64_t)b * p.Hkv + hk) * p.nkb;
  const float c2q = p.scale_log2 * p.q_scale[((int64_t)b * p.Hq + h) * p.nqb + mblk];
  float sv_max;
  {
    float m = 0.f;
    for (int i = tid; i < p.nkb; i += T::kThreads) m = vmax(m, vs[i]);
#pragma unroll
    for (int s = 32; s >= 1; s /= 2) m = vmax(m, __shfl_xor(m, s));
    float* red = reinterpret_cast<float*>(smem);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    sv_max = vmax(vmax(red[0], red[1]), vmax(red[2], red[3]));
    __syncthreads();  // the LDS words are reused by the tiles
  }

  // ---- Q^T fragments: Q[qrow][64c + 32H .. +31] as two 16-byte halves
  Frag32 qf[NC];
  {
    const uint8_t* qp = p.q + ((int64_t)b * Sq + qrow) * q_stride + (int64_t)h * D + 32 * H;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c].lo = qrow < Sq ? ld16(qp + 64 * c) : z;
      qf[c].hi = qrow < Sq ? ld16(qp + 64 * c + 16) : z;
    }
    // in flight with the first K and V tiles; the first step's wait_vmem() retires them
  }

  // ---- direct HBM -> LDS loads of K and V tiles (as the bf16 kernel, 1-byte elements)
  const char* kbase = reinterpret_cast<const char*>(p.k) + ((int64_t)b * Sk * p.Hkv + hk) * D;
  const char* vbase = reinterpret_cast<const char*>(p.v) + ((int64_t)b * Sk * p.Hkv + hk) * D;
  int koff[LOADS];
#pragma unroll
  for (int k = 0; k < LOADS; ++k) {
    const int slot = 64 * (LOADS * wave + k) + lane;
    const int r = slot / CPR, ph = slot % CPR;
    koff[k] = r * kv_row_bytes + 16 * (ph ^ T::key(r));
  }
  const uint32_t smem_addr = lds_addr(smem);
  auto par = [&](int t) { return (n_max - 1 - t) & 1; };
  auto kbuf = [&](int t) { return smem_addr + par(t) * TILE; };
  auto issue = [&](const char* base, int t, uint32_t lds) {
    const int rows_left = t >= 0 ? Sk - t * BN : 0;
    const uint32_t bytes = (uint32_t)rows_left * (uint32_t)kv_row_bytes;
    const int64_t toff = t >= 0 ? (int64_t)t * BN * kv_row_bytes : 0;
    const i32x4 rd = buffer_desc(base + toff, bytes);
    const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds + 1024 * LOADS * wave);
#pragma unroll
    for (int k = 0; k < LOADS; ++k) buffer_load_lds16(rd, koff[k], l0 + 1024 * k);
  };

  // ---- LDS read addresses.  GEMM0: K row 32 kb + n, chunks 4c + 2H and 4c + 2H + 1.
  int ka[NC][2];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int x = 0; x < 2; ++x) ka[c][x] = n * ROWB + 16 * ((4 * c + 2 * H + x) ^ T::key(n));
  // GEMM1 (PV product db, transposing read r = 0..3 of its 32 bytes): in 16-lane group g
  // (half H = g / 2), source lane s addresses key row 16 r + 8 (s / 2 / 4) + (s / 2) % 4
  // + 4 H, dcols 32 db + 16 (g % 2) + 8 (s % 2); the swizzle key is the same for every r.
  const int g = lane >> 4, s = lane & 15;
  const int vrow = 8 * ((s >> 1) >> 2) + ((s >> 1) & 3) + 4 * H;
  int va[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    va[db] = vrow * ROWB + 16 * ((2 * db + (g & 1)) ^ T::key(vrow)) + 8 * (s & 1);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  auto kread = [&](uint32_t kl, int i) {  // fragment i = (c, kb): two 16-byte halves
    const int c = i >> 1, kb = i & 1;
    const uint32_t base = kl + kb * 32 * ROWB;
    return Frag32{lds_ld16(base + ka[c][0]), lds_ld16(base + ka[c][1])};
  };
  // QK^T of the K tile at kl, then the result drain (which also holds the K fragments of
  // the last two products).
  auto gemm0 = [&](uint32_t kl, f32x16* sc) {
    sc[0] = f32x16{};
    sc[1] = f32x16{};
    Frag32 kf;
#pragma unroll
    for (int i = 0; i < 2 * NC; ++i) {
      kf = kread(kl, i);
      sc[i & 1] = mfma32_fp8(kf, qf[i >> 1], sc[i & 1]);
    }
    fp8_mfma_drain_hold(sc[0], sc[1], kf);
  };
  // Score element e (block e / 16, index e % 16 = 4j + i) of tile t is key
  // t BN + 4H + key_off(e), key_off(e) = 32 (e / 16) + 8 j + i.
  auto key_off = [](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3); };
  const int last_key = CAUSAL && qrow + Sk - Sq < Sk - 1 ? qrow + Sk - Sq : Sk - 1;
  auto vis_lim = [&](int t) { return last_key - t * BN - 4 * H; };
  auto mask = [&](f32x16* sc, int t) {
    const int vl = vis_lim(t);
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (key_off(e) > vl) sc[e >> 4][e & 15] = -INFINITY;
  };
  auto rowmax = [&](const f32x16* sc) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = vmax(mx, sc[kb][e]);
    return max_xor32(mx);
  };
  // Per-tile constants: exponent factor, log2(sv / sv_max), sv_max / sv.  The last two
  // only scale probabilities, so the hardware log2 and reciprocal (about 1 ulp) serve;
  // IEEE divisions cost ~20 vector instructions per tile in a loop bound by vector work.
  struct TileScale {
    float c2, lr, ir;
  };
  // The block scales are held in registers, 64 blocks per window, lane l holding block
  // bhi - 64 w - l of window w, and read with readlane: a scale loaded at the top of its
  // step would make that step wait for the load's full latency (it joins the wait for
  // the tile's own loads), which cost up to half of each step.  A window is reloaded
  // once every 128 steps.
  const float inv_sv_max = 1.f / sv_max;
  const int bhi = (n_max - 1) >> 1;
  float ksw, vsw;
  auto load_window = [&](int w) {
    const int blk = bhi - 64 * w - lane;
    ksw = blk >= 0 ? ks[blk] : 0.f;
    vsw = blk >= 0 ? vs[blk] : 0.f;
  };
  load_window(0);
  auto tile_scale = [&](int t) {
    const int j = bhi - (t >> 1);  // wave-uniform
    if ((j & 63) == 0 && j > 0) load_window(j >> 6);
    const float sk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ksw), j & 63));
    const float sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vsw), j & 63));
    const float r = sv * inv_sv_max;
    return TileScale{c2q * sk, fast_log2(r), __builtin_amdgcn_rcpf(r)};
  };

  // ---- key loop, tiles n_max-1 down to 0: K and V of tile t-1 load while tile t is
  // computed (double-buffered LDS).  Each step is QK^T, then mask, row max and the
  // probabilities, then PV.  The two wavefronts sharing a SIMD overlap one's products
  // with the other's vector work.
  int t = n_max - 1;
  if ((t + 1) * BN > Sk) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < TILE / 16; i += T::kThreads) {
      st16(smem + 16 * i, z);
      st16(smem + 2 * TILE + 16 * i, z);
    }
    __syncthreads();
  }
  issue(kbase, t, kbuf(t));
  issue(vbase, t, smem_addr + (2 + par(t)) * TILE);

  constexpr int NG1 = D / 32;  // PV MFMAs per tile: one per 32 dcols
  auto step = [&](auto par_tag, int t, auto mask_tag) {
    constexpr int P = decltype(par_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    const TileScale ts = tile_scale(t);
    wait_vmem();          // this wave's share of tile t is in LDS
    __syncthreads();      // everyone's share; and tile t+1's buffers are free again
    issue(kbase, t - 1, smem_addr + (P ^ 1) * TILE);
    issue(vbase, t - 1, smem_addr + (2 + (P ^ 1)) * TILE);

    f32x16 sc[2];
    gemm0(smem_addr + P * TILE, sc);
    if constexpr (MASK) mask(sc, t);
    const float mx = rowmax(sc) * ts.c2;
    const bool raise = mx > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;
      m_run = raise ? mx : m_run;
      l_run *= alpha;
      fp8_mfma_drain(oacc);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    // p~ = 2^(s c2 - m + lr): the V block's scale ratio rides in the exponent
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    const float off = ts.lr - m_use;
    float lsum[2] = {-0.f, -0.f};  // -0: the first adds fold away
    Frag32 pb;
    static_for<8>([&](auto W) {  // four probabilities -> one dword of the B operand
      constexpr int w = decltype(W)::value, e0 = 4 * w;
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[q] = fast_exp2(__builtin_fmaf(sc[e0 >> 4][(e0 & 15) + q], ts.c2, off));
        lsum[q & 1] += x[q];
      }
      const uint32_t pk = pack_fp8x4(x[0], x[1], x[2], x[3]);
      if constexpr (w < 4) pb.lo[w] = pk;
      else pb.hi[w - 4] = pk;
    });
    l_run += (lsum[0] + lsum[1]) * ts.ir;

    const uint32_t vl = smem_addr + (2 + P) * TILE;
    Frag32 vf;
#pragma unroll
    for (int db = 0; db < NG1; ++db) {
      const uint32_t a = vl + va[db];
      const u32x2 r0 = ds_read_tr8_b64<0>(a), r1 = ds_read_tr8_b64<16 * ROWB>(a);
      const u32x2 r2 = ds_read_tr8_b64<32 * ROWB>(a), r3 = ds_read_tr8_b64<48 * ROWB>(a);
      vf = Frag32{u32x4{r0[0], r0[1], r1[0], r1[1]}, u32x4{r2[0], r2[1], r3[0], r3[1]}};
      oacc[db] = mfma32_fp8(vf, pb, oacc[db]);
    }
    fp8_mfma_hold(vf, pb);
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  using Yes = MaskTag<true>;
  using No = MaskTag<false>;
  // Masked tiles (key tail, causal diagonal) come first, in pairs so that each pair
  // starts at parity 0; masking a tile that needs none changes nothing.
  int n_masked = n_max - (n_mask_lo > 0 ? n_mask_lo : 0);
  n_masked = n_masked < 0 ? 0 : n_masked;
  for (int pair = 0; pair < (n_masked + 1) / 2 && t >= 1; ++pair, t -= 2) {
    step(Par0{}, t, Yes{});
    step(Par1{}, t - 1, Yes{});
  }
  for (; t >= 1; t -= 2) {
    step(Par0{}, t, No{});
    step(Par1{}, t - 1, No{});
  }
  if (t == 0) step(Par0{}, 0, Yes{});

  // ---- epilogue: O = sv_max o / l, LSE = (m + log2 l) ln 2.  The rows leave through LDS
  // as in the bf16 kernel, whole rows per store instruction with the non-temporal hint,
  // but in two passes of PD dcols: the tile buffers hold 32 rows of PD fp32 values per
  // wavefront.  Each staged row is a whole number of 128-byte lines, its 16-byte chunks
  // XOR-swizzled by row (both LDS passes free of bank conflicts).
  fp8_mfma_drain(oacc);
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? sv_max / l_tot : 0.f;
  constexpr int PD = T::kLds / (4 * 32 * 4);  // dcols per pass: 64 (d = 128), 32 (d = 64)
  constexpr int PCH = PD / 4;                 // 16-byte chunks per staged row
  constexpr int PROWB = PD * 4;               // bytes per staged row
  constexpr int RPI = 64 / PCH;               // rows per store instruction
  constexpr int DBP = PD / 32;                // accumulator blocks per pass
  static_assert(D % PD == 0 && PD % 32 == 0 && PCH <= 16, "staging passes");
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  wait_vmem();      // the last step's (empty) tile loads have retired: LDS is not written again
  __syncthreads();  // every wavefront is past its last read of the tiles
  const uint32_t ost = smem_addr + wave * 32 * PROWB;
  const int rr = lane / PCH, cc = lane % PCH;
  const int row0 = q0 + 32 * wave;
  float* obase = p.o + ((int64_t)b * Sq + row0) * q_stride + (int64_t)h * D + 4 * cc;
  static_for<D / PD>([&](auto PS) {
    constexpr int ps = decltype(PS)::value;
#pragma unroll
    for (int dbp = 0; dbp < DBP; ++dbp)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int db = ps * DBP + dbp;
        const f32x4 val = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                           oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
        const int c = 8 * dbp + 2 * j + H;  // dcols 32 db + 8 j + 4 H .. + 3 of this pass
        *reinterpret_cast<lds_f32x4*>((uintptr_t)(ost + n * PROWB + 16 * (c ^ (n & 7)))) = val;
      }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + rr;
      const f32x4 val =
          *reinterpret_cast<const lds_f32x4*>((uintptr_t)(ost + r * PROWB + 16 * (cc ^ (r & 7))));
      if (row0 + r < Sq) st16f_nt(obase + (int64_t)r * q_stride + ps * PD, val);
    }
    wave_lds_sync();  // the next pass rewrites the staged rows
  });
  if (qrow < Sq && H == 0)
    p.lse[lse_base + qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
#endif
}

}  // namespace ff
