// libflashfwd: C-ABI entry points (declared in include/flashfwd.h).
//
// Host side of the attention forward path: argument checks, the tile and split
// plans, and kernel launches on the caller's stream.  No allocation, no
// synchronisation, no fallback: every step of the path runs in the kernels of
// prefill.h and splitkv.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>

#include "flashfwd.h"
#include "prefill.h"
#include "splitkv.h"
#include "combine.h"
#include "append.h"
#include "backward.h"
#include "quantize.h"
#include "fp8.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;
constexpr int kSplitRows = ff::SplitTraits<128>::BMD;  // folded rows per split workgroup
// Split workgroups counted per CU.  The split kernel keeps its next key step in
// flight, so one workgroup streams at close to a CU's share of HBM bandwidth; a
// second, partial round of workgroups costs more than it gains.
constexpr int kSplitWgPerCu = 1;
constexpr int kMinBlocksPerSplit = 4;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Opt-in trace of the host's plans: with FLASHFWD_LOG set to anything but "0", every
// launch prints its kernel, grid and tiling or split decisions on stderr.
bool log_on() {
  static const bool on = [] {
    const char* e = getenv("FLASHFWD_LOG");
    return e && *e && !(e[0] == '0' && e[1] == 0);
  }();
  return on;
}

__attribute__((format(printf, 1, 2))) void plan_log(const char* fmt, ...) {
  if (!log_on()) return;
  va_list ap;
  va_start(ap, fmt);
  fputs("[flashfwd] ", stderr);
  vfprintf(stderr, fmt, ap);
  fputc('\n', stderr);
  va_end(ap);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Shape checks shared by the forward entry points.
int check_dims(int B, int Sq, int Sk, int Hq, int Hkv, int d) {
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1) return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FF_ERR_GQA;
  if ((int64_t)B * Sq * Hq * d >= kMaxElems || (int64_t)B * Sk * Hkv * d >= kMaxElems)
    return FF_ERR_SHAPE;
  return FF_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Cache geometry shared by attn_fwd_kvcache and attn_kvcache_append.  With a block table
// the caches hold num_blocks blocks of page_size positions (page_size a multiple of 32)
// and a batch addresses max_blocks_per_seq of them; without one they are [B, page_size,
// ...] and the other two sizes are ignored.  `extra` new keys must fit on top of a full
// cache in an int.  Returns the block count and a batch's capacity in positions.
int check_cache(int B, int Hkv, const int* block_table, int num_blocks, int page_size,
                int max_blocks_per_seq, int extra, int64_t* blocks, int64_t* cap) {
  if (B < 1 || Hkv < 1 || page_size < 1 || extra < 0) return FF_ERR_SHAPE;
  if (block_table) {
    if (num_blocks < 1 || max_blocks_per_seq < 1 || page_size % 32 != 0) return FF_ERR_SHAPE;
    *blocks = num_blocks;
    *cap = (int64_t)max_blocks_per_seq * page_size;
  } else {
    *blocks = B;
    *cap = page_size;
  }
  if (*cap + extra >= kMaxElems || *blocks * page_size >= kMaxElems) return FF_ERR_SHAPE;
  return FF_OK;
}

int check_scale(float scale) {
  if (!isfinite(scale) || !(scale > 0.f)) return FF_ERR_SCALE;
  return FF_OK;
}

int check_io(const void* q, const void* k, const void* v, int B, int Sq, int Sk, int Hq,
             int Hkv, int d, const void* const* outs, const int64_t* out_bytes, int nout) {
  const int64_t qb = (int64_t)B * Sq * Hq * d * 2, kvb = (int64_t)B * Sk * Hkv * d * 2;
  for (int i = 0; i < nout; ++i) {
    if (overlaps(outs[i], out_bytes[i], q, qb) || overlaps(outs[i], out_bytes[i], k, kvb) ||
        overlaps(outs[i], out_bytes[i], v, kvb))
      return FF_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FF_ERR_ALIAS;
  }
  return FF_OK;
}

std::atomic<int> g_cu_count[64];

int device_cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FF_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return FF_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
    return FF_ERR_HIP;
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *out = c;
  return FF_OK;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? FF_OK : FF_ERR_HIP;
}

// Mask and bias options of the _ex entry points, checked, with the variant kernel that
// serves them (0 = none set: the plain kernel).
struct Variant {
  int wl = -1, wr = -1;
  const float* alibi = nullptr;
  int alibi_bstride = 0;
  float softcap = 0.f;
  int var = 0;
};

int check_variant(int window_left, int window_right, const float* alibi_slopes,
                  int alibi_batch_stride, float softcap, int Hq, Variant* v) {
  if (window_left < -1 || window_right < -1) return FF_ERR_OPTION;
  if (!isfinite(softcap) || softcap < 0.f) return FF_ERR_OPTION;
  if (alibi_slopes && alibi_batch_stride != 0 && alibi_batch_stride != Hq) return FF_ERR_OPTION;
  if (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)) return FF_ERR_ALIGN;
  v->wl = window_left;
  v->wr = window_right;
  v->alibi = alibi_slopes;
  v->alibi_bstride = alibi_slopes ? alibi_batch_stride : 0;
  v->softcap = softcap;
  const bool any = window_left >= 0 || window_right >= 0 || alibi_slopes || softcap > 0.f;
  v->var = any ? ff::kVarWindow | (alibi_slopes ? ff::kVarAlibi : 0) |
                     (softcap > 0.f ? ff::kVarSoftcap : 0)
               : 0;
  return FF_OK;
}

// The slopes an ALiBi call reads: [B, Hq] or [Hq].
int64_t alibi_bytes(const Variant& v, int B, int Hq) {
  if (!v.alibi) return 0;
  return (v.alibi_bstride ? (int64_t)B * Hq : (int64_t)Hq) * 4;
}

template <typename P>
void set_variant(P& p, const Variant& v, float scale) {
  p.wl = v.wl;
  p.wr = v.wr;
  p.alibi = v.alibi;
  p.alibi_bstride = v.alibi_bstride;
  p.cap_k = v.softcap > 0.f ? 2.f * scale * ff::kLog2e / v.softcap : 0.f;
  p.cap2 = v.softcap * ff::kLog2e;
}

// dQ first: its prologue writes each row's D and base-2 LSE into ws, which the dK/dV
// kernel reads.  var: 0, or the window with or without ALiBi (no soft cap).
template <int D, bool CAUSAL, int VAR>
void launch_bwd_var(dim3 g_dq, dim3 g_dkdv, hipStream_t s, const ff::BwdParams& p) {
  hipLaunchKernelGGL((ff::attn_bwd_dq<D, CAUSAL, VAR>), g_dq, dim3(256), 0, s, p);
  hipLaunchKernelGGL((ff::attn_bwd_dkdv<D, CAUSAL, VAR>), g_dkdv, dim3(512), 0, s, p);
}

template <int D>
void launch_bwd(bool causal, int var, dim3 g_dq, dim3 g_dkdv, hipStream_t s,
                const ff::BwdParams& p) {
  using namespace ff;
  plan_log("attn_bwd d=%d causal=%d var=%d: attn_bwd_dq %u workgroups of 256 threads, then "
           "attn_bwd_dkdv %u workgroups of 512 threads", D, (int)causal, var, g_dq.x, g_dkdv.x);
  constexpr int W = kVarWindow, WA = kVarWindow | kVarAlibi;
  if (causal) {
    if (var == 0) launch_bwd_var<D, true, 0>(g_dq, g_dkdv, s, p);
    else if (var == W) launch_bwd_var<D, true, W>(g_dq, g_dkdv, s, p);
    else launch_bwd_var<D, true, WA>(g_dq, g_dkdv, s, p);
  } else {
    if (var == 0) launch_bwd_var<D, false, 0>(g_dq, g_dkdv, s, p);
    else if (var == W) launch_bwd_var<D, false, W>(g_dq, g_dkdv, s, p);
    else launch_bwd_var<D, false, WA>(g_dq, g_dkdv, s, p);
  }
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case FF_OK: return "ok";
    case FF_ERR_NULL: return "a required pointer is NULL";
    case FF_ERR_SHAPE: return "invalid or too large shape (B, Sq, Sk, Hq, Hkv)";
    case FF_ERR_HEADDIM: return "head dimension must be 64 or 128";
    case FF_ERR_GQA: return "Hq must be a multiple of Hkv";
    case FF_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case FF_ERR_SPLITS: return "num_splits must be in [1, FF_MAX_SPLITS]";
    case FF_ERR_SCALE: return "scale must be finite and positive";
    case FF_ERR_HIP: return "HIP runtime error";
    case FF_ERR_ALIAS: return "an output buffer overlaps another buffer";
    case FF_ERR_OPTION:
      return "invalid mask/bias option (window < -1, softcap < 0 or not finite, "
             "or ALiBi batch stride not 0 or Hq)";
    case FF_ERR_SCRATCH:
      return "the split partials need more than FF_NOALLOC_SCRATCH_FLOATS floats";
    default: return "unknown status";
  }
}

long long attn_bwd_workspace_floats(int B, int Sq, int Hq) {
  if (B < 1 || Sq < 1 || Hq < 1) return -FF_ERR_SHAPE;
  return 2LL * B * Hq * cdiv(Sq, 64) * 64;
}

int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, float* ws, int B, int Sq,
                int Sk, int Hq, int Hkv, int d, int causal, int window_left, int window_right,
                const float* alibi_slopes, int alibi_batch_stride, float softcap, float scale,
                void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !ws) return FF_ERR_NULL;
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return st;
  Variant var;
  if ((st = check_variant(window_left, window_right, alibi_slopes, alibi_batch_stride, softcap,
                          Hq, &var)))
    return st;
  if (var.softcap > 0.f) return FF_ERR_OPTION;  // the backward takes no soft cap
  const void* ptrs[10] = {q, k, v, o, lse, dout, dq, dk, dv, ws};
  for (const void* x : ptrs)
    if (!aligned16(x)) return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const int64_t sq_pad = cdiv(Sq, 64) * 64;
  const int64_t qf32 = (int64_t)B * Sq * Hq * d * 4, kvf32 = (int64_t)B * Sk * Hkv * d * 4;
  const int64_t wsb = 2 * (int64_t)B * Hq * sq_pad * 4;
  const void* outs[4] = {dq, dk, dv, ws};
  const int64_t ob[4] = {qf32, kvf32, kvf32, wsb};
  if ((st = check_io(q, k, v, B, Sq, Sk, Hq, Hkv, d, outs, ob, 4))) return st;
  const int64_t in_b[3] = {qf32, (int64_t)B * Hq * Sq * 4, (int64_t)B * Sq * Hq * d * 2};
  const void* ins[3] = {o, lse, dout};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], ob[i], ins[j], in_b[j])) return FF_ERR_ALIAS;
    if (var.alibi && overlaps(outs[i], ob[i], var.alibi, alibi_bytes(var, B, Hq)))
      return FF_ERR_ALIAS;
  }

  ff::BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.dout = (const uint16_t*)dout;
  p.o = o;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dsum = ws;
  p.lse2 = ws + (int64_t)B * Hq * sq_pad;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.sq_pad = (int)sq_pad;
  p.num_m = (int)cdiv(Sq, 128);
  p.num_n = (int)cdiv(Sk, 128);
  p.u_per = (int)cdiv((int64_t)B * Hkv, 8);
  const int64_t n_dq = 8 * (int64_t)p.u_per * p.G * p.num_m;  // unit slots of all 8 XCDs
  const int64_t n_dkdv = 8 * (int64_t)p.u_per * p.num_n;
  if (n_dq >= kMaxElems || n_dkdv >= kMaxElems) return FF_ERR_SHAPE;
  p.scale = scale;
  p.scale_log2 = scale * ff::kLog2e;
  p.wl = var.wl;
  p.wr = var.wr;
  p.alibi = var.alibi;
  p.alibi_bstride = var.alibi_bstride;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g_dq((unsigned)n_dq);
  const dim3 g_dkdv((unsigned)n_dkdv);
  if (d == 128) launch_bwd<128>(causal != 0, var.var, g_dq, g_dkdv, s, p);
  else launch_bwd<64>(causal != 0, var.var, g_dq, g_dkdv, s, p);
  return launch_status();
}

int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, float* ws, int B, int Sq, int Sk,
             int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Sq, Sk, Hq, Hkv, d, causal, -1,
                     -1, nullptr, 0, 0.f, scale, stream);
}

}  // extern "C"

namespace {

template <int D, bool CAUSAL>
void launch_prefill_var(int var, dim3 grid, dim3 block, hipStream_t s, const ff::FwdParams& p) {
  using namespace ff;
  switch (var) {
    case 0: hipLaunchKernelGGL((attn_fwd_prefill<D, CAUSAL, 0>), grid, block, 0, s, p); break;
    case kVarWindow:
      hipLaunchKernelGGL((attn_fwd_prefill<D, CAUSAL, kVarWindow>), grid, block, 0, s, p);
      break;
    case kVarWindow | kVarAlibi:
      hipLaunchKernelGGL((attn_fwd_prefill<D, CAUSAL, kVarWindow | kVarAlibi>), grid, block, 0,
                         s, p);
      break;
    case kVarWindow | kVarSoftcap:
      hipLaunchKernelGGL((attn_fwd_prefill<D, CAUSAL, kVarWindow | kVarSoftcap>), grid, block,
                         0, s, p);
      break;
    default:
      hipLaunchKernelGGL((attn_fwd_prefill<D, CAUSAL, kVarWindow | kVarAlibi | kVarSoftcap>),
                         grid, block, 0, s, p);
      break;
  }
}

// Fills the work-list fields of p (B, Sq = longest query sequence, Hq, Hkv set) and
// launches the prefill kernel (the variant kernel var; p's variant fields set).
int launch_prefill(ff::FwdParams& p, int d, int causal, float scale, void* stream, int var = 0) {
  p.G = p.Hq / p.Hkv;
  p.num_m = (int)cdiv(p.Sq, ff::PrefillTraits<128>::BM);
  p.u_per = (int)cdiv((int64_t)p.B * p.Hkv, 8);
  const int64_t total = 8 * (int64_t)p.u_per * p.G * p.num_m;  // unit slots of all 8 XCDs
  if (total >= kMaxElems) return FF_ERR_SHAPE;
  p.total = (int)total;
  p.scale_log2 = scale * ff::kLog2e;
  // Causal grids that are resident all at once (two workgroups per CU at d = 128, three at
  // d = 64) take their items in snake order over the CUs of each XCD.
  p.snake = 0;
  if (causal) {
    int cus = 0;
    const int st = device_cu_count(&cus);
    if (st) return st;
    if (cus % 8 == 0 && total <= (int64_t)cus * (d == 64 ? 3 : 2)) p.snake = cus / 8;
  }
  plan_log("attn_fwd_prefill d=%d causal=%d var=%d%s: %lld workgroups of 256 threads, "
           "query tiles of 128 rows x key tiles of 64, %d query tiles x %d unit slots per XCD "
           "x %d query heads per kv head, snake=%d", d, causal, var, p.cu_q ? " varlen" : "",
           (long long)total, p.num_m, p.u_per, p.G, p.snake);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)total), block(256);
  if (d == 128) {
    if (causal) launch_prefill_var<128, true>(var, grid, block, s, p);
    else launch_prefill_var<128, false>(var, grid, block, s, p);
  } else {
    if (causal) launch_prefill_var<64, true>(var, grid, block, s, p);
    else launch_prefill_var<64, false>(var, grid, block, s, p);
  }
  return launch_status();
}

int fwd_dense(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Sq,
              int Sk, int Hq, int Hkv, int d, int causal, float scale, const Variant& var,
              void* stream) {
  if (!q || !k || !v || !o || !lse) return FF_ERR_NULL;
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const void* outs[2] = {o, lse};
  const int64_t ob[2] = {(int64_t)B * Sq * Hq * d * 4, (int64_t)B * Hq * Sq * 4};
  if ((st = check_io(q, k, v, B, Sq, Sk, Hq, Hkv, d, outs, ob, 2))) return st;
  for (int i = 0; i < 2; ++i)
    if (overlaps(outs[i], ob[i], var.alibi, alibi_bytes(var, B, Hq))) return FF_ERR_ALIAS;

  ff::FwdParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.cu_q = p.cu_k = nullptr;
  set_variant(p, var, scale);
  return launch_prefill(p, d, causal, scale, stream, var.var);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Sq,
             int Sk, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  return fwd_dense(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale, Variant{}, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                int Sq, int Sk, int Hq, int Hkv, int d, int causal, int window_left,
                int window_right, const float* alibi_slopes, int alibi_batch_stride,
                float softcap, float scale, void* stream) {
  Variant var;
  int st = check_variant(window_left, window_right, alibi_slopes, alibi_batch_stride, softcap,
                         Hq, &var);
  if (st) return st;
  return fwd_dense(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, d, causal, scale, var, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                    int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                    void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FF_ERR_NULL;
  if (B < 1 || max_seqlen_q < 1 || total_q < 1 || total_k < 1 || Hq < 1 || Hkv < 1)
    return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FF_ERR_GQA;
  if ((int64_t)total_q * Hq * d >= kMaxElems || (int64_t)total_k * Hkv * d >= kMaxElems ||
      max_seqlen_q > total_q)
    return FF_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      ((uintptr_t)cu_seqlens_q & 3u) || ((uintptr_t)cu_seqlens_k & 3u))
    return FF_ERR_ALIGN;
  int st = check_scale(scale);
  if (st) return st;
  // As a [1, total, H, d] problem for the overlap checks.
  const void* outs[2] = {o, lse};
  const int64_t ob[2] = {(int64_t)total_q * Hq * d * 4, (int64_t)Hq * total_q * 4};
  if ((st = check_io(q, k, v, 1, total_q, total_k, Hq, Hkv, d, outs, ob, 2))) return st;
  for (int i = 0; i < 2; ++i)
    if (overlaps(outs[i], ob[i], cu_seqlens_q, (int64_t)(B + 1) * 4) ||
        overlaps(outs[i], ob[i], cu_seqlens_k, (int64_t)(B + 1) * 4))
      return FF_ERR_ALIAS;

  ff::FwdParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = max_seqlen_q;
  p.Sk = 0;  // per sequence
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  return launch_prefill(p, d, causal, scale, stream);
}

int attn_splits_efficiency_rule(int units, int slots, int max_splits) {
  if (units < 1 || slots < 1 || max_splits < 1) return -FF_ERR_SHAPE;
  double best = 0.0;
  for (int S = 1; S <= max_splits; ++S) {
    const double w = (double)units * S / slots;
    const double eff = w / ceil(w);
    if (eff > best) best = eff;
  }
  for (int S = 1; S <= max_splits; ++S) {
    const double w = (double)units * S / slots;
    if (w / ceil(w) >= 0.85 * best) return S;
  }
  return 1;
}

int attn_splitkv_num_splits(int B, int Sq, int Sk, int Hq, int Hkv, int d, int num_cus) {
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return -st;
  // benchmark sweeps: FLASHFWD_NUM_SPLITS=n (1 .. FF_MAX_SPLITS) replaces the rule
  if (const char* e = getenv("FLASHFWD_NUM_SPLITS")) {
    char* end = nullptr;
    const long n = strtol(e, &end, 10);
    if (end != e && *end == 0 && n >= 1 && n <= FF_MAX_SPLITS) {
      plan_log("attn_splitkv_num_splits: %ld from FLASHFWD_NUM_SPLITS", n);
      return (int)n;
    }
  }
  if (num_cus <= 0 && (st = device_cu_count(&num_cus))) return -st;
  const int64_t rows = (int64_t)Sq * (Hq / Hkv);
  const int64_t units = (int64_t)B * Hkv * cdiv(rows, kSplitRows);
  const int64_t nblocks = cdiv(Sk, FF_SPLIT_BLOCK_N);
  int64_t max_splits = nblocks / kMinBlocksPerSplit;
  if (max_splits > FF_MAX_SPLITS) max_splits = FF_MAX_SPLITS;
  if (max_splits < 1) max_splits = 1;
  const int64_t slots = (int64_t)num_cus * kSplitWgPerCu;
  const int n = units >= slots
                    ? 1
                    : attn_splits_efficiency_rule((int)units, (int)slots, (int)max_splits);
  plan_log("attn_splitkv_num_splits: %d (%lld workgroups per split, %lld slots, at most %lld "
           "splits)", n, (long long)units, (long long)slots, (long long)max_splits);
  return n;
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, float* o_accum,
                     float* lse_accum, float* o, float* lse, int B, int Sq, int Sk, int Hq,
                     int Hkv, int d, int causal, float scale, int num_splits, void* stream) {
  if (!q || !k || !v) return FF_ERR_NULL;
  if (num_splits < 1 || num_splits > FF_MAX_SPLITS) return FF_ERR_SPLITS;
  if (num_splits == 1 && (!o || !lse)) return FF_ERR_NULL;
  if (num_splits > 1 && (!o_accum || !lse_accum)) return FF_ERR_NULL;
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return FF_ERR_ALIGN;
  if (num_splits == 1 && (!aligned16(o) || !aligned16(lse))) return FF_ERR_ALIGN;
  if (num_splits > 1 && (!aligned16(o_accum) || !aligned16(lse_accum))) return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const int64_t rows_all = (int64_t)B * Hq * Sq;
  if ((int64_t)num_splits * rows_all * d >= kMaxElems) return FF_ERR_SHAPE;
  if (num_splits == 1) {
    const void* outs[2] = {o, lse};
    const int64_t ob[2] = {rows_all * d * 4, rows_all * 4};
    if ((st = check_io(q, k, v, B, Sq, Sk, Hq, Hkv, d, outs, ob, 2))) return st;
  } else {
    const void* outs[2] = {o_accum, lse_accum};
    const int64_t ob[2] = {num_splits * rows_all * d * 4, num_splits * rows_all * 4};
    if ((st = check_io(q, k, v, B, Sq, Sk, Hq, Hkv, d, outs, ob, 2))) return st;
  }

  ff::SplitParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o_accum = o_accum;
  p.lse_accum = lse_accum;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.rows = Sq * p.G;
  p.num_mb = (int)cdiv(p.rows, kSplitRows);
  p.num_splits = num_splits;
  const int64_t nblocks = cdiv(Sk, FF_SPLIT_BLOCK_N);
  p.split_keys = (int)(cdiv(nblocks, num_splits) * FF_SPLIT_BLOCK_N);
  p.causal = (causal && Sq > 1) ? 1 : 0;
  p.scale_log2 = scale * ff::kLog2e;
  const int64_t total = (int64_t)B * Hkv * p.num_mb * num_splits;
  if (total >= kMaxElems) return FF_ERR_SHAPE;
  plan_log("attn_fwd_splitkv d=%d causal=%d: %lld workgroups = %d batches x %d kv heads x %d "
           "row blocks of %d folded rows x %d splits of %d keys", d, p.causal, (long long)total,
           B, Hkv, p.num_mb, kSplitRows, num_splits, p.split_keys);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)total), block(256);
  if (d == 128) hipLaunchKernelGGL((ff::attn_fwd_splitkv<128, false, 0>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((ff::attn_fwd_splitkv<64, false, 0>), grid, block, 0, s, p);
  return launch_status();
}

}  // extern "C"

namespace {

template <int D>
void launch_cache_var(int var, dim3 grid, dim3 block, hipStream_t s, const ff::SplitParams& p) {
  using namespace ff;
  switch (var) {
    case 0: hipLaunchKernelGGL((attn_fwd_splitkv<D, true, 0>), grid, block, 0, s, p); break;
    case kVarWindow:
      hipLaunchKernelGGL((attn_fwd_splitkv<D, true, kVarWindow>), grid, block, 0, s, p);
      break;
    case kVarWindow | kVarAlibi:
      hipLaunchKernelGGL((attn_fwd_splitkv<D, true, kVarWindow | kVarAlibi>), grid, block, 0, s,
                         p);
      break;
    case kVarWindow | kVarSoftcap:
      hipLaunchKernelGGL((attn_fwd_splitkv<D, true, kVarWindow | kVarSoftcap>), grid, block, 0,
                         s, p);
      break;
    default:
      hipLaunchKernelGGL((attn_fwd_splitkv<D, true, kVarWindow | kVarAlibi | kVarSoftcap>), grid,
                         block, 0, s, p);
      break;
  }
}

int fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                const int* cache_seqlens, const int* cache_leftpad, const int* block_table,
                float* o_accum, float* lse_accum, float* o, float* lse, int B, int Sq, int Hq,
                int Hkv, int d, int num_blocks, int page_size, int max_blocks_per_seq,
                int new_keys, int causal, float scale, int num_splits, const Variant& var,
                void* stream) {
  if (!q || !k_cache || !v_cache || !cache_seqlens) return FF_ERR_NULL;
  if (num_splits < 1 || num_splits > FF_MAX_SPLITS) return FF_ERR_SPLITS;
  if (num_splits == 1 && (!o || !lse)) return FF_ERR_NULL;
  if (num_splits > 1 && (!o_accum || !lse_accum)) return FF_ERR_NULL;
  int64_t blocks = 0, cap = 0;
  int st = check_cache(B, Hkv, block_table, num_blocks, page_size, max_blocks_per_seq, new_keys,
                       &blocks, &cap);
  if (st) return st;
  if (Sq < 1 || Hq < 1) return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  if (Hq % Hkv != 0) return FF_ERR_GQA;
  const int64_t rows_all = (int64_t)B * Hq * Sq;
  if (rows_all * d >= kMaxElems || (int64_t)num_splits * rows_all * d >= kMaxElems)
    return FF_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(cache_seqlens) ||
      !aligned4(cache_leftpad) || !aligned4(block_table))
    return FF_ERR_ALIGN;
  if (num_splits == 1 && (!aligned16(o) || !aligned16(lse))) return FF_ERR_ALIGN;
  if (num_splits > 1 && (!aligned16(o_accum) || !aligned16(lse_accum))) return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const int64_t cache_b = blocks * page_size * Hkv * d * 2;
  const void* ins[6] = {q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table};
  const int64_t in_b[6] = {rows_all * d * 2, cache_b, cache_b, (int64_t)B * 4, (int64_t)B * 4,
                           (int64_t)B * max_blocks_per_seq * 4};
  const void* outs[2];
  int64_t ob[2];
  if (num_splits == 1) {
    outs[0] = o, outs[1] = lse, ob[0] = rows_all * d * 4, ob[1] = rows_all * 4;
  } else {
    outs[0] = o_accum, outs[1] = lse_accum;
    ob[0] = num_splits * rows_all * d * 4, ob[1] = num_splits * rows_all * 4;
  }
  if (overlaps(outs[0], ob[0], outs[1], ob[1])) return FF_ERR_ALIAS;
  for (int i = 0; i < 2; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], ob[i], ins[j], in_b[j])) return FF_ERR_ALIAS;
    if (overlaps(outs[i], ob[i], var.alibi, alibi_bytes(var, B, Hq))) return FF_ERR_ALIAS;
  }

  ff::SplitParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k_cache;
  p.v = (const uint16_t*)v_cache;
  p.o_accum = o_accum;
  p.lse_accum = lse_accum;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = Sq;
  p.Sk = 0;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.rows = Sq * p.G;
  p.num_mb = (int)cdiv(p.rows, kSplitRows);
  p.num_splits = num_splits;
  p.split_keys = 0;
  p.causal = (causal && Sq > 1) ? 1 : 0;
  p.scale_log2 = scale * ff::kLog2e;
  p.kv_seqlens = cache_seqlens;
  p.leftpad = cache_leftpad;
  p.block_table = block_table;
  p.num_blocks = (int)blocks;
  p.page = page_size;
  p.max_blocks = block_table ? max_blocks_per_seq : 1;
  p.new_keys = new_keys;
  set_variant(p, var, scale);
  const int64_t total = (int64_t)B * Hkv * p.num_mb * num_splits;
  if (total >= kMaxElems) return FF_ERR_SHAPE;
  plan_log("attn_fwd_splitkv (key/value cache%s) d=%d causal=%d var=%d: %lld workgroups = %d "
           "batches x %d kv heads x %d row blocks of %d folded rows x %d splits",
           block_table ? ", paged" : "", d, p.causal, var.var, (long long)total, B, Hkv,
           p.num_mb, kSplitRows, num_splits);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)total), block(256);
  if (d == 128) launch_cache_var<128>(var.var, grid, block, s, p);
  else launch_cache_var<64>(var.var, grid, block, s, p);
  return launch_status();
}

}  // namespace

extern "C" {

int attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                     const int* cache_seqlens, const int* cache_leftpad, const int* block_table,
                     float* o_accum, float* lse_accum, float* o, float* lse, int B, int Sq,
                     int Hq, int Hkv, int d, int num_blocks, int page_size,
                     int max_blocks_per_seq, int new_keys, int causal, float scale,
                     int num_splits, void* stream) {
  return fwd_kvcache(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table, o_accum,
                     lse_accum, o, lse, B, Sq, Hq, Hkv, d, num_blocks, page_size,
                     max_blocks_per_seq, new_keys, causal, scale, num_splits, Variant{}, stream);
}

int attn_fwd_kvcache_ex(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_seqlens, const int* cache_leftpad,
                        const int* block_table, float* o_accum, float* lse_accum, float* o,
                        float* lse, int B, int Sq, int Hq, int Hkv, int d, int num_blocks,
                        int page_size, int max_blocks_per_seq, int new_keys, int causal,
                        int window_left, int window_right, const float* alibi_slopes,
                        int alibi_batch_stride, float softcap, float scale, int num_splits,
                        void* stream) {
  Variant var;
  int st = check_variant(window_left, window_right, alibi_slopes, alibi_batch_stride, softcap,
                         Hq, &var);
  if (st) return st;
  return fwd_kvcache(q, k_cache, v_cache, cache_seqlens, cache_leftpad, block_table, o_accum,
                     lse_accum, o, lse, B, Sq, Hq, Hkv, d, num_blocks, page_size,
                     max_blocks_per_seq, new_keys, causal, scale, num_splits, var, stream);
}

int attn_kvcache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int* cache_seqlens, const int* block_table, int B, int S_new,
                        int Hkv, int d, int num_blocks, int page_size, int max_blocks_per_seq,
                        void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !cache_seqlens) return FF_ERR_NULL;
  int64_t blocks = 0, cap = 0;
  int st = check_cache(B, Hkv, block_table, num_blocks, page_size, max_blocks_per_seq, S_new,
                       &blocks, &cap);
  if (st) return st;
  if (S_new < 1) return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  const int64_t new_elems = (int64_t)B * S_new * Hkv * d;
  if (new_elems >= kMaxElems) return FF_ERR_SHAPE;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned4(cache_seqlens) || !aligned4(block_table))
    return FF_ERR_ALIGN;
  const int64_t cache_b = blocks * page_size * Hkv * d * 2;
  const void* ins[4] = {k_new, v_new, cache_seqlens, block_table};
  const int64_t in_b[4] = {new_elems * 2, new_elems * 2, (int64_t)B * 4,
                           (int64_t)B * max_blocks_per_seq * 4};
  if (overlaps(k_cache, cache_b, v_cache, cache_b)) return FF_ERR_ALIAS;
  for (int j = 0; j < 4; ++j)
    if (overlaps(k_cache, cache_b, ins[j], in_b[j]) || overlaps(v_cache, cache_b, ins[j], in_b[j]))
      return FF_ERR_ALIAS;

  ff::AppendParams p;
  p.k_new = (const uint16_t*)k_new;
  p.v_new = (const uint16_t*)v_new;
  p.k_cache = (uint16_t*)k_cache;
  p.v_cache = (uint16_t*)v_cache;
  p.seqlens = cache_seqlens;
  p.block_table = block_table;
  p.B = B;
  p.S_new = S_new;
  p.Hkv = Hkv;
  p.num_blocks = (int)blocks;
  p.page = page_size;
  p.max_blocks = block_table ? max_blocks_per_seq : 1;
  p.chunks = new_elems / 8;
  plan_log("attn_kvcache_append d=%d: %lld 16-byte chunks, %lld workgroups", d,
           (long long)p.chunks, (long long)cdiv(p.chunks, 256));
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)cdiv(p.chunks, 256)), block(256);
  if (d == 128) hipLaunchKernelGGL(ff::attn_kvcache_append<128>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(ff::attn_kvcache_append<64>, grid, block, 0, s, p);
  return launch_status();
}

int attn_splitkv_combine(const float* o_accum, const float* lse_accum, float* o, float* lse,
                         int B, int Sq, int Hq, int d, int num_splits, void* stream) {
  if (!o_accum || !lse_accum || !o || !lse) return FF_ERR_NULL;
  if (B < 1 || Sq < 1 || Hq < 1) return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  if (num_splits < 1 || num_splits > FF_MAX_SPLITS) return FF_ERR_SPLITS;
  if (!aligned16(o_accum) || !aligned16(lse_accum) || !aligned16(o) || !aligned16(lse))
    return FF_ERR_ALIGN;
  const int64_t rows = (int64_t)B * Hq * Sq;
  if ((int64_t)num_splits * rows * d >= kMaxElems) return FF_ERR_SHAPE;
  const int64_t ab = num_splits * rows * d * 4, lb = num_splits * rows * 4;
  if (overlaps(o, rows * d * 4, o_accum, ab) || overlaps(o, rows * d * 4, lse_accum, lb) ||
      overlaps(lse, rows * 4, o_accum, ab) || overlaps(lse, rows * 4, lse_accum, lb) ||
      overlaps(o, rows * d * 4, lse, rows * 4))
    return FF_ERR_ALIAS;
  ff::CombineParams p;
  p.o_accum = o_accum;
  p.lse_accum = lse_accum;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = Sq;
  p.Hq = Hq;
  p.num_splits = num_splits;
  p.rows = (int)rows;
  plan_log("attn_splitkv_combine d=%d: %lld rows x %d splits, %lld workgroups", d,
           (long long)rows, num_splits, (long long)cdiv(rows, 4));
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)cdiv(rows, 4)), block(256);
  if (d == 128) hipLaunchKernelGGL(ff::attn_splitkv_combine<128>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(ff::attn_splitkv_combine<64>, grid, block, 0, s, p);
  return launch_status();
}

}  // extern "C"

namespace {

// The split partials of attn_fwd_splitkv_noalloc.  Each GPU the library runs on holds its
// own copy until the process ends.  On the host, `scratch` only names the array: its
// device address (per GPU) comes from hipGetSymbolAddress and is kept in g_scratch.
static __device__ __align__(256) float scratch[FF_NOALLOC_SCRATCH_FLOATS];
std::atomic<float*> g_scratch[64];

// The current device's address of `scratch`, looked up on the first call on that device.
int scratch_address(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FF_ERR_HIP;
  float* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return FF_ERR_HIP;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return FF_OK;
}

}  // namespace

extern "C" {

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                             int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                             float scale, int num_splits, void* stream) {
  if (!q || !k || !v || !o || !lse) return FF_ERR_NULL;
  if (num_splits < 1 || num_splits > FF_MAX_SPLITS) return FF_ERR_SPLITS;
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const int64_t rows = (int64_t)B * Hq * Sq;
  const void* outs[2] = {o, lse};
  const int64_t ob[2] = {rows * d * 4, rows * 4};
  if ((st = check_io(q, k, v, B, Sq, Sk, Hq, Hkv, d, outs, ob, 2))) return st;
  if (num_splits == 1)
    return attn_fwd_splitkv(q, k, v, nullptr, nullptr, o, lse, B, Sq, Sk, Hq, Hkv, d, causal,
                            scale, 1, stream);
  if ((int64_t)num_splits * rows * (d + 1) > FF_NOALLOC_SCRATCH_FLOATS) return FF_ERR_SCRATCH;
  float* base = nullptr;
  if ((st = scratch_address(&base))) return st;
  // partial O first, then the partial LSEs (16-byte aligned: d is a multiple of 4)
  float* o_accum = base;
  float* lse_accum = base + (int64_t)num_splits * rows * d;
  if ((st = attn_fwd_splitkv(q, k, v, o_accum, lse_accum, nullptr, nullptr, B, Sq, Sk, Hq, Hkv,
                             d, causal, scale, num_splits, stream)))
    return st;
  return attn_splitkv_combine(o_accum, lse_accum, o, lse, B, Sq, Hq, d, num_splits, stream);
}

}  // extern "C"

extern "C" {

int attn_quantize_fp8(const void* x, void* x_fp8, float* scales, int B, int S, int H, int d,
                      int rotate, void* stream) {
  if (!x || !x_fp8 || !scales) return FF_ERR_NULL;
  if (B < 1 || S < 1 || H < 1) return FF_ERR_SHAPE;
  if (d != 64 && d != 128) return FF_ERR_HEADDIM;
  const int64_t elems = (int64_t)B * S * H * d;
  if (elems >= kMaxElems) return FF_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(x_fp8) || !aligned16(scales)) return FF_ERR_ALIGN;
  const int nblk = (int)cdiv(S, 128);
  const int64_t sb = (int64_t)B * H * nblk * 4;
  if (overlaps(x_fp8, elems, x, elems * 2) || overlaps(scales, sb, x, elems * 2) ||
      overlaps(scales, sb, x_fp8, elems))
    return FF_ERR_ALIAS;
  ff::QuantParams p;
  p.x = (const uint16_t*)x;
  p.codes = (uint8_t*)x_fp8;
  p.scales = scales;
  p.B = B;
  p.S = S;
  p.H = H;
  p.nblk = nblk;
  p.rotate = rotate ? 1 : 0;
  plan_log("attn_quantize_fp8 d=%d: %lld workgroups = %d batches x %d heads x %d blocks of "
           "positions", d, (long long)B * H * nblk, B, H, nblk);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)((int64_t)B * H * nblk)), block(256);
  if (d == 128) hipLaunchKernelGGL(ff::attn_quantize_fp8<128>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(ff::attn_quantize_fp8<64>, grid, block, 0, s, p);
  return launch_status();
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                 const float* k_scale, const float* v_scale, float* o, float* lse, int B,
                 int Sq, int Sk, int Hq, int Hkv, int d, int causal, float scale, void* stream) {
  if (!q || !k || !v || !q_scale || !k_scale || !v_scale || !o || !lse) return FF_ERR_NULL;
  int st = check_dims(B, Sq, Sk, Hq, Hkv, d);
  if (st) return st;
  const void* ptrs[8] = {q, k, v, q_scale, k_scale, v_scale, o, lse};
  for (const void* x : ptrs)
    if (!aligned16(x)) return FF_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  const int nqb = (int)cdiv(Sq, 128), nkb = (int)cdiv(Sk, 128);
  const int64_t qb = (int64_t)B * Sq * Hq * d, kvb = (int64_t)B * Sk * Hkv * d;
  const void* ins[6] = {q, k, v, q_scale, k_scale, v_scale};
  const int64_t in_b[6] = {qb, kvb, kvb, (int64_t)B * Hq * nqb * 4, (int64_t)B * Hkv * nkb * 4,
                           (int64_t)B * Hkv * nkb * 4};
  const void* outs[2] = {o, lse};
  const int64_t ob[2] = {qb * 4, (int64_t)B * Hq * Sq * 4};
  if (overlaps(o, ob[0], lse, ob[1])) return FF_ERR_ALIAS;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], ob[i], ins[j], in_b[j])) return FF_ERR_ALIAS;

  ff::Fp8Params p;
  p.q = (const uint8_t*)q;
  p.k = (const uint8_t*)k;
  p.v = (const uint8_t*)v;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.num_m = (int)cdiv(Sq, ff::Fp8Traits<128>::BM);
  p.u_per = (int)cdiv((int64_t)B * Hkv, 8);
  const int64_t total = 8 * (int64_t)p.u_per * p.G * p.num_m;
  if (total >= kMaxElems) return FF_ERR_SHAPE;
  p.total = (int)total;
  p.nqb = nqb;
  p.nkb = nkb;
  p.scale_log2 = scale * ff::kLog2e;
  plan_log("attn_fwd_fp8 d=%d causal=%d: %lld workgroups of 256 threads, %d query tiles x %d "
           "unit slots per XCD x %d query heads per kv head", d, causal, (long long)total,
           p.num_m, p.u_per, p.G);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)total), block(256);
  if (d == 128) {
    if (causal) hipLaunchKernelGGL((ff::attn_fwd_fp8<128, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((ff::attn_fwd_fp8<128, false>), grid, block, 0, s, p);
  } else {
    if (causal) hipLaunchKernelGGL((ff::attn_fwd_fp8<64, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((ff::attn_fwd_fp8<64, false>), grid, block, 0, s, p);
  }
  return launch_status();
}

}  // extern "C"
