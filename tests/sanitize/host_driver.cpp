// Calls every entry point of libflashfwd with arguments that its host-side checks must
// reject before any HIP call, and the pure host routines (the split rule, the workspace
// size, the status strings), so that a build with AddressSanitizer and
// UndefinedBehaviorSanitizer covers the validation code.  Fake pointers are never
// dereferenced: every call here fails validation first.  Exits non-zero on a wrong code.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "flashfwd.h"

static int failures = 0;
static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAILED: %s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  char* const Q = (char*)(uintptr_t)(1ull << 20);
  char* const K = (char*)(uintptr_t)(2ull << 30);
  char* const V = (char*)(uintptr_t)(3ull << 30);
  float* const O = (float*)(uintptr_t)(4ull << 32);
  float* const L = (float*)(uintptr_t)(5ull << 32);
  float* const A = (float*)(uintptr_t)(6ull << 32);
  float* const W = (float*)(uintptr_t)(7ull << 32);
  int* const C = (int*)(uintptr_t)(8ull << 32);
  int* const T = (int*)(uintptr_t)(9ull << 32);
  const float nan = NAN, inf = INFINITY;

  expect(attn_fwd(nullptr, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, 0.125f, nullptr), FF_ERR_NULL, "fwd null");
  expect(attn_fwd(Q, K, V, O, L, 0, 8, 8, 2, 1, 64, 0, 0.125f, nullptr), FF_ERR_SHAPE, "fwd B");
  expect(attn_fwd(Q, K, V, O, L, 1, 8, 8, 2, 1, 96, 0, 0.125f, nullptr), FF_ERR_HEADDIM, "fwd d");
  expect(attn_fwd(Q, K, V, O, L, 1, 8, 8, 3, 2, 64, 0, 0.125f, nullptr), FF_ERR_GQA, "fwd gqa");
  expect(attn_fwd(Q + 8, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, 0.125f, nullptr), FF_ERR_ALIGN, "fwd align");
  expect(attn_fwd(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, nan, nullptr), FF_ERR_SCALE, "fwd nan");
  expect(attn_fwd(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, inf, nullptr), FF_ERR_SCALE, "fwd inf");
  expect(attn_fwd(Q, K, V, (float*)Q, L, 1, 8, 8, 2, 1, 64, 0, 0.125f, nullptr), FF_ERR_ALIAS, "fwd alias");
  expect(attn_fwd(Q, K, V, O, L, 1 << 12, 1 << 12, 8, 1 << 4, 1, 128, 0, 0.125f, nullptr), FF_ERR_SHAPE, "fwd size");
  expect(attn_fwd_ex(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, -2, -1, nullptr, 0, 0.f, 0.125f, nullptr), FF_ERR_OPTION, "ex window");
  expect(attn_fwd_ex(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, -1, -1, nullptr, 0, -1.f, 0.125f, nullptr), FF_ERR_OPTION, "ex cap");
  expect(attn_fwd_ex(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, -1, -1, A, 3, 0.f, 0.125f, nullptr), FF_ERR_OPTION, "ex stride");
  expect(attn_fwd_ex(Q, K, V, O, L, 1, 8, 8, 2, 1, 64, 0, -1, -1, (float*)((char*)A + 2), 0, 0.f, 0.125f, nullptr), FF_ERR_ALIGN, "ex slopes align");
  expect(attn_fwd_varlen(Q, K, V, O, L, nullptr, C, 2, 8, 16, 16, 2, 1, 64, 1, 0.125f, nullptr), FF_ERR_NULL, "varlen null");
  expect(attn_fwd_varlen(Q, K, V, O, L, C, C, 2, 17, 16, 16, 2, 1, 64, 1, 0.125f, nullptr), FF_ERR_SHAPE, "varlen max");
  expect(attn_fwd_varlen(Q, K, V, O, L, C, (int*)((char*)C + 2), 2, 8, 16, 16, 2, 1, 64, 1, 0.125f, nullptr), FF_ERR_ALIGN, "varlen align");
  expect(attn_splitkv_num_splits(6, 1, 8192, 8, 8, 128, 108), 2, "num_splits");
  expect(attn_splitkv_num_splits(0, 1, 8192, 8, 8, 128, 108), -FF_ERR_SHAPE, "num_splits shape");
  expect(attn_splits_efficiency_rule(48, 108, 128), 2, "rule 48 on 108");
  expect(attn_splits_efficiency_rule(0, 108, 8), -FF_ERR_SHAPE, "rule shape");
  expect(attn_fwd_splitkv(Q, K, V, W, A, O, L, 1, 1, 64, 8, 2, 128, 0, 0.1f, 0, nullptr), FF_ERR_SPLITS, "split 0");
  expect(attn_fwd_splitkv(Q, K, V, W, A, O, L, 1, 1, 64, 8, 2, 128, 0, 0.1f, 129, nullptr), FF_ERR_SPLITS, "split 129");
  expect(attn_fwd_splitkv(Q, K, V, nullptr, A, O, L, 1, 1, 64, 8, 2, 128, 0, 0.1f, 4, nullptr), FF_ERR_NULL, "split accum");
  expect(attn_splitkv_combine(W, A, O, L, 1, 1, 8, 128, 0, nullptr), FF_ERR_SPLITS, "combine splits");
  expect(attn_splitkv_combine(nullptr, A, O, L, 1, 1, 8, 128, 2, nullptr), FF_ERR_NULL, "combine null");
  expect(attn_fwd_kvcache(Q, K, V, C, nullptr, T, W, A, O, L, 2, 1, 8, 2, 128, 4, 48, 2, 0, 0, 0.1f, 1, nullptr), FF_ERR_SHAPE, "kvcache page");
  expect(attn_fwd_kvcache_ex(Q, K, V, C, nullptr, nullptr, W, A, O, L, 2, 1, 8, 2, 128, 0, 64, 0, 0, 0, -3, -1, nullptr, 0, 0.f, 0.1f, 1, nullptr), FF_ERR_OPTION, "kvcache_ex window");
  expect(attn_kvcache_append(Q, K, (void*)V, (void*)O, C, nullptr, 2, 1, 2, 100, 0, 64, 0, nullptr), FF_ERR_HEADDIM, "append d");
  expect(attn_quantize_fp8(Q, (void*)K, A, 1, 8, 2, 96, 0, nullptr), FF_ERR_HEADDIM, "quantize d");
  expect(attn_fwd_fp8(Q, K, V, nullptr, A, W, O, L, 1, 8, 8, 2, 2, 128, 0, 0.1f, nullptr), FF_ERR_NULL, "fp8 scales");
  expect((int)attn_bwd_workspace_floats(2, 65, 3), 2 * 2 * 3 * 128, "workspace");
  expect((int)attn_bwd_workspace_floats(0, 65, 3), -FF_ERR_SHAPE, "workspace shape");
  expect(attn_bwd(Q, K, V, O, L, Q, W, A, A, A, 1, 8, 8, 2, 1, 64, 0, 0.125f, nullptr), FF_ERR_ALIAS, "bwd alias");
  expect(attn_bwd_ex(Q, K, V, O, L, Q, W, A, O, L, 1, 8, 8, 2, 1, 64, 0, -1, -1, nullptr, 0, 2.f, 0.125f, nullptr), FF_ERR_OPTION, "bwd softcap");
  expect(attn_fwd_splitkv_noalloc(Q, K, V, O, L, 8, 16, 64, 32, 8, 128, 0, 0.1f, 128, nullptr), FF_ERR_SCRATCH, "noalloc size");
  expect(attn_fwd_splitkv_noalloc(Q, K, V, O, L, 1, 1, 64, 8, 2, 128, 0, 0.1f, 0, nullptr), FF_ERR_SPLITS, "noalloc splits");
  expect(attn_fwd_splitkv_noalloc(Q, K, V, (float*)K, L, 1, 1, 64, 8, 2, 128, 0, 0.1f, 4, nullptr), FF_ERR_ALIAS, "noalloc alias");
  for (int s = 0; s <= 12; ++s)
    if (!attn_status_string(s)[0]) expect(0, 1, "status string");
  if (failures) return 1;
  printf("host driver: all checks passed\n");
  return 0;
}
