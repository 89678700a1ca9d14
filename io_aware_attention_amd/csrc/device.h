// Device building blocks for the gfx950 attention kernels: vector types, the two
// bf16 matrix-core instructions, 128-bit memory helpers, bf16 packing and
// cross-lane reductions.  Wavefronts are 64 lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace ff {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32).  Lane l supplies A[l%32][8*(l/32) .. +7] and
// B[8*(l/32) .. +7][l%32]; it receives D[8*j + 4*(l/32) + i][l%32] in element
// 4*j + i (j, i in 0..3).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; it receives D[4*(l/16) + i][l%16] in element i.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two floats to packed bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 pack8(float a0, float a1, float a2, float a3, float a4,
                                       float a5, float a6, float a7) {
  u32x4 r;
  r[0] = pack_bf16(a0, a1);
  r[1] = pack_bf16(a2, a3);
  r[2] = pack_bf16(a4, a5);
  r[3] = pack_bf16(a6, a7);
  return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ void st16f(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
// The same with the non-temporal hint, for outputs that are written once and not read
// back by the kernel: they stream through L2 without displacing the key/value tiles
// that other workgroups are about to read.  Only for whole 128-byte lines: scattered
// 16-byte pieces stored this way lose the write combining (an FP8 forward whose lanes
// each stored 16 bytes of a row took 237 instead of 179 us).
__device__ __forceinline__ void st16f_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float vmax(float a, float b) { return __builtin_fmaxf(a, b); }

// Low 16 bits of a and b packed (a in the low half); high halves likewise.
__device__ __forceinline__ uint32_t lo_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// max over lanes l and l^32 (v_permlane32_swap exchanges the two wave halves).
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// ds_read_b64_tr_b16 at LDS byte address a + OFF.  Within each group of 16 lanes,
// result lane i, element j is element (i & 3) of the 8 bytes that lane 4j + (i >> 2)
// addressed.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64(uint32_t a) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(uintptr_t)(a + OFF));
  return __builtin_bit_cast(u32x2, r);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of the buffer-load builtins: the non-temporal hint (the nt bit),
// for data read exactly once, such as the key/value stream of a decode step.
constexpr int kLoadStreaming = 2;

// Buffer descriptor (gfx9 layout: base, stride 0, num_records bytes, raw dword3).
// Reads at byte offsets >= num_records return zero.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t num_records) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)num_records,
               0x00020000};
}

// 16 bytes per lane from buffer `desc` at byte offset voff straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds; lds_base is wave-uniform).
// Written as inline assembly: the compiler then neither tracks nor orders other LDS
// reads behind these loads, so the caller must wait (vmcnt) and synchronise before
// reading what they wrote.  The LDS address travels in M0, which the "{m0}" operand has
// the compiler load itself (so no live value of its own sits in M0 across the
// statement).  On this GPU generation an LDS DMA that reads M0 needs one wait state
// after the scalar write of M0, and the compiler does not know what the statement
// holds: the s_nop provides it.
__device__ __forceinline__ void buffer_load_lds16(i32x4 desc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(desc), "{m0}"(lds_base)
               : "memory");
}

// All of this wave's vector-memory loads (including loads into LDS) have completed.  The
// inline wait covers the loads the compiler cannot see (the buffer loads into LDS); the
// builtin one after it tells the compiler's own wait tracking that its loads are done too.
// Without that, a compiler load still pending in its model (a scale, say) gets a vmcnt(n)
// at its first use, and by then the counter also holds the next tile's loads into LDS:
// the wait would stall on the prefetch.
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unconstrained
}

__device__ __forceinline__ float sum_xor32(float x) { return x + __shfl_xor(x, 32); }

// Wavefront-local LDS handoff: the lanes of one wavefront exchange data through
// LDS; the fences order the accesses and the wave barrier keeps the compiler
// from moving them across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, fully unrolled.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Mask and bias variants of the forward kernels (their VAR template argument), after the
// walk-through's Is_local, Has_alibi and Is_softcap flags: the sliding window (window
// limits of -1 mask nothing), the ALiBi bias and the soft cap.  VAR = 0 is the plain
// kernel; any variant kernel includes the window.
constexpr int kVarWindow = 1, kVarAlibi = 2, kVarSoftcap = 4;

// Soft-capped logit in base-2 units, c log2(e) tanh(y) with y = s scale / c, from
// tanh(y) = 1 - 2 / (e^(2y) + 1) and e^(2y) = 2^(s k), k = 2 scale log2(e) / c;
// cap2 = c log2(e).  The limits come out exact: e^(2y) = inf gives cap2, 0 gives -cap2.
__device__ __forceinline__ float softcap2(float s, float k, float cap2) {
  const float e = fast_exp2(s * k);
  return __builtin_fmaf(__builtin_amdgcn_rcpf(e + 1.f), -2.f * cap2, cap2);
}

}  // namespace ff
