// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4).
//
// Formats (reading of "DeepSeek-V4.1 模型结构（0）：一张图看懂 DeepSeek-V4.1-Flash", Q&A on
// the 890-byte count, and "DeepSeek V4.1 Flash 深度解析", part-4 entry on FP4 in the KV
// cache): FP4 E2M1 values, element 2i in the low nibble of byte i; main-KV scales are
// E4M3 bytes, one per 16 values; indexer scale is one fp32 per entry; the sliding
// window is raw E4M3.  Conversions use the gfx950 converters: v_cvt_scalef32_pk_f32_fp4
// (low nibble -> element 0) and v_cvt_pk_f32_fp8.  The fp4 converter's scale operand is
// applied as a power of two only, so it is always 1.0 here and real scales are
// multiplied separately.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kDIdx = 128;          // indexer key width
constexpr int kDKv = 512;           // main KV width
constexpr int kHeads = 16;          // query heads sharing every entry
constexpr int kSwa = 128;           // sliding-window rows
constexpr int kIdxCodeBytes = 64;   // 128 x 4 bit
constexpr int kKvCodeBytes = 256;   // 512 x 4 bit
constexpr int kKvScaleBytes = 32;   // one E4M3 per 16 values

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two E2M1 values held in byte SEL of w, unscaled (exact in f32).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2(uint32_t w) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  return v;
}

// Two E2M1 values in byte SEL of w as a packed bf16 pair (exact).
template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// Two E4M3 bytes of w (HI selects bytes 2,3) as f32.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2(uint32_t w) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
  return v;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(byte, false);
  return v.x;
}

// Order-preserving map f32 -> u32: a larger score gives a larger key; -0 maps like +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Agent-scope release / acquire around the row barriers of the fused scan + top-k.
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace csa2
