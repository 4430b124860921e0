// Device-side building blocks for the gfx950 attention kernels: MFMA operand types, the
// 32x32 MFMA wrappers, 16-bit conversions and lane exchanges.
//
// MFMA layout used throughout (v_mfma_f32_32x32x16_{bf16,f16}, wave64): lane l = 32*g + r
// (g = l / 32, r = l % 32).
//   A operand (32 x 16): lane l supplies row r, 8 values along the contraction (group g).
//   B operand (16 x 32): lane l supplies column r, the same 8 contraction positions (group g).
//   C (32 x 32, fp32): lane l holds column r, rows 8*(i/4) + 4*g + (i%4) for i = 0..15.
// Only the pairing of A and B contraction slots matters for the result, so any fixed map of
// contraction index -> (g, slot) that both operands share is valid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 8 16-bit values (16 bytes) as raw bits.
struct alignas(16) Frag16 {
  u32x4 w;
};

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(const Frag16& a, const Frag16& b, f32x16 c) {
  if constexpr (IS_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                   __builtin_bit_cast(bf16x8, b.w), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.w),
                                                  __builtin_bit_cast(f16x8, b.w), c, 0, 0, 0);
  }
}

// Round-to-nearest-even float -> 16-bit storage, two at a time (low half = a).
template <bool IS_BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (IS_BF16) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  } else {
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
  }
}

template <bool IS_BF16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (IS_BF16) {
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa
