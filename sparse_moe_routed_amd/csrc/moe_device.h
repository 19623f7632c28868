// Device-side helpers shared by the routed-MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// v_mfma_f32_16x16x32_bf16.  Operand lane layout (wave64):
//   A: lane l supplies row (l % 16), reduction slots 8*(l/16) .. +7
//   B: lane l supplies column (l % 16), reduction slots 8*(l/16) .. +7
//   D: lane l holds rows 4*(l/16) + j (j = 0..3) of column (l % 16).
// Any assignment of real k to reduction slots works as long as A and B
// agree; the kernels feed 8 consecutive k per lane.
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float fp16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float silu(float g) {
  return g / (1.0f + __expf(-g));
}

// Two floats holding small integers (exact in bf16) -> packed bf16 pair
// (lo = a, hi = b): the bf16 pattern of such a float is its top 16 bits.
__device__ __forceinline__ uint32_t pack_bf16_exact(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// Signed bit-field extract (v_bfe_i32); the builtin's result type is unsigned,
// so the sign must be restored by the cast before any conversion to float.
__device__ __forceinline__ int sbfe(uint32_t w, int off, int width) {
  return static_cast<int>(__builtin_amdgcn_sbfe(static_cast<int>(w), off, width));
}

// 8 signed 4-bit codes (little-endian nibbles of w) -> 4 packed bf16 pairs.
__device__ __forceinline__ u32x4_t dequant_int4x8(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = static_cast<float>(sbfe(w, 8 * i, 4));
    const float b = static_cast<float>(sbfe(w, 8 * i + 4, 4));
    r[i] = pack_bf16_exact(a, b);
  }
  return r;
}

// 8 signed 2-bit codes (little-endian pairs of bits of w16) -> 4 bf16 pairs.
__device__ __forceinline__ u32x4_t dequant_int2x8(uint32_t w16) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = static_cast<float>(sbfe(w16, 4 * i, 2));
    const float b = static_cast<float>(sbfe(w16, 4 * i + 2, 2));
    r[i] = pack_bf16_exact(a, b);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace moe
