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

// 16-byte load of data read once (weights): non-temporal (`nt`)
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
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

// Offset ("magic") dequantization for the tiled low-bit layouts.  A code q is
// turned into the exact bf16 integer 128 + (q + bias) by OR-ing its offset
// binary value into the mantissa of 128.0 (bf16 0x4300): bias 8 for int4
// (values 136 + q) and 2 for int2 (130 + q); the constant part is removed by
// an MFMA against a fragment of -136 / -130 (kNegOffset*), which is exact in
// bf16.  One AND-OR per pair of codes.
constexpr uint32_t kNegOffset4 = 0xC308C308u;   // bf16 pair (-136, -136)
constexpr uint32_t kNegOffset2 = 0xC302C302u;   // bf16 pair (-130, -130)

// Tiled low-bit codes are stored offset-binary (code + 8 for int4, code + 2
// for int2), so one AND with a field mask and one OR with 0x4300 per bf16
// half give the exact bf16 value 128 + stored code.  The mask and the magic
// word arrive in registers: gfx9 VOP3 instructions take no literal operand,
// so with constants the AND-OR would split into two instructions.
struct Dq {
  uint32_t mask, magic;
};

// Moves a constant into a VGPR the compiler cannot fold back into literals.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// int4: one 32-bit word per k chunk, stored code 2m at nibble m and code
// 2m+1 at nibble m+4 -> 4 bf16 pairs (136 + q_2m, 136 + q_2m+1).
__device__ __forceinline__ u32x4_t dequant_int4_tiled(uint32_t w, Dq d) {
  u32x4_t r;
  r[0] = (w & d.mask) | d.magic;
  r[1] = ((w >> 4) & d.mask) | d.magic;
  r[2] = ((w >> 8) & d.mask) | d.magic;
  r[3] = ((w >> 12) & d.mask) | d.magic;
  return r;
}

// int2: one 32-bit word per pair of k chunks; chunk `sub` (0, 1) has stored
// code 2m at bits 8 sub + 2m and code 2m+1 at bits 16 + 8 sub + 2m ->
// 4 bf16 pairs (130 + q_2m, 130 + q_2m+1).
template <int SUB>
__device__ __forceinline__ u32x4_t dequant_int2_tiled(uint32_t w, Dq d) {
  u32x4_t r;
  r[0] = ((w >> (8 * SUB)) & d.mask) | d.magic;
  r[1] = ((w >> (8 * SUB + 2)) & d.mask) | d.magic;
  r[2] = ((w >> (8 * SUB + 4)) & d.mask) | d.magic;
  r[3] = ((w >> (8 * SUB + 6)) & d.mask) | d.magic;
  return r;
}

// Staging of activation rows through LDS (256-thread workgroups, 16-row
// blocks, 128-wide k units of bf16).
// Per-thread share of one unit: NB 16-byte chunks.  Chunk i of thread
// (wave w, lane l) is row 16 i + 4 w + l / 16, k chunk l % 16 of the unit.
// LDS layout: fragment f = st * NB + b holds 64 16-byte slots; the chunk of
// MFMA lane r + 16 q sits in slot 16 q + (r ^ (4 st + q)).  The XOR keeps the
// 16 lanes that store one row segment, and the 16 lanes that read one
// fragment quarter, on 16 distinct bank groups.
template <int NB>
struct XUnit {
  const uint16_t* src[NB];   // row base + chunk offset (elements)
  int dst[NB];               // byte offset in one LDS buffer
  u32x4_t v[NB];

  // `row_of(R)` gives the element offset of tile row R (clamped by caller)
  template <typename RowOf>
  __device__ __forceinline__ void init(const uint16_t* base, RowOf row_of) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int c = l & 15, r = 4 * w + (l >> 4);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      src[i] = base + row_of(16 * i + r) + c * 8;
      dst[i] = (((c >> 2) * NB + i) * 64 + 16 * (c & 3) + (r ^ c)) * 16;
    }
  }
  __device__ __forceinline__ void load(int u) {
#pragma unroll
    for (int i = 0; i < NB; ++i) v[i] = ld16(src[i] + 128 * u);
  }
  __device__ __forceinline__ void store(char* buf) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4_t*>(buf + dst[i]) = v[i];
  }
};

// The same staging with the rows read through a raw buffer (base and size
// in SGPRs, one 32-bit byte offset per row instead of a 64-bit pointer).
// The matrix must be under 4 GiB; loads past its size return 0.
template <int NB>
struct XUnitBuf {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t src[NB];   // byte offset of the row base + chunk
  int dst[NB];
  u32x4_t v[NB];

  template <typename RowOf>
  __device__ __forceinline__ void init(const uint16_t* base, uint32_t bytes, RowOf row_of) {
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int c = l & 15, r = 4 * w + (l >> 4);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      src[i] = static_cast<uint32_t>((row_of(16 * i + r) + c * 8) * 2);
      dst[i] = (((c >> 2) * NB + i) * 64 + 16 * (c & 3) + (r ^ c)) * 16;
    }
  }
  __device__ __forceinline__ void load(int u) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(src[i]), 256 * u, 0);
  }
  __device__ __forceinline__ void store(char* buf) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) *reinterpret_cast<u32x4_t*>(buf + dst[i]) = v[i];
  }
};

// A fragment (k chunk st, row block b) of the staged unit in `buf`.
template <int NB>
__device__ __forceinline__ u32x4_t xfrag(const char* buf, int st, int b, int lane) {
  const int q = lane >> 4, r = lane & 15;
  return *reinterpret_cast<const u32x4_t*>(
      buf + ((st * NB + b) * 64 + 16 * q + (r ^ (4 * st + q))) * 16);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// DPP lane permutations within 16-lane rows (few-cycle latency, no LDS).
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each row

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Maximum of a float over the wave, returned to every lane (wave-uniform).
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Minimum of an unsigned value over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppHalfMirror>(v));
  v = min(v, dpp_u32<kDppMirror>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// Maximum of an unsigned value over the wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Inclusive prefix sum over the 64 lanes of a wave, in VALU: DPP row
// shifts by 1, 2, 4, 8 scan each row of 16 lanes, then lane 15 of rows 0
// and 2 is added to rows 1 and 3 and lane 31 to rows 2 and 3 (row
// broadcasts).  Lanes without a source in a step add nothing.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Sum of a float over the wave in a fixed association (wave-uniform result).
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v)));
  const float r0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 0));
  const float r1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 16));
  const float r2 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 32));
  const float r3 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace moe

namespace moe {

// Memory operations coherent across the whole device, for data that one
// workgroup hands to another inside a launch.  On gfx950 every XCD has its
// own L2, and a device-scope fence (__threadfence) writes back and
// invalidates that whole L2: thousands of workgroups doing it cost hundreds
// of microseconds (measured: the decode down kernel with a fence per
// workgroup took ~550 us longer).  Instead the handed-over data is stored
// and loaded as device-scope relaxed atomics (the sc1 cache policy), and the
// writer waits for its stores to complete before it signals with an
// atomic.

__device__ __forceinline__ void store_dev_i32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_dev_i32(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every memory operation this thread issued has completed (the compiler
// keeps memory operations on their side of the wait).
__device__ __forceinline__ void wait_memory_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace moe
