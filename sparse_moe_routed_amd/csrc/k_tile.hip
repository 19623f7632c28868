// One-time conversion of row-major expert weights into the tiled layout read
// by the tiled grouped-FFN kernels (layout defined in include/moe.h): every
// 16-row x 32-k MFMA operand fragment becomes contiguous, so a wave's load
// instruction reads one contiguous block.  Pure byte permutations.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// bf16 matrix stack [NR][K] (NR = E * N rows): one thread per 16-byte chunk.
__global__ __launch_bounds__(256) void k_tile_bf16(const uint16_t* __restrict__ src,
                                                   uint16_t* __restrict__ dst, size_t n_chunks,
                                                   int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_chunks) return;
  const int l = static_cast<int>(idx & 63);
  const size_t rest = idx >> 6;
  const size_t ks = rest % static_cast<size_t>(K / 32), nb = rest / static_cast<size_t>(K / 32);
  const int r = l & 15, q = l >> 4;
  const size_t s = (nb * 16 + r) * static_cast<size_t>(K) + ks * 32 + q * 8;
  *reinterpret_cast<u32x4_t*>(dst + idx * 8) = ld16(src + s);
}

// int4 / int2 codes [NR][K * bits / 8]: one thread per (row block, k unit,
// lane) output unit of 4 pieces of `bits` bytes (8 codes each).
template <int BITS>
__global__ __launch_bounds__(256) void k_tile_codes(const uint8_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, size_t n_units,
                                                    int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_units) return;
  const int l = static_cast<int>(idx & 63);
  const size_t rest = idx >> 6;
  const size_t kb = rest % static_cast<size_t>(K / 128), nb = rest / static_cast<size_t>(K / 128);
  const int r = l & 15, q = l >> 4;
  const size_t row = (nb * 16 + r) * (static_cast<size_t>(K) * BITS / 8);
  uint8_t* o = dst + idx * (4 * BITS);
  uint32_t piece[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const size_t b = row + (kb * 128 + s * 32 + q * 8) * BITS / 8;
    piece[s] = BITS == 4 ? *reinterpret_cast<const uint32_t*>(src + b)
                         : *reinterpret_cast<const uint16_t*>(src + b);
  }
  if constexpr (BITS == 4) {
    // natural nibble order c0..c7 -> stored c_2m at nibble m, c_2m+1 at
    // nibble m+4; two's complement -> offset binary (xor 8)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t t = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        t |= ((piece[s] >> (8 * m)) & 0xFu) << (4 * m);
        t |= ((piece[s] >> (8 * m + 4)) & 0xFu) << (4 * (m + 4));
      }
      *reinterpret_cast<uint32_t*>(o + s * 4) = t ^ 0x88888888u;
    }
  } else {
    // chunks 2w and 2w+1 share word w: chunk sub's c_2m at bits 8 sub + 2m,
    // c_2m+1 at bits 16 + 8 sub + 2m; two's complement -> offset binary (xor 2)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t t = 0;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const uint32_t v = piece[2 * w + sub];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          t |= ((v >> (4 * m)) & 3u) << (8 * sub + 2 * m);
          t |= ((v >> (4 * m + 2)) & 3u) << (16 + 8 * sub + 2 * m);
        }
      }
      *reinterpret_cast<uint32_t*>(o + w * 4) = t ^ 0xAAAAAAAAu;
    }
  }
}

// fp16 scales [NR][K/32] -> [NR/16][K/128][16][4]: one thread per
// (row block, k unit, row).
__global__ __launch_bounds__(256) void k_tile_scales(const uint16_t* __restrict__ src,
                                                     uint16_t* __restrict__ dst, size_t n_rows4,
                                                     int K) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n_rows4) return;
  const int r = static_cast<int>(idx & 15);
  const size_t rest = idx >> 4;
  const size_t kb = rest % static_cast<size_t>(K / 128), nb = rest / static_cast<size_t>(K / 128);
  const uint16_t* s = src + (nb * 16 + r) * static_cast<size_t>(K / 32) + kb * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) dst[idx * 4 + j] = s[j];
}

static void tile_matrix(const moe_shape& s, const void* src, void* dst, const uint16_t* ssrc,
                        uint16_t* sdst, size_t rows, int K, hipStream_t st) {
  const unsigned blk = 256;
  if (s.wfmt == MOE_WF_DENSE) {
    const size_t n = rows * (K / 8);
    hipLaunchKernelGGL(k_tile_bf16, dim3(static_cast<unsigned>((n + blk - 1) / blk)), dim3(blk), 0,
                       st, static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), n, K);
    return;
  }
  const size_t nu = (rows / 16) * (K / 128) * 64;
  if (s.wfmt == MOE_WF_INT4_G32)
    hipLaunchKernelGGL(k_tile_codes<4>, dim3(static_cast<unsigned>((nu + blk - 1) / blk)), dim3(blk),
                       0, st, static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), nu, K);
  else
    hipLaunchKernelGGL(k_tile_codes<2>, dim3(static_cast<unsigned>((nu + blk - 1) / blk)), dim3(blk),
                       0, st, static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), nu, K);
  const size_t ns = (rows / 16) * (K / 128) * 16;
  hipLaunchKernelGGL(k_tile_scales, dim3(static_cast<unsigned>((ns + blk - 1) / blk)), dim3(blk), 0,
                     st, ssrc, sdst, ns, K);
}

hipError_t launch_tile_experts(const moe_shape& s, const moe_experts& src, const moe_experts& dst,
                               hipStream_t st) {
  const size_t E = static_cast<size_t>(s.E);
  tile_matrix(s, src.gate, const_cast<void*>(dst.gate), src.gate_scale,
              const_cast<uint16_t*>(dst.gate_scale), E * s.I, s.H, st);
  tile_matrix(s, src.up, const_cast<void*>(dst.up), src.up_scale,
              const_cast<uint16_t*>(dst.up_scale), E * s.I, s.H, st);
  tile_matrix(s, src.down, const_cast<void*>(dst.down), src.down_scale,
              const_cast<uint16_t*>(dst.down_scale), E * s.H, s.I, st);
  return hipGetLastError();
}

}  // namespace moe
