// Route-rank-order weighted combine (+ residual).
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Hypothesis H4: ExpertMajor
// should stream as a wavefront, not a barrier": experts write separate result
// slots and the final weighted sum follows a deterministic route-rank order.
//
// out[t][n] = residual[t][n] + sum_{j=0}^{k-1} w[t][j] * y[pair_row[t*k+j]][n]
// The sum runs in float32 with j ascending, then the residual is added and
// the result rounded once to the activation type.  One thread per 8 (bf16)
// or 4 (float32) consecutive features; loads are 16 bytes.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// KB route slots per batch: all index/weight loads of a batch, then all its
// row loads, then the float32 accumulation in ascending j; KB >= k makes the
// whole combine two dependent memory round trips.
template <int KB>
__global__ __launch_bounds__(256) void k_combine_bf16(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ res,
                                                      uint16_t* __restrict__ out, int T, int H,
                                                      int k) {
  const int chunks = H >> 3;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks);
  const int P = T * k;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const int32_t* pr = pair_row + static_cast<size_t>(t) * k;
  const float* wt = w + static_cast<size_t>(t) * k;
  const u32x4_t rv = res ? ld16(res + static_cast<size_t>(t) * H + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
  for (int j0 = 0; j0 < k; j0 += KB) {
    int row[KB];
    float wj[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = min(j0 + u, k - 1);
      row[u] = min(max(pr[j], 0), P - 1);
      wj[u] = wt[j];
    }
    u32x4_t v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) v[u] = ld16(y + static_cast<size_t>(row[u]) * H + c * 8);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (j0 + u < k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(wj[u], __uint_as_float(v[u][i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wj[u], __uint_as_float(v[u][i] & 0xffff0000u), acc[2 * i + 1]);
        }
      }
    }
  }
  if (res) {
    const u32x4_t v = rv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(v[i] << 16);
      acc[2 * i + 1] += __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(t) * H + c * 8) = o;
}

__global__ __launch_bounds__(256) void k_combine_f32(const float* __restrict__ y,
                                                     const int32_t* __restrict__ pair_row,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ res,
                                                     float* __restrict__ out, int T, int H, int k) {
  const int chunks = H >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * chunks) return;
  const int t = static_cast<int>(idx / chunks), c = static_cast<int>(idx % chunks);
  const int P = T * k;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int row = min(max(pair_row[static_cast<size_t>(t) * k + j], 0), P - 1);
    const float wj = w[static_cast<size_t>(t) * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + static_cast<size_t>(row) * H + c * 4);
    acc[0] = fmaf(wj, v.x, acc[0]);
    acc[1] = fmaf(wj, v.y, acc[1]);
    acc[2] = fmaf(wj, v.z, acc[2]);
    acc[3] = fmaf(wj, v.w, acc[3]);
  }
  if (res) {
    const float4 v = *reinterpret_cast<const float4*>(res + static_cast<size_t>(t) * H + c * 4);
    acc[0] += v.x;
    acc[1] += v.y;
    acc[2] += v.z;
    acc[3] += v.w;
  }
  *reinterpret_cast<float4*>(out + static_cast<size_t>(t) * H + c * 4) =
      make_float4(acc[0], acc[1], acc[2], acc[3]);
}

hipError_t launch_combine(const moe_shape& s, const void* y, const int32_t* pair_row,
                          const float* w, const void* residual, void* out, hipStream_t st) {
  if (s.act == MOE_DT_BF16) {
    const size_t n = static_cast<size_t>(s.T) * (s.H / 8);
    auto kern = s.top_k <= 16 ? k_combine_bf16<16> : k_combine_bf16<8>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       st, static_cast<const uint16_t*>(y), pair_row, w,
                       static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(out), s.T,
                       s.H, s.top_k);
  } else {
    const size_t n = static_cast<size_t>(s.T) * (s.H / 4);
    hipLaunchKernelGGL(k_combine_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       st, static_cast<const float*>(y), pair_row, w,
                       static_cast<const float*>(residual), static_cast<float*>(out), s.T, s.H,
                       s.top_k);
  }
  return hipGetLastError();
}

}  // namespace moe
