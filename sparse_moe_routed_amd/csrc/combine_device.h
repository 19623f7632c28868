// Device code of the route-rank-order combine, shared by the combine kernel
// and the down kernel that combines an output slice in its last workgroup
// (down + combine in one launch), so both compute the same bits.
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Hypothesis H4: ExpertMajor
// should stream as a wavefront, not a barrier": experts write separate
// result slots and the final weighted sum follows a deterministic
// route-rank order.
#pragma once

#include "moe_device.h"

namespace moe {

// out[t][8c .. 8c+7] = residual + sum_{j=0}^{k-1} w[t][j] * y[row_of(j)][...]:
// float32 fused multiply-adds with j ascending, then the residual added,
// then one rounding to bf16.  load_y(row, c) returns the 8 bf16 values
// y[row][8c .. 8c+7].  KB slots per batch: all weight loads and row
// indices of a batch, then all its row loads, then the accumulation, so
// KB >= k makes the whole sum two dependent memory round trips.
template <int KB, typename LoadY, typename RowOf>
__device__ __forceinline__ void combine_chunk_bf16(LoadY load_y, RowOf row_of,
                                                   const float* __restrict__ w,
                                                   const uint16_t* __restrict__ res,
                                                   uint16_t* __restrict__ out, int t, int c, int H,
                                                   int k) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  const float* wt = w + static_cast<size_t>(t) * k;
  const u32x4_t rv = res ? ld16(res + static_cast<size_t>(t) * H + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
  for (int j0 = 0; j0 < k; j0 += KB) {
    int row[KB];
    float wj[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = min(j0 + u, k - 1);
      row[u] = row_of(j);
      wj[u] = wt[j];
    }
    u32x4_t v[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) v[u] = load_y(row[u], c);
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(rv[i] << 16);
      acc[2 * i + 1] += __uint_as_float(rv[i] & 0xffff0000u);
    }
  }
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(t) * H + c * 8) = o;
}

}  // namespace moe
