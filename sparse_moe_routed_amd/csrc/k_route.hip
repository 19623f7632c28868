// Router logits and exact top-k selection.
//
// Reference: "Agent Field Notes -- full corpus", AFN-001 "Porting
// Qwen3.8-Flash-Next to Hebrus: evidence before execution", section "Phase 1:
// separate math from acceleration" (float32 router softmax and normalized
// top-10 selection); AFN-021 "Replay decode as prefill", section "The key
// equivalence -- and where it breaks" (exact IDs in rank order); AFN-017 "Top-k
// chooses the set; time chooses the order", section "Tie handling belongs to
// membership" (equal scores: the smaller index is chosen during membership).
#include <climits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// bf16 router: one 16-expert x 16-token tile per workgroup; wave w sums the
// K quarter [w H/4, (w+1) H/4).  Each v_mfma_f32_16x16x32_bf16 sums 32 exact
// bf16 products in float32; those chunk sums are accumulated in float64 in k
// order, the four quarter sums are added in wave order, the bias is added,
// and the total is rounded once to float32.  The association is the same
// for every token and every batch size, so a token's logits do not depend on
// which other tokens share the call.
// grid (ceil(T/16), ceil(E/16)), block 256.
__global__ __launch_bounds__(256) void k_router_bf16(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wr,
                                                     const float* __restrict__ bias, int T, int H,
                                                     int E, float* __restrict__ logits) {
  __shared__ double red[4][64][4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int kq = H >> 2;
  const int kbeg = wave * kq;
  const int tt = min(t0 + r, T - 1);
  const int ee = min(e0 + r, E - 1);
  const uint16_t* xp = x + static_cast<size_t>(tt) * H + kbeg + q * 8;
  const uint16_t* wp = wr + static_cast<size_t>(ee) * H + kbeg + q * 8;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int kk = 0; kk < kq; kk += 32) {
    const u32x4_t a = ld16(wp + kk);
    const u32x4_t b = ld16(xp + kk);
    const f32x4_t c = mfma_bf16(a, b, zero);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += static_cast<double>(c[j]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][lane][j] = acc[j];
  __syncthreads();
  if (wave == 0) {
    const int t = t0 + r;
    if (t < T) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 4 * q + j;
        if (e < E) {
          double s = ((red[0][lane][j] + red[1][lane][j]) + red[2][lane][j]) + red[3][lane][j];
          if (bias) s += static_cast<double>(bias[e]);
          logits[static_cast<size_t>(t) * E + e] = static_cast<float>(s);
        }
      }
    }
  }
}

// float32 router: one thread per (token, expert), products and sums in
// float64 in ascending h, bias added, rounded once to float32.
__global__ __launch_bounds__(256) void k_router_f32(const float* __restrict__ x,
                                                    const float* __restrict__ wr,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, float* __restrict__ logits) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * E) return;
  const int t = static_cast<int>(idx / E), e = static_cast<int>(idx % E);
  const float* xp = x + static_cast<size_t>(t) * H;
  const float* wp = wr + static_cast<size_t>(e) * H;
  double s = 0.0;
  for (int h = 0; h < H; ++h) s += static_cast<double>(xp[h]) * static_cast<double>(wp[h]);
  if (bias) s += static_cast<double>(bias[e]);
  logits[idx] = static_cast<float>(s);
}

// Exact top-k per token, one wave per token (E <= 1024: 16 logits per lane).
// Selection uses the total order (logit descending, index ascending) on the
// float32 logits, k rounds of a wave arg-max.  Weights: exp(l_j - l_0) / sum
// over the selected, in float32 (the full softmax renormalized over the
// selection).
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const bool active = t < T;
  float v[16];
  uint32_t live = 0;
  if (active) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = j * 64 + lane;
      v[j] = 0.f;
      if (e < E) {
        v[j] = logits[static_cast<size_t>(t) * E + e];
        live |= 1u << j;
      }
    }
    for (int rnk = 0; rnk < k; ++rnk) {
      float bv = 0.f;
      int be = INT_MAX;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if ((live >> j) & 1u) {
          const int e = j * 64 + lane;
          if (be == INT_MAX || v[j] > bv || (v[j] == bv && e < be)) {
            bv = v[j];
            be = e;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oe = __shfl_xor(be, off, kWave);
        const bool take = oe != INT_MAX && (be == INT_MAX || ov > bv || (ov == bv && oe < be));
        if (take) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) live &= ~(1u << (be >> 6));
      if (lane == 0) {
        ids[static_cast<size_t>(t) * k + rnk] = be;
        sel[wave][rnk] = bv;
      }
    }
  }
  __syncthreads();
  if (active) {
    const float m0 = sel[wave][0];
    float sum = 0.f;
    for (int rnk = lane; rnk < k; rnk += 64) {
      const float ex = expf(sel[wave][rnk] - m0);
      sel[wave][rnk] = ex;
      sum += ex;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    for (int rnk = lane; rnk < k; rnk += 64) w[static_cast<size_t>(t) * k + rnk] = sel[wave][rnk] / sum;
  }
}

hipError_t launch_route(const moe_shape& s, const Plan& pl, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* w, float* logits, void* ws,
                        hipStream_t st) {
  float* lg = logits ? logits : reinterpret_cast<float*>(static_cast<char*>(ws) + pl.logits_off);
  if (s.act == MOE_DT_BF16) {
    dim3 grid((s.T + 15) / 16, (s.E + 15) / 16);
    hipLaunchKernelGGL(k_router_bf16, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, lg);
  } else {
    const size_t n = static_cast<size_t>(s.T) * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), bias, s.T,
                       s.H, s.E, lg);
  }
  hipLaunchKernelGGL(k_topk, dim3((s.T + 3) / 4), dim3(256), 0, st, lg, s.T, s.E, s.top_k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
