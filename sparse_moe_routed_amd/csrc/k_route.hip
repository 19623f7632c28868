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

// bf16 router.  The dot product over H is cut into `nparts` parts of
// `cpp` chunks of 32 (nparts = the largest divisor of H/32 that is <= 16, so
// the cut depends on H alone).  Each v_mfma_f32_16x16x32_bf16 sums the 32
// exact bf16 products of a chunk in float32; the chunk sums of a part are
// added in float64 in k order, the part sums are added in part order, the
// bias is added, and the total is rounded once to float32.  Both kernels
// below use exactly this association, so a token's logits are bit-identical
// whatever the batch size or the kernel that computed them.
constexpr int kRouterBatch = 8;

// Small batches: one 16-token x 16-expert tile per workgroup, one wave per
// part, part sums combined through LDS.  grid (ceil(T/16), ceil(E/16)),
// block 64 * nparts.
__global__ __launch_bounds__(1024) void k_router_parts(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       const float* __restrict__ bias, int T,
                                                       int H, int E, int nparts,
                                                       float* __restrict__ logits) {
  __shared__ double red[16][64][4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int cpp = H / 32 / nparts;
  const int kbeg = wave * cpp * 32;
  const int tt = min(t0 + r, T - 1);
  const int ee = min(e0 + r, E - 1);
  const uint16_t* xp = x + static_cast<size_t>(tt) * H + kbeg + q * 8;
  const uint16_t* wp = wr + static_cast<size_t>(ee) * H + kbeg + q * 8;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < cpp; c += kRouterBatch) {
    u32x4_t a[kRouterBatch], b[kRouterBatch];
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (c + u < cpp) {
        a[u] = ld16(wp + (c + u) * 32);
        b[u] = ld16(xp + (c + u) * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < kRouterBatch; ++u) {
      if (c + u < cpp) {
        const f32x4_t f = mfma_bf16(a[u], b[u], zero);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += static_cast<double>(f[j]);
      }
    }
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
          double s = red[0][lane][j];
          for (int w = 1; w < nparts; ++w) s += red[w][lane][j];
          if (bias) s += static_cast<double>(bias[e]);
          logits[static_cast<size_t>(t) * E + e] = static_cast<float>(s);
        }
      }
    }
  }
}

// Large batches: each wave owns a 32-token x 32-expert tile (2 x 2 MFMA
// tiles) and walks all parts itself, keeping a float64 part sum and a float64
// total per output (same association as above).  grid (ceil(T/64),
// ceil(E/64)), block 256 (waves 2 x 2 over the 64 x 64 workgroup tile).
__global__ __launch_bounds__(256) void k_router_tiles(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wr,
                                                      const float* __restrict__ bias, int T, int H,
                                                      int E, int nparts,
                                                      float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int t0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int e0 = blockIdx.y * 64 + (wave >> 1) * 32;
  if (t0 >= T || e0 >= E) return;
  const int cpp = H / 32 / nparts;
  const uint16_t* xp[2];
  const uint16_t* wp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xp[i] = x + static_cast<size_t>(min(t0 + 16 * i + r, T - 1)) * H + q * 8;
    wp[i] = wr + static_cast<size_t>(min(e0 + 16 * i + r, E - 1)) * H + q * 8;
  }
  double tot[2][2][4], part[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) tot[a][b][j] = 0.0;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int pidx = 0; pidx < nparts; ++pidx) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[a][b][j] = 0.0;
    const int kb = pidx * cpp * 32;
    for (int c = 0; c < cpp; c += 4) {
      u32x4_t wa[4][2], xb[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c + u < cpp) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            wa[u][i] = ld16(wp[i] + kb + (c + u) * 32);
            xb[u][i] = ld16(xp[i] + kb + (c + u) * 32);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c + u < cpp) {
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const f32x4_t f = mfma_bf16(wa[u][a], xb[u][b], zero);
#pragma unroll
              for (int j = 0; j < 4; ++j) part[a][b][j] += static_cast<double>(f[j]);
            }
        }
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) tot[a][b][j] += part[a][b][j];
  }
  // lane holds experts e0 + 16a + 4q + j of token t0 + 16b + r
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int t = t0 + 16 * b + r;
    if (t >= T) continue;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 16 * a + 4 * q + j;
        if (e < E) {
          double s = tot[a][b][j];
          if (bias) s += static_cast<double>(bias[e]);
          logits[static_cast<size_t>(t) * E + e] = static_cast<float>(s);
        }
      }
  }
}

int router_parts(int H) {
  const int chunks = H / 32;
  int best = 1;
  for (int d = 1; d <= 16; ++d)
    if (chunks % d == 0) best = d;
  return best;
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

// Exact top-k per token, one wave per token; lane l holds the logits of
// experts l, 64 + l, ... (NV slots, E <= 64 NV).  Each of the k rounds takes
// the wave maximum m of the remaining logits, then the smallest expert index
// whose logit equals m -- the total order (logit descending, index
// ascending) -- with DPP row reductions and readlanes (no LDS round trips).
// -0.0 and +0.0 compare equal.  Weights: exp(l_j - l_0) / sum over the
// selected, in float32 (the full softmax renormalized over the selection).
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel[4][1024];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;   // whole wave leaves; no workgroup barrier below
  const float* lt = logits + static_cast<size_t>(t) * E;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = lt[min(j * 64 + lane, E - 1)];
  uint32_t live = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j)
    if (j * 64 + lane < E) live |= 1u << j;
  for (int rnk = 0; rnk < k; ++rnk) {
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if ((live >> j) & 1u) lm = fmaxf(lm, v[j]);
    const float m = wave_max_f32(lm);
    uint32_t li = 0xffffffffu;
#pragma unroll
    for (int j = NV - 1; j >= 0; --j)
      if (((live >> j) & 1u) && v[j] == m) li = static_cast<uint32_t>(j * 64 + lane);
    const uint32_t e = wave_min_u32(li);
    if (static_cast<int>(e & 63u) == lane) live &= ~(1u << (e >> 6));
    if (lane == 0) {
      ids[static_cast<size_t>(t) * k + rnk] = static_cast<int32_t>(e);
      sel[wave][rnk] = m;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float m0 = sel[wave][0];
  float part = 0.f;
  for (int rnk = lane; rnk < k; rnk += 64) {
    const float ex = expf(sel[wave][rnk] - m0);
    sel[wave][rnk] = ex;
    part += ex;
  }
  const float sum = wave_sum_f32(part);
  for (int rnk = lane; rnk < k; rnk += 64) w[static_cast<size_t>(t) * k + rnk] = sel[wave][rnk] / sum;
}

template <int NV>
static void launch_topk(const moe_shape& s, const float* lg, int32_t* ids, float* w, hipStream_t st) {
  hipLaunchKernelGGL((k_topk<NV>), dim3((s.T + 3) / 4), dim3(256), 0, st, lg, s.T, s.E, s.top_k, ids, w);
}

hipError_t launch_route(const moe_shape& s, const Plan& pl, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* w, float* logits, void* ws,
                        hipStream_t st) {
  float* lg = logits ? logits : reinterpret_cast<float*>(static_cast<char*>(ws) + pl.logits_off);
  if (s.act == MOE_DT_BF16) {
    const int np = router_parts(s.H);
    if (s.T <= 64) {
      dim3 grid((s.T + 15) / 16, (s.E + 15) / 16);
      hipLaunchKernelGGL(k_router_parts, grid, dim3(64 * np), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, np, lg);
    } else {
      dim3 grid((s.T + 63) / 64, (s.E + 63) / 64);
      hipLaunchKernelGGL(k_router_tiles, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, np, lg);
    }
  } else {
    const size_t n = static_cast<size_t>(s.T) * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), bias, s.T,
                       s.H, s.E, lg);
  }
  const int nv = (s.E + 63) / 64;
  if (nv <= 1) launch_topk<1>(s, lg, ids, w, st);
  else if (nv <= 2) launch_topk<2>(s, lg, ids, w, st);
  else if (nv <= 4) launch_topk<4>(s, lg, ids, w, st);
  else if (nv <= 8) launch_topk<8>(s, lg, ids, w, st);
  else launch_topk<16>(s, lg, ids, w, st);
  return hipGetLastError();
}

}  // namespace moe
