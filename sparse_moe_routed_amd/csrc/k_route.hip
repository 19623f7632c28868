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
#include "route_device.h"

namespace moe {

// bf16 router.  The dot product over H is cut into `nparts` parts of
// `cpp` chunks of 32 (nparts = the largest divisor of H/32 that is <= 16, so
// the cut depends on H alone).  Each v_mfma_f32_16x16x32_bf16 sums the 32
// exact bf16 products of a chunk in float32; the chunk sums of a part are
// added in float64 in k order, the part sums are added in part order, the
// bias is added, and the total is rounded once to float32.  Both kernels
// below use exactly this association, so a token's logits are bit-identical
// whatever the batch size or the kernel that computed them.

// Small batches: one 16-token x 16-expert tile per workgroup, one wave per
// part, part sums combined through LDS.  grid (ceil(T/16), ceil(E/16)),
// block 64 * nparts.
__global__ __launch_bounds__(1024) void k_router_parts(const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ wr,
                                                       const float* __restrict__ bias, int T,
                                                       int H, int E, int nparts,
                                                       float* __restrict__ logits) {
  __shared__ double red[16][64][4];
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  router_part(x, wr, T, H, E, nparts, t0, e0, wave, red);
  __syncthreads();
  if (wave == 0) router_store(red, bias, T, E, nparts, t0, e0, logits);
}

// Larger batches: workgroup tile of 32 A tokens x 32 A experts, four waves
// in 2 x 2, each (16 A) x (16 A).  Token rows and router rows are staged in
// LDS once per workgroup and 128-wide k unit (in MFMA fragment order), and
// each wave walks the 32-wide chunks in k order, keeping a float64 part sum
// and a float64 total per output (the association above).  Two LDS buffers:
// the next unit is loaded while the current one is multiplied.
// grid (ceil(T / 32 A), ceil(E / 32 A)), block 256.
template <int A>
__global__ __launch_bounds__(256) void k_router_lds(const uint16_t* __restrict__ x,
                                                    const uint16_t* __restrict__ wr,
                                                    const float* __restrict__ bias, int T, int H,
                                                    int E, int nparts,
                                                    float* __restrict__ logits) {
  constexpr int NB = 2 * A;   // 16-row blocks per staged tile
  __shared__ __align__(16) char xs[2][NB * 4096];
  __shared__ __align__(16) char wsm[2][NB * 4096];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int tb = blockIdx.x * 32 * A, eb = blockIdx.y * 32 * A;
  const int tblk = (wave & 1) * A, eblk = (wave >> 1) * A;
  const int cpp = H / 32 / nparts;
  const int units = H / 128;

  XUnit<NB> xu, wu;
  xu.init(x, [&](int R) { return static_cast<size_t>(min(tb + R, T - 1)) * H; });
  wu.init(wr, [&](int R) { return static_cast<size_t>(min(eb + R, E - 1)) * H; });

  double part[A][A][4], tot[A][A][4];
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int i = 0; i < A; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[a][i][j] = tot[a][i][j] = 0.0;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  xu.load(0);
  wu.load(0);
  xu.store(xs[0]);
  wu.store(wsm[0]);
  __syncthreads();
  for (int u = 0; u < units; ++u) {
    if (u + 1 < units) {
      xu.load(u + 1);
      wu.load(u + 1);
    }
    const char* bx = xs[u & 1];
    const char* bw = wsm[u & 1];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4_t xa[A], wa[A];
#pragma unroll
      for (int i = 0; i < A; ++i) xa[i] = xfrag<NB>(bx, st, tblk + i, lane);
#pragma unroll
      for (int a = 0; a < A; ++a) wa[a] = xfrag<NB>(bw, st, eblk + a, lane);
#pragma unroll
      for (int a = 0; a < A; ++a)
#pragma unroll
        for (int i = 0; i < A; ++i) {
          const f32x4_t f = mfma_bf16(wa[a], xa[i], zero);
#pragma unroll
          for (int j = 0; j < 4; ++j) part[a][i][j] += static_cast<double>(f[j]);
        }
      if ((4 * u + st + 1) % cpp == 0) {
#pragma unroll
        for (int a = 0; a < A; ++a)
#pragma unroll
          for (int i = 0; i < A; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              tot[a][i][j] += part[a][i][j];
              part[a][i][j] = 0.0;
            }
      }
    }
    if (u + 1 < units) {
      xu.store(xs[(u + 1) & 1]);
      wu.store(wsm[(u + 1) & 1]);
    }
    __syncthreads();
  }
  // lane holds experts eb + 16 (eblk + a) + 4 q + j of token tb + 16 (tblk + i) + r
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int t = tb + 16 * (tblk + i) + r;
    if (t >= T) continue;
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = eb + 16 * (eblk + a) + 4 * q + j;
        if (e < E) {
          double sum = tot[a][i][j];
          if (bias) sum += static_cast<double>(bias[e]);
          logits[static_cast<size_t>(t) * E + e] = static_cast<float>(sum);
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

// Exact top-k, one wave per token (topk_token).  grid ceil(T/4), block 256.
template <int NV>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel[4][1024];
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;   // whole wave leaves; no workgroup barrier below
  const size_t o = static_cast<size_t>(t) * k;
  topk_token<NV>(logits + static_cast<size_t>(t) * E, E, k, sel[wave], ids + o, w + o, nullptr);
}

template <int NV>
static void launch_topk(const moe_shape& s, const float* lg, int32_t* ids, float* w, hipStream_t st) {
  hipLaunchKernelGGL((k_topk<NV>), dim3((s.T + 3) / 4), dim3(256), 0, st, lg, s.T, s.E, s.top_k, ids, w);
}

static hipError_t launch_router(const moe_shape& s, const void* x, const void* w_router,
                                const float* bias, float* lg, hipStream_t st) {
  if (s.act == MOE_DT_BF16) {
    const int np = router_parts(s.H);
    if (s.T <= 64) {
      dim3 grid((s.T + 15) / 16, (s.E + 15) / 16);
      hipLaunchKernelGGL(k_router_parts, grid, dim3(64 * np), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, np, lg);
    } else if (s.T <= 1024) {
      dim3 grid((s.T + 31) / 32, (s.E + 31) / 32);
      hipLaunchKernelGGL(k_router_lds<1>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, np, lg);
    } else {
      dim3 grid((s.T + 63) / 64, (s.E + 63) / 64);
      hipLaunchKernelGGL(k_router_lds<2>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                         static_cast<const uint16_t*>(w_router), bias, s.T, s.H, s.E, np, lg);
    }
  } else {
    const size_t n = static_cast<size_t>(s.T) * s.E;
    hipLaunchKernelGGL(k_router_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), bias, s.T,
                       s.H, s.E, lg);
  }
  return hipGetLastError();
}

hipError_t launch_route(const moe_shape& s, const Plan& pl, const void* x, const void* w_router,
                        const float* bias, int32_t* ids, float* w, float* logits, void* ws,
                        hipStream_t st) {
  float* lg = logits ? logits : reinterpret_cast<float*>(static_cast<char*>(ws) + pl.logits_off);
  hipError_t e = launch_router(s, x, w_router, bias, lg, st);
  if (e != hipSuccess) return e;
  const int nv = (s.E + 63) / 64;
  if (nv <= 1) launch_topk<1>(s, lg, ids, w, st);
  else if (nv <= 2) launch_topk<2>(s, lg, ids, w, st);
  else if (nv <= 4) launch_topk<4>(s, lg, ids, w, st);
  else if (nv <= 8) launch_topk<8>(s, lg, ids, w, st);
  else launch_topk<16>(s, lg, ids, w, st);
  return hipGetLastError();
}

}  // namespace moe
