// Gate/up -> down as component waves inside one kernel, with the weighted
// combine reading the per-slice partial results.
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist", section "Hypothesis H4: ExpertMajor
// should stream as a wavefront, not a barrier": gate and up are used together
// and down only once the SwiGLU intermediate exists; expert work proceeds in
// bounded waves (widths 2, 4 or all selected experts) rather than behind one
// barrier; results go to separate slots and the final weighted sum keeps the
// route-rank order.
//
// Work item = (tile, slice): kFusedCols consecutive intermediate columns of
// the tile's expert.  The workgroup computes
//   h[row][c] = silu(Wg[c] . x[row]) * (Wu[c] . x[row])        (its 64 columns c)
// keeps h in LDS as bf16 (the rounding the two-kernel path applies to its
// intermediate), and right away applies the matching 64 columns of the down
// projection:
//   part[slice][row][n] = sum over its c of Wd[n][c] h[row][c]   (all n < H)
// in float32.  The expert output of a row is the sum of its slices in
// ascending slice order.  No workgroup waits for another: the intermediate
// never leaves the CU and nothing separates the gate/up of one item from its
// down.  Items are numbered in waves of `band` tiles, slice-major inside a
// wave (tile_item); with T <= 16 every active expert is one tile, so a wave
// of W tiles is a wave of W experts.
#include "ffn_tiled.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kHsStride = kFusedCols + 8;   // LDS row stride of h in bf16 (padded)

// One workgroup of 4 waves per item.  Gate/up: wave w owns intermediate
// columns 16w .. 16w+15 of the slice for gate and for up over the full K = H,
// loading US 128-k units before computing them.  Down: wave w owns H/4 output
// features in 16-row blocks, DG blocks per load batch, K = the slice's 64
// columns (half of one 128-k unit of the tiled down matrix).
template <int WF, int NB, int US, int DG>
__global__ __launch_bounds__(256) void k_ffn_fused(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint8_t* __restrict__ wd, const uint16_t* __restrict__ sg,
    const uint16_t* __restrict__ su, const uint16_t* __restrict__ sd,
    const int32_t* __restrict__ tiles, int max_tiles, const int32_t* __restrict__ sorted_pair,
    int k, int H, int I, int P, float* __restrict__ part, int band,
    uint64_t* __restrict__ clock) {
  __shared__ __align__(16) uint16_t hs[NB * 16 * kHsStride];
  const uint64_t t0 = static_cast<uint64_t>(wall_clock64());
  int ti, sl;
  if (!tile_item(tiles[3 * max_tiles], I / kFusedCols, band, false, ti, sl)) return;
  const Tile tl = read_tile(tiles, ti);
  const size_t item = blockIdx.x;
  if (tl.rows <= 0) {
    if (clock && threadIdx.x == 0) clock[3 * item] = clock[3 * item + 1] = clock[3 * item + 2] = t0;
    return;
  }
  // wave index as a uniform value (the slab bases below must live in SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const Dq dq = dq_consts<WF>();

  // ---- gate/up + SwiGLU for columns c0 .. c0+15 ------------------------------
  const int c0 = sl * kFusedCols + wave * 16;
  const size_t gb = (static_cast<size_t>(tl.e) * I + c0) / 16;
  const Slab<WF> Sg(wg, sg, gb, 1, H), Su(wu, su, gb, 1, H);
  const uint16_t* px[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int rr = min(b * 16 + r, tl.rows - 1);
    int p = sorted_pair[tl.row0 + rr];
    p = min(max(p, 0), P - 1);
    px[b] = x + static_cast<size_t>(p / k) * H + q * 8;
  }
  f32x4_t acc[2][NB];
#pragma unroll
  for (int gu = 0; gu < 2; ++gu)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[gu][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int units = H / 128;
  for (int u0 = 0; u0 < units; u0 += US) {
    TScales sc[US][2];
    TRaw<WF> raw[US][2];
    u32x4_t xa[US][4][NB];
#pragma unroll
    for (int v = 0; v < US; ++v) {
      const int u = min(u0 + v, units - 1);   // a tail batch reloads the last unit, unused
      if constexpr (WF != WF_BF16) {
        sc[v][0] = tscales<WF, weight_aux<NB>()>(Sg, 0, u, r);
        sc[v][1] = tscales<WF, weight_aux<NB>()>(Su, 0, u, r);
      }
      raw[v][0] = tload<WF, weight_aux<NB>()>(Sg, 0, u, lane);
      raw[v][1] = tload<WF, weight_aux<NB>()>(Su, 0, u, lane);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < NB; ++b) xa[v][st][b] = ld16(px[b] + 128 * u + 32 * st);
    }
    SCHED_FENCE();
#pragma unroll
    for (int v = 0; v < US; ++v) {
      if (u0 + v >= units) break;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        f32x4_t corr[NB];
        if constexpr (WF != WF_BF16) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
            corr[b] = mfma_bf16(xa[v][st][b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          const u32x4_t wv = tdecode<WF>(raw[v][gu], st, dq);
          if constexpr (WF == WF_BF16) {
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[gu][b] = mfma_bf16(xa[v][st][b], wv, acc[gu][b]);
          } else {
            const float sv = sc[v][gu].f32(st);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const f32x4_t pp = mfma_bf16(xa[v][st][b], wv, corr[b]);
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[gu][b][j] = fmaf(sv, pp[j], acc[gu][b][j]);
            }
          }
        }
      }
    }
  }
  // lane (r, q) holds tokens b*16 + 4q + j of column c0 + r
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      hs[(b * 16 + 4 * q + j) * kHsStride + wave * 16 + r] =
          f32_to_bf16(silu(acc[0][b][j]) * acc[1][b][j]);
  __syncthreads();
  const uint64_t t1 = static_cast<uint64_t>(wall_clock64());

  // ---- down: part[sl][row][n] for this wave's H/4 features -------------------
  // A operand of chunk c: token row b*16 + r, slice columns 32c + 8q .. +7
  u32x4_t ha[2][NB];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      ha[c][b] = *reinterpret_cast<const u32x4_t*>(&hs[(b * 16 + r) * kHsStride + 32 * c + 8 * q]);
  f32x4_t corr[2][NB];
  if constexpr (WF != WF_BF16) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        corr[c][b] = mfma_bf16(ha[c][b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
  }
  const int nblk = H / 64;                      // 16-row output blocks per wave
  const size_t db = static_cast<size_t>(tl.e) * (H / 16) + static_cast<size_t>(wave) * nblk;
  const Slab<WF> Sd(wd, sd, db, nblk, I);
  const int kb = sl >> 1, hf = sl & 1;          // 128-k unit holding the slice, and its half
  float* prow = part + (static_cast<size_t>(sl) * P + tl.row0) * H + static_cast<size_t>(wave) * nblk * 16;
  for (int m0 = 0; m0 < nblk; m0 += DG) {
    u32x4_t wb[WF == WF_BF16 ? DG : 1][2];
    u32x2_t w4[WF == WF_INT4 ? DG : 1];
    uint32_t w2[WF == WF_INT2 ? DG : 1];
    uint32_t scd[WF != WF_BF16 ? DG : 1];
#pragma unroll
    for (int i = 0; i < DG; ++i) {
      const int m = min(m0 + i, nblk - 1);      // a tail batch reloads the last block, unused
      if constexpr (WF == WF_BF16) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
          wb[i][c] = __builtin_amdgcn_raw_buffer_load_b128(Sd.w, lane * 16,
                                                           (m * (I / 32) + 2 * sl + c) * 1024, weight_aux<NB>());
      } else if constexpr (WF == WF_INT4) {
        w4[i] = __builtin_amdgcn_raw_buffer_load_b64(Sd.w, lane * 16 + 8 * hf,
                                                     (m * (I / 128) + kb) * 1024, weight_aux<NB>());
      } else {
        w2[i] = __builtin_amdgcn_raw_buffer_load_b32(Sd.w, lane * 8 + 4 * hf,
                                                     (m * (I / 128) + kb) * 512, weight_aux<NB>());
      }
      if constexpr (WF != WF_BF16)
        scd[i] = __builtin_amdgcn_raw_buffer_load_b32(Sd.s, r * 8 + 4 * hf, (m * (I / 128) + kb) * 128,
                                                      weight_aux<NB>());
    }
    SCHED_FENCE();
#pragma unroll
    for (int i = 0; i < DG; ++i) {
      if (m0 + i >= nblk) break;
      f32x4_t o[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4_t wv;
        if constexpr (WF == WF_BF16) wv = wb[i][c];
        else if constexpr (WF == WF_INT4) wv = dequant_int4_tiled(w4[i][c], dq);
        else wv = c ? dequant_int2_tiled<1>(w2[i], dq) : dequant_int2_tiled<0>(w2[i], dq);
        if constexpr (WF == WF_BF16) {
#pragma unroll
          for (int b = 0; b < NB; ++b) o[b] = mfma_bf16(ha[c][b], wv, o[b]);
        } else {
          const float sv = fp16_to_f32(static_cast<uint16_t>(c ? scd[i] >> 16 : scd[i]));
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t pp = mfma_bf16(ha[c][b], wv, corr[c][b]);
#pragma unroll
            for (int j = 0; j < 4; ++j) o[b][j] = fmaf(sv, pp[j], o[b][j]);
          }
        }
      }
      // lane (r, q) holds tokens b*16 + 4q + j of output feature 16 (m0+i) + r
      const int n = (m0 + i) * 16 + r;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = b * 16 + 4 * q + j;
          if (rr < tl.rows) prow[static_cast<size_t>(rr) * H + n] = o[b][j];
        }
    }
  }
  if (clock) {
    __syncthreads();
    if (threadIdx.x == 0) {
      clock[3 * item] = t0;
      clock[3 * item + 1] = t1;
      clock[3 * item + 2] = static_cast<uint64_t>(wall_clock64());
    }
  }
}

template <int WF, int NB>
static void fused_launch(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                         const int32_t* sorted_pair, const int32_t* tiles, float* part, int band,
                         uint64_t* clock, hipStream_t st) {
  // units per gate/up batch and down blocks per batch: about 256 B of weights
  // in flight per lane, fewer when the token tile is taller
  constexpr int US = NB > 1 ? 1 : (WF == WF_BF16 ? 2 : 4);
  constexpr int DG = (WF == WF_BF16 ? 8 : 16) / NB;
  const int64_t n = static_cast<int64_t>(pl.max_tiles) * fused_slices(s);
  hipLaunchKernelGGL((k_ffn_fused<WF, NB, US, DG>), dim3(static_cast<unsigned>((n + 7) / 8 * 8)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(x),
                     static_cast<const uint8_t*>(ex.gate), static_cast<const uint8_t*>(ex.up),
                     static_cast<const uint8_t*>(ex.down), ex.gate_scale, ex.up_scale,
                     ex.down_scale, tiles, pl.max_tiles, sorted_pair, s.top_k, s.H, s.I,
                     s.T * s.top_k, part, band, clock);
}

template <int WF>
static void fused_nb(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                     const int32_t* sp, const int32_t* tiles, float* part, int band,
                     uint64_t* clock, hipStream_t st) {
  switch (pl.nb) {
    case 1: fused_launch<WF, 1>(s, pl, x, ex, sp, tiles, part, band, clock, st); break;
    case 2: fused_launch<WF, 2>(s, pl, x, ex, sp, tiles, part, band, clock, st); break;
    default: fused_launch<WF, 4>(s, pl, x, ex, sp, tiles, part, band, clock, st); break;
  }
}

hipError_t launch_ffn_fused(const moe_shape& s, const Plan& pl, const void* x,
                            const moe_experts& ex, const int32_t* sorted_pair,
                            const int32_t* tiles, float* part, int wave_tiles, uint64_t* clock,
                            hipStream_t st) {
  const int band = wave_tiles <= 0 ? pl.max_tiles : std::min(wave_tiles, pl.max_tiles);
  if (s.wfmt == MOE_WF_DENSE) fused_nb<WF_BF16>(s, pl, x, ex, sorted_pair, tiles, part, band, clock, st);
  else if (s.wfmt == MOE_WF_INT4_G32) fused_nb<WF_INT4>(s, pl, x, ex, sorted_pair, tiles, part, band, clock, st);
  else fused_nb<WF_INT2>(s, pl, x, ex, sorted_pair, tiles, part, band, clock, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Consumers of the partial slots.
// ---------------------------------------------------------------------------

// Sum of the S slices of 8 consecutive features of one row, slices in
// ascending order; loads of up to 8 slices are issued before they are added.
__device__ __forceinline__ void sum_slices(const float* __restrict__ part, int S, size_t slice_stride,
                                           float (&a)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4_t v[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* p = part + static_cast<size_t>(min(s0 + u, S - 1)) * slice_stride;
      v[u][0] = *reinterpret_cast<const f32x4_t*>(p);
      v[u][1] = *reinterpret_cast<const f32x4_t*>(p + 4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < S) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] += v[u][0][i];
          a[4 + i] += v[u][1][i];
        }
      }
    }
  }
}

// y[row] = bf16(sum of the row's slices); one thread per 8 features.
__global__ __launch_bounds__(256) void k_reduce_parts(const float* __restrict__ part, int S, int P,
                                                      int H, uint16_t* __restrict__ y) {
  const int chunks = H >> 3;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(P) * chunks) return;
  const size_t row = idx / chunks;
  const int c = static_cast<int>(idx % chunks);
  float a[8];
  sum_slices(part + row * H + c * 8, S, static_cast<size_t>(P) * H, a);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = static_cast<uint32_t>(f32_to_bf16(a[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16(a[2 * i + 1])) << 16);
  *reinterpret_cast<u32x4_t*>(y + row * H + c * 8) = o;
}

// out[t][n] = residual[t][n] + sum_j w[t][j] * y_j[n], j ascending, where
// y_j (float32, not rounded) is the slice sum of row pair_row[t*k + j].
// Workgroup = 16 route slots x 16 chunks of 8 features (128 features of one
// token): the 16 slots of a batch are summed in parallel into LDS, then one
// thread per chunk accumulates them in rank order.
constexpr int kCombineSlots = 16;

__global__ __launch_bounds__(256) void k_combine_parts(const float* __restrict__ part, int S,
                                                       const int32_t* __restrict__ pair_row,
                                                       const float* __restrict__ w,
                                                       const uint16_t* __restrict__ res,
                                                       uint16_t* __restrict__ out, int T, int H,
                                                       int k) {
  __shared__ float yv[kCombineSlots][16][8];
  const int groups = H / 128;
  const int t = static_cast<int>(blockIdx.x) / groups, g = static_cast<int>(blockIdx.x) % groups;
  const int js = threadIdx.x >> 4, cl = threadIdx.x & 15;
  const int n = g * 128 + cl * 8;
  const int P = T * k;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
    if (j0 + js < k) {
      const int row = min(max(pair_row[static_cast<size_t>(t) * k + j0 + js], 0), P - 1);
      float a[8];
      sum_slices(part + static_cast<size_t>(row) * H + n, S, static_cast<size_t>(P) * H, a);
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[js][cl][i] = a[i];
    }
    __syncthreads();
    if (js == 0) {
      const int nj = min(kCombineSlots, k - j0);
      for (int u = 0; u < nj; ++u) {
        const float wj = w[static_cast<size_t>(t) * k + j0 + u];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, yv[u][cl][i], acc[i]);
      }
    }
    __syncthreads();
  }
  if (js != 0) return;
  if (res) {
    const u32x4_t v = ld16(res + static_cast<size_t>(t) * H + n);
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
  *reinterpret_cast<u32x4_t*>(out + static_cast<size_t>(t) * H + n) = o;
}

hipError_t launch_reduce_parts(const moe_shape& s, const float* part, void* y, hipStream_t st) {
  const size_t n = static_cast<size_t>(s.T) * s.top_k * (s.H / 8);
  hipLaunchKernelGGL(k_reduce_parts, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                     part, fused_slices(s), s.T * s.top_k, s.H, static_cast<uint16_t*>(y));
  return hipGetLastError();
}

hipError_t launch_combine_parts(const moe_shape& s, const float* part, const int32_t* pair_row,
                                const float* w, const void* residual, void* out, hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>(s.T) * static_cast<unsigned>(s.H / 128);
  hipLaunchKernelGGL(k_combine_parts, dim3(blocks), dim3(256), 0, st, part, fused_slices(s),
                     pair_row, w, static_cast<const uint16_t*>(residual),
                     static_cast<uint16_t*>(out), s.T, s.H, s.top_k);
  return hipGetLastError();
}

}  // namespace moe
