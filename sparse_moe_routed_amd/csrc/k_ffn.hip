// Grouped SwiGLU experts: gate+up with the SwiGLU epilogue, then down.
//
// Reference: "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses
// before the router knows they exist":
//   section "Hypothesis H4: ExpertMajor should stream as a wavefront, not a
//   barrier" -- gate and up are consumed together, down only after the SwiGLU
//   intermediate exists, and every (token, expert) result goes to its own slot;
//   section "Why overlap alone cannot defeat the byte roofline" -- one expert
//   is gate [I x H] + up [I x H] + down [H x I]; rows grouped by expert and
//   low-bit storage reduce the bytes that must move.
//
// Work decomposition.  The permutation groups each expert's rows; a tile is
// up to 16*NB consecutive rows of one expert.  A workgroup streams a slab of
// weight rows of that expert exactly once from HBM and applies it to every
// row of the tile, so an expert with <= 16*NB rows is read once per call.
// MFMA v_mfma_f32_16x16x32_bf16 with A = activations (16 tokens) and
// B = weights (16 weight rows): lane (r, q) = (l % 16, l / 16) loads 8
// consecutive k of weight row r and of token row r, and the result lane holds
// tokens 4q..4q+3 of weight row r -- so every lane's outputs share one weight
// row, and one group scale per 32-wide k chunk serves all of them.
//
// Low-bit weights: one MFMA per group of 32 codes (codes -> exact bf16
// integers), the float32 group partial is multiplied by the fp16 scale and
// accumulated in float32.
#include <type_traits>

#include "ffn_tiled.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Raw weight bits of one 32-wide k chunk starting at kk for lane chunk q:
// bf16 -> 16 bytes (8 weights), int4 -> 4 bytes (8 codes), int2 -> 2 bytes.
template <int WF>
struct Raw;
template <>
struct Raw<0> {
  typedef u32x4_t type;
};
template <>
struct Raw<1> {
  typedef uint32_t type;
};
template <>
struct Raw<2> {
  typedef uint32_t type;
};

template <int WF>
__device__ __forceinline__ typename Raw<WF>::type load_raw(const uint8_t* row, int kk, int q) {
  if constexpr (WF == WF_BF16) {
    return ld16(row + static_cast<size_t>(kk) * 2 + q * 16);
  } else if constexpr (WF == WF_INT4) {
    return *reinterpret_cast<const uint32_t*>(row + (kk >> 1) + q * 4);
  } else {
    return *reinterpret_cast<const uint16_t*>(row + (kk >> 2) + q * 2);
  }
}

template <int WF>
__device__ __forceinline__ u32x4_t decode_raw(typename Raw<WF>::type v) {
  if constexpr (WF == WF_BF16) {
    return v;
  } else if constexpr (WF == WF_INT4) {
    return dequant_int4x8(v);
  } else {
    return dequant_int2x8(v);
  }
}

template <int U>
__device__ __forceinline__ Scales<U> load_scales(const uint16_t* row, int g) {
  Scales<U> r;
  if constexpr (U == 4) {
    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(row + g);
    r.s[0] = static_cast<uint16_t>(v[0]);
    r.s[1] = static_cast<uint16_t>(v[0] >> 16);
    r.s[2] = static_cast<uint16_t>(v[1]);
    r.s[3] = static_cast<uint16_t>(v[1] >> 16);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) r.s[u] = row[g + u];
  }
  return r;
}

// gate/up + SwiGLU.  32 intermediate rows (two 16-row MFMA blocks) of gate and
// of up per wave.  KSPLIT == 4: the 4 waves of a workgroup share those rows
// and split K, partial sums are added in LDS in wave order (deterministic).
// KSPLIT == 1: each wave owns 32 rows and the full K.  The k loop issues the
// loads of U chunks of 32 before consuming them, so a wave keeps U times more
// bytes in flight (U = 4 needs the wave's k range to be a multiple of 128).
// grid (I / (32 * 4 / KSPLIT), max_tiles), block 256: consecutive workgroups
// stream adjacent row slabs of the same expert.
template <int WF, int NB, int KSPLIT, int U>
__global__ __launch_bounds__(256) void k_gateup(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su,
    const int32_t* __restrict__ tiles, int max_tiles, const int32_t* __restrict__ sorted_pair,
    int k, int H, int I, int P, uint16_t* __restrict__ h) {
  __shared__ f32x4_t red[KSPLIT > 1 ? KSPLIT : 1][2][2][NB][64];
  const int n_tiles = tiles[3 * max_tiles];
  if (static_cast<int>(blockIdx.y) >= n_tiles) return;
  const Tile tl = read_tile(tiles, blockIdx.y);
  if (tl.rows <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int i0 = KSPLIT > 1 ? blockIdx.x * 32 : (blockIdx.x * 4 + wave) * 32;
  const int kq = H / KSPLIT;
  const int kbeg = KSPLIT > 1 ? wave * kq : 0;
  const size_t rb = row_bytes<WF>(H);
  const int ng = H / 32;

  const uint8_t* pw[2][2];
  const uint16_t* ps[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const size_t irow = static_cast<size_t>(tl.e) * I + i0 + mb * 16 + r;
    pw[mb][0] = wg + irow * rb;
    pw[mb][1] = wu + irow * rb;
    if constexpr (WF != WF_BF16) {
      ps[mb][0] = sg + irow * ng;
      ps[mb][1] = su + irow * ng;
    }
  }
  const uint16_t* px[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int rr = min(b * 16 + r, tl.rows - 1);
    int p = sorted_pair[tl.row0 + rr];
    p = min(max(p, 0), P - 1);
    px[b] = x + static_cast<size_t>(p / k) * H + q * 8;
  }

  f32x4_t acc[2][2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[mb][gu][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kk = kbeg; kk < kbeg + kq; kk += 32 * U) {
    Scales<U> sc[2][2];
    if constexpr (WF != WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) sc[mb][gu] = load_scales<U>(ps[mb][gu], kk >> 5);
    }
    u32x4_t xa[U][NB];
    typename Raw<WF>::type raw[U][2][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int b = 0; b < NB; ++b) xa[u][b] = ld16(px[b] + kk + 32 * u);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) raw[u][mb][gu] = load_raw<WF>(pw[mb][gu], kk + 32 * u, q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          const u32x4_t wv = decode_raw<WF>(raw[u][mb][gu]);
          if constexpr (WF == WF_BF16) {
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[mb][gu][b] = mfma_bf16(xa[u][b], wv, acc[mb][gu][b]);
          } else {
            const float s = fp16_to_f32(sc[mb][gu].s[u]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const f32x4_t pp = mfma_bf16(xa[u][b], wv, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mb][gu][b][j] = fmaf(s, pp[j], acc[mb][gu][b][j]);
            }
          }
        }
      }
    }
  }

  if constexpr (KSPLIT > 1) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int gu = 0; gu < 2; ++gu)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[wave][mb][gu][b][lane] = acc[mb][gu][b];
    __syncthreads();
    for (int idx = wave; idx < 2 * NB; idx += 4) {
      const int mb = idx & 1, b = idx >> 1;
      f32x4_t G = red[0][mb][0][b][lane], U_ = red[0][mb][1][b][lane];
#pragma unroll
      for (int w = 1; w < KSPLIT; ++w) {
        G += red[w][mb][0][b][lane];
        U_ += red[w][mb][1][b][lane];
      }
      const int i = i0 + mb * 16 + r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = b * 16 + 4 * q + j;
        if (rr < tl.rows) h[static_cast<size_t>(tl.row0 + rr) * I + i] = f32_to_bf16(silu(G[j]) * U_[j]);
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int i = i0 + mb * 16 + r;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = b * 16 + 4 * q + j;
          if (rr < tl.rows)
            h[static_cast<size_t>(tl.row0 + rr) * I + i] =
                f32_to_bf16(silu(acc[mb][0][b][j]) * acc[mb][1][b][j]);
        }
    }
  }
}

// down: y[row][n] = sum_i W_down[e][n][i] h[row][i].  32 output features per
// wave (two 16-row MFMA blocks), 128 per workgroup, full K = I, loads of U
// k chunks issued before they are consumed (U = 4 needs I % 128 == 0).
// grid (H / 128, max_tiles), block 256.
template <int WF, int NB, int U>
__global__ __launch_bounds__(256) void k_down(const uint16_t* __restrict__ h,
                                              const uint8_t* __restrict__ wd,
                                              const uint16_t* __restrict__ sd,
                                              const int32_t* __restrict__ tiles, int max_tiles,
                                              int H, int I, uint16_t* __restrict__ y) {
  const int n_tiles = tiles[3 * max_tiles];
  if (static_cast<int>(blockIdx.y) >= n_tiles) return;
  const Tile tl = read_tile(tiles, blockIdx.y);
  if (tl.rows <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int n0 = (blockIdx.x * 4 + wave) * 32;
  const size_t rb = row_bytes<WF>(I);
  const int ng = I / 32;
  const uint8_t* pw[2];
  const uint16_t* ps[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const size_t nrow = static_cast<size_t>(tl.e) * H + n0 + mb * 16 + r;
    pw[mb] = wd + nrow * rb;
    if constexpr (WF != WF_BF16) ps[mb] = sd + nrow * ng;
  }
  const uint16_t* ph[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    ph[b] = h + static_cast<size_t>(tl.row0 + min(b * 16 + r, tl.rows - 1)) * I + q * 8;

  f32x4_t acc[2][NB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kk = 0; kk < I; kk += 32 * U) {
    Scales<U> sc[2];
    if constexpr (WF != WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sc[mb] = load_scales<U>(ps[mb], kk >> 5);
    }
    u32x4_t ha[U][NB];
    typename Raw<WF>::type raw[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int b = 0; b < NB; ++b) ha[u][b] = ld16(ph[b] + kk + 32 * u);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) raw[u][mb] = load_raw<WF>(pw[mb], kk + 32 * u, q);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4_t wv = decode_raw<WF>(raw[u][mb]);
        if constexpr (WF == WF_BF16) {
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[mb][b] = mfma_bf16(ha[u][b], wv, acc[mb][b]);
        } else {
          const float s = fp16_to_f32(sc[mb].s[u]);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t pp = mfma_bf16(ha[u][b], wv, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mb][b][j] = fmaf(s, pp[j], acc[mb][b][j]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int n = n0 + mb * 16 + r;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = b * 16 + 4 * q + j;
        if (rr < tl.rows) y[static_cast<size_t>(tl.row0 + rr) * H + n] = f32_to_bf16(acc[mb][b][j]);
      }
  }
}

// gate/up + SwiGLU on tiled weights.  A wave owns MB 16-row blocks of gate
// and of up (16 MB intermediate rows); a workgroup has 4 waves = (4/KSPLIT)
// row groups x KSPLIT k parts, and the k parts of a row group are added in
// LDS in part order (two row blocks at a time).  Low-bit codes enter the MFMA
// as 128 + offset + q; the C operand carries -offset * sum(x) (one MFMA of x
// against a constant fragment per 32-k chunk, shared by all the wave's rows),
// so each group partial is sum(q x) before its fp16 scale is applied.
// 1-D grid over (tile, slice) items, I / (16 MB 4 / KSPLIT) slices per tile;
// block 256.
// Low-bit gate/up with one token block per tile: weight loads rolled a unit
// ahead in place (see k_gateup_t).
template <int WF, int NB>
constexpr bool kRollLowBit() {
  return WF != WF_BF16 && NB == 1;
}

// One row block's k unit in the rolled low-bit kernels: the four chunks are
// decoded, then their four MFMAs issued back to back, then the group scales
// applied, so each MFMA's latency is covered by the MFMAs after it (with the
// chunks interleaved, every scale FMA waited for its MFMA with NOPs).  The
// additions into `acc` run in chunk order.  PS: int2 codes decoded in place
// (tdecode_int2_ps, token fragments prescaled); SP: the 4-row layout.
template <int WF, bool PS, bool SP>
__device__ __forceinline__ void rolled_block_unit(const TRaw<WF>& raw, const TScales& sc,
                                                  const u32x4_t (&a)[4], const f32x4_t (&corr)[4],
                                                  Dq dq, DqPs dps, f32x4_t& acc) {
  u32x4_t wv[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if constexpr (PS) wv[st] = tdecode_int2_ps(raw, st, dps);
    else wv[st] = tdecode<WF>(raw, st, dq);
  }
  f32x4_t pp[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) pp[st] = mfma_bf16(a[st], wv[st], corr[st]);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const float sv = sc.f32(st);
    if constexpr (SP) {
      acc[0] = fmaf(sv, pp[st][0], acc[0]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(sv, pp[st][j], acc[j]);
    }
  }
}

template <int WF, int NB, int KSPLIT, int MB, bool PF>
__global__ __launch_bounds__(256) void k_gateup_t(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su,
    const int32_t* __restrict__ tiles, int max_tiles, const int32_t* __restrict__ sorted_pair,
    int k, int H, int I, int P, uint16_t* __restrict__ h, int band, int xcd) {
  constexpr int RG = 4 / KSPLIT;
  // row blocks reduced per LDS pass: all of them for the low-bit 16-row
  // tiles (one barrier round, 32 KB at MB = 4; verify_int2 gate/up 21.8 ->
  // 21.2 us), two otherwise
  constexpr int RB = kRollLowBit<WF, NB>() ? MB : (MB < 2 ? MB : 2);
  __shared__ f32x4_t red[KSPLIT > 1 ? 4 : 1][RB][2][NB][64];
  int ti, sl;
  if (!tile_item(tiles[3 * max_tiles], I / (16 * MB * RG), band, xcd != 0, ti, sl)) return;
  const Tile tl = read_tile(tiles, ti);
  if (tl.rows <= 0) return;
  // wave index as a uniform value (the slab base below must live in SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const Dq dq = dq_consts<WF>();
  const int kp = wave % KSPLIT, rg = wave / KSPLIT;
  const int i0 = (sl * RG + rg) * 16 * MB;
  const int units = H / 128 / KSPLIT;
  const int ub = kp * units;
  const size_t nb0 = (static_cast<size_t>(tl.e) * I + i0) / 16;
  const Slab<WF> Sg(wg, sg, nb0, MB, H), Su(wu, su, nb0, MB, H);

  const uint16_t* px[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int rr = min(b * 16 + r, tl.rows - 1);
    int p = sorted_pair[tl.row0 + rr];
    p = min(max(p, 0), P - 1);
    px[b] = x + static_cast<size_t>(p / k) * H + q * 8;
  }

  f32x4_t acc[MB][2][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[mb][gu][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    TScales sc[MB][2];
    TRaw<WF> raw[MB][2];
    u32x4_t xa[4][NB];
  };
  auto load = [&](Stage& S, int u) {
    if constexpr (WF != WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        S.sc[mb][0] = tscales<WF, weight_aux<NB>()>(Sg, mb, u, r);
        S.sc[mb][1] = tscales<WF, weight_aux<NB>()>(Su, mb, u, r);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      S.raw[mb][0] = tload<WF, weight_aux<NB>()>(Sg, mb, u, lane);
      S.raw[mb][1] = tload<WF, weight_aux<NB>()>(Su, mb, u, lane);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int b = 0; b < NB; ++b) S.xa[st][b] = ld16(px[b] + 128 * u + 32 * st);
  };
  auto compute = [&](const Stage& S) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4_t corr[NB];
      if constexpr (WF != WF_BF16) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          corr[b] = mfma_bf16(S.xa[st][b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          const u32x4_t wv = tdecode<WF>(S.raw[mb][gu], st, dq);
          if constexpr (WF == WF_BF16) {
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[mb][gu][b] = mfma_bf16(S.xa[st][b], wv, acc[mb][gu][b]);
          } else {
            const float sv = S.sc[mb][gu].f32(st);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const f32x4_t pp = mfma_bf16(S.xa[st][b], wv, corr[b]);
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mb][gu][b][j] = fmaf(sv, pp[j], acc[mb][gu][b][j]);
            }
          }
        }
      }
    }
  };
  // low-bit tiles of at most 4 rows take the 4-row layout (acc_row)
  const bool spread = kRollLowBit<WF, NB>() && tl.rows <= 4;
  if constexpr (kRollLowBit<WF, NB>()) {
    // low-bit, one token block: the loads of a (row block, gate/up) pair
    // for unit u+1 are issued into its registers as soon as unit u is done
    // with them, and the token fragments of unit u+1 at the start of unit
    // u, so every load has one unit of multiplies to arrive in, without a
    // second register stage.  Per accumulator the additions run in the same
    // order as in compute() (chunk order within a unit, units in order).
    // SP: the 4-row layout, one scale FMA per product instead of four.
    // PS: int2 codes decoded in place against prescaled token fragments
    // (tdecode_int2_ps)
    constexpr bool PS = WF == WF_INT2;
    const DqPs dps = dq_ps_consts();
    auto rolled = [&](auto sp_tag) {
      constexpr bool SP = decltype(sp_tag)::value;
      const uint16_t* pxr;
      {
        const int rr = min(SP ? (r >> 2) : r, tl.rows - 1);
        int p = sorted_pair[tl.row0 + rr];
        p = min(max(p, 0), P - 1);
        pxr = x + static_cast<size_t>(p / k) * H + q * 8;
      }
      TScales sc[MB][2];
      TRaw<WF> raw[MB][2];
      u32x4_t xa[4], xn[4];
      auto load_pair = [&](int mb, int gu, int u) {
        const Slab<WF>& S = gu == 0 ? Sg : Su;
        sc[mb][gu] = tscales<WF, weight_aux<NB>()>(S, mb, u, r);
        raw[mb][gu] = tload<WF, weight_aux<NB>()>(S, mb, u, lane);
      };
      auto load_x = [&](u32x4_t (&xv)[4], int u) {
#pragma unroll
        for (int st = 0; st < 4; ++st) xv[st] = ld16(pxr + 128 * u + 32 * st);
      };
      // ROLL: the loads of unit u + 1 go out as unit u's registers free up
      auto unit = [&](int u, auto roll_tag) {
        constexpr bool ROLL = decltype(roll_tag)::value;
        if constexpr (ROLL) load_x(xn, u + 1);
        f32x4_t corr[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if constexpr (PS) {
            xa[st] = prescale_x_int2(xa[st]);
            corr[st] = mfma_bf16(xa[st], neg_offset_fragment_ps(), f32x4_t{0.f, 0.f, 0.f, 0.f});
          } else {
            corr[st] = mfma_bf16(xa[st], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
          }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int gu = 0; gu < 2; ++gu) {
            rolled_block_unit<WF, PS, SP>(raw[mb][gu], sc[mb][gu], xa, corr, dq, dps,
                                          acc[mb][gu][0]);
            SCHED_FENCE();   // pair by pair: each waits for its own loads only
            if constexpr (ROLL) {
              load_pair(mb, gu, u + 1);
              SCHED_FENCE();
            }
          }
        }
        if constexpr (ROLL) {
#pragma unroll
          for (int st = 0; st < 4; ++st) xa[st] = xn[st];
        }
      };
      // the token fragments first, as in the loop body: with the loads
      // issued in the same order on both paths into the loop, each pair
      // waits for its own loads only (given the other order here, the
      // compiler waits for every outstanding load at the top of each unit)
      load_x(xa, ub);
      SCHED_FENCE();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        load_pair(mb, 0, ub);
        load_pair(mb, 1, ub);
        SCHED_FENCE();
      }
      // the last unit is peeled off so that every load in the loop body is
      // unconditional (a load under a branch makes the compiler wait for all
      // outstanding loads where it needs any of them)
      for (int u = ub; u + 1 < ub + units; ++u) unit(u, std::true_type{});
      unit(ub + units - 1, std::false_type{});
    };
    if (spread) rolled(std::true_type{});
    else rolled(std::false_type{});
  } else {
    unit_loop<PF, Stage>(ub, ub + units, load, compute);
  }

  if constexpr (KSPLIT > 1) {
#pragma unroll
    for (int m0 = 0; m0 < MB; m0 += RB) {
      if (m0 > 0) __syncthreads();
#pragma unroll
      for (int mm = 0; mm < RB; ++mm)
#pragma unroll
        for (int gu = 0; gu < 2; ++gu)
#pragma unroll
          for (int b = 0; b < NB; ++b) red[wave][mm][gu][b][lane] = acc[m0 + mm][gu][b];
      __syncthreads();
      for (int idx = wave; idx < RG * RB * NB; idx += 4) {
        const int g_ = idx / (RB * NB), rem = idx % (RB * NB);
        const int mm = rem % RB, b = rem / RB;
        f32x4_t G = red[g_ * KSPLIT][mm][0][b][lane], U_ = red[g_ * KSPLIT][mm][1][b][lane];
#pragma unroll
        for (int w = 1; w < KSPLIT; ++w) {
          G += red[g_ * KSPLIT + w][mm][0][b][lane];
          U_ += red[g_ * KSPLIT + w][mm][1][b][lane];
        }
        const int i = (sl * RG + g_) * 16 * MB + (m0 + mm) * 16 + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = b * 16 + acc_row(spread, q, j);
          if (rr < tl.rows) h[static_cast<size_t>(tl.row0 + rr) * I + i] = f32_to_bf16(silu(G[j]) * U_[j]);
        }
      }
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int i = i0 + mb * 16 + r;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = b * 16 + acc_row(spread, q, j);
          if (rr < tl.rows)
            h[static_cast<size_t>(tl.row0 + rr) * I + i] =
                f32_to_bf16(silu(acc[mb][0][b][j]) * acc[mb][1][b][j]);
        }
    }
  }
}

// down on tiled weights: MB 16-row blocks of output features per wave,
// 64 MB per workgroup, full K = I.  1-D grid over (tile, slice) items, block 256.
// SH: the tile's intermediate rows [16 NB][I] are copied into LDS once (rows
// of 2 I + 16 bytes, dynamic LDS) and the four waves read their fragments
// there, instead of each wave gathering the same rows from L2 for every k
// unit.  PAIRY: row r of the tile is stored at y[sorted_pair[row0 + r]] (its
// pair slot) instead of y[row0 + r], so the combine reads a token's slots
// without the pair -> row indirection.
template <int WF, int NB, int MB, bool PF, bool SH, bool PAIRY>
__global__ __launch_bounds__(256) void k_down_t(const uint16_t* __restrict__ h,
                                                const uint8_t* __restrict__ wd,
                                                const uint16_t* __restrict__ sd,
                                                const int32_t* __restrict__ tiles, int max_tiles,
                                                int H, int I, uint16_t* __restrict__ y,
                                                int band, int xcd,
                                                const int32_t* __restrict__ sorted_pair, int P) {
  // the output tile goes through LDS when a wave owns 2+ row blocks (int4
  // stack step -1.2%); with one (bf16 decode) direct stores measured 0.3%
  // faster
  constexpr bool kStageOut = MB >= 2;
  __shared__ __align__(16) char ot[kStageOut ? out_tile_bytes<NB, MB>() : 16];
  extern __shared__ __align__(16) char hs[];   // SH: the intermediate rows
  int ti, sl;
  if (!tile_item(tiles[3 * max_tiles], H / (64 * MB), band, xcd != 0, ti, sl)) return;
  const Tile tl = read_tile(tiles, ti);
  if (tl.rows <= 0) return;
  // the output row of tile row rr
  auto out_row = [&](int rr) -> size_t {
    if constexpr (PAIRY) return static_cast<size_t>(min(max(sorted_pair[tl.row0 + rr], 0), P - 1));
    else return static_cast<size_t>(tl.row0 + rr);
  };
  // low-bit tiles of at most 4 rows with the rows in LDS take the 4-row
  // layout (acc_row)
  const bool spread = SH && kRollLowBit<WF, NB>() && tl.rows <= 4;
  size_t orow[NB][4];   // direct stores: the rows this lane writes (16 b + acc_row)
  // 4-row layout: the output row of lane quarter q (its component 0), read
  // now so that the direct stores at the end do not wait for it
  const size_t srow = spread ? out_row(min((static_cast<int>(threadIdx.x) & 63) >> 4, tl.rows - 1)) : 0;
  if constexpr (!kStageOut) {
    const int q4 = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        orow[b][j] = out_row(min(b * 16 + acc_row(spread, q4, j), tl.rows - 1));
  }
  const int hp = 2 * I + 16;   // SH: LDS row pitch in bytes (rows 16 bytes = 4 banks apart)
  // wave index as a uniform value (the slab base below must live in SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const Dq dq = dq_consts<WF>();
  const int n0 = (sl * 4 + wave) * 16 * MB;
  const size_t nb0 = (static_cast<size_t>(tl.e) * H + n0) / 16;
  const Slab<WF> Sd(wd, sd, nb0, MB, I);
  const uint16_t* ph[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    ph[b] = h + static_cast<size_t>(tl.row0 + min(b * 16 + r, tl.rows - 1)) * I + q * 8;

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    TScales sc[MB];
    TRaw<WF> raw[MB];
    u32x4_t ha[SH ? 1 : 4][NB];
    int u;
  };
  auto load = [&](Stage& S, int u) {
    if constexpr (WF != WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) S.sc[mb] = tscales<WF, weight_aux<NB>()>(Sd, mb, u, r);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) S.raw[mb] = tload<WF, weight_aux<NB>()>(Sd, mb, u, lane);
    if constexpr (!SH) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int b = 0; b < NB; ++b) S.ha[st][b] = ld16(ph[b] + 128 * u + 32 * st);
    }
    S.u = u;
  };
  auto hfrag = [&](const Stage& S, int st, int b) -> u32x4_t {
    if constexpr (SH)
      return *reinterpret_cast<const u32x4_t*>(hs + (b * 16 + r) * hp +
                                               (128 * S.u + 32 * st + 8 * q) * 2);
    else
      return S.ha[st][b];
  };
  auto compute = [&](const Stage& S) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      u32x4_t ha[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ha[b] = hfrag(S, st, b);
      f32x4_t corr[NB];
      if constexpr (WF != WF_BF16) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          corr[b] = mfma_bf16(ha[b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4_t wv = tdecode<WF>(S.raw[mb], st, dq);
        if constexpr (WF == WF_BF16) {
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[mb][b] = mfma_bf16(ha[b], wv, acc[mb][b]);
        } else {
          const float sv = S.sc[mb].f32(st);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t pp = mfma_bf16(ha[b], wv, corr[b]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mb][b][j] = fmaf(sv, pp[j], acc[mb][b][j]);
          }
        }
      }
    }
  };
  auto stage_h = [&]() {
    // 16-byte chunks; rows past the tile repeat its last row (never stored).
    // The 4-row layout reads rows 0 .. 3 only.
    // Up to 8 chunks per thread in flight: one round of loads for 16 rows at
    // I <= 1024.
    constexpr int SB = 8;
    const int cpr = I / 8, nch = (spread ? 4 : 16 * NB) * cpr;
    for (int c0 = threadIdx.x; c0 < nch; c0 += SB * 256) {
      u32x4_t v[SB];
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int c = c0 + i * 256;
        if (c < nch) {
          const int row = c / cpr, c8 = c - row * cpr;
          v[i] = ld16(h + static_cast<size_t>(tl.row0 + min(row, tl.rows - 1)) * I + c8 * 8);
        }
      }
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int c = c0 + i * 256;
        if (c < nch) {
          const int row = c / cpr, c8 = c - row * cpr;
          // int2 (rolled path): rows stored prescaled for tdecode_int2_ps
          // (a 16-byte chunk is one MFMA A fragment of a lane)
          if constexpr (WF == WF_INT2 && kRollLowBit<WF, NB>()) v[i] = prescale_x_int2(v[i]);
          *reinterpret_cast<u32x4_t*>(hs + row * hp + c8 * 16) = v[i];
        }
      }
    }
    __syncthreads();
  };
  if constexpr (SH && kRollLowBit<WF, NB>()) {
    // low-bit, one token block, rows in LDS: the loads of row block mb for
    // unit u+1 are issued into its registers as soon as unit u is done with
    // them (as in k_gateup_t), so every weight load has one unit of
    // multiplies to arrive in.  Per accumulator the additions run in the
    // order of compute() (chunk order within a unit, units in order).  SP:
    // the 4-row layout, one scale FMA per product instead of four.
    // PS: int2 codes decoded in place; the rows were prescaled when staged
    constexpr bool PS = WF == WF_INT2;
    const DqPs dps = dq_ps_consts();
    auto rolled = [&](auto sp_tag) {
      constexpr bool SP = decltype(sp_tag)::value;
      const int hrow = SP ? (r >> 2) : r;   // LDS rows past the tile repeat its last row
      TScales sc[MB];
      TRaw<WF> raw[MB];
      auto load_blk = [&](int mb, int u) {
        sc[mb] = tscales<WF, weight_aux<NB>()>(Sd, mb, u, r);
        raw[mb] = tload<WF, weight_aux<NB>()>(Sd, mb, u, lane);
      };
      auto unit = [&](int u, auto roll_tag) {
        constexpr bool ROLL = decltype(roll_tag)::value;
        u32x4_t ha[4];
        f32x4_t corr[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          ha[st] =
              *reinterpret_cast<const u32x4_t*>(hs + hrow * hp + (128 * u + 32 * st + 8 * q) * 2);
          if constexpr (PS)
            corr[st] = mfma_bf16(ha[st], neg_offset_fragment_ps(), f32x4_t{0.f, 0.f, 0.f, 0.f});
          else
            corr[st] = mfma_bf16(ha[st], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          rolled_block_unit<WF, PS, SP>(raw[mb], sc[mb], ha, corr, dq, dps, acc[mb][0]);
          SCHED_FENCE();   // block by block: each waits for its own loads only
          if constexpr (ROLL) {
            load_blk(mb, u + 1);
            SCHED_FENCE();
          }
        }
      };
      // the first unit's weights are in flight while the rows are staged;
      // issued block by block, in the loop body's order
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        load_blk(mb, 0);
        SCHED_FENCE();
      }
      stage_h();
      SCHED_FENCE();
      const int nu = I / 128;
      for (int u = 0; u + 1 < nu; ++u) unit(u, std::true_type{});
      unit(nu - 1, std::false_type{});
    };
    if (spread) rolled(std::true_type{});
    else rolled(std::false_type{});
  } else if constexpr (SH && !PF) {
    // the first unit's weights are in flight while the rows are staged
    Stage s0;
    load(s0, 0);
    stage_h();
    SCHED_FENCE();
    compute(s0);
    unit_loop<false, Stage>(1, I / 128, load, compute);
  } else {
    if constexpr (SH) stage_h();
    unit_loop<PF, Stage>(0, I / 128, load, compute);
  }
  if constexpr (kStageOut) {
    if (spread) {
      // at most 4 rows: direct 2-byte stores of component 0 (row q), no
      // round trip through LDS and its two barriers
      if (q < tl.rows) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) y[srow * H + n0 + mb * 16 + r] = f32_to_bf16(acc[mb][0][0]);
      }
    } else {
      store_tile_rows<NB, MB>(ot, [&](int mb, int b, int j) { return acc[mb][b][j]; }, tl.rows,
                              [&](int row, int col, u32x4_t v) {
                                *reinterpret_cast<u32x4_t*>(y + out_row(row) * H + col) = v;
                              },
                              sl * 64 * MB);
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int n = n0 + mb * 16 + r;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = b * 16 + acc_row(spread, q, j);
          if (rr < tl.rows) y[orow[b][j] * H + n] = f32_to_bf16(acc[mb][b][j]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Large batches: token rows staged through LDS.
//
// With 64- or 128-row token tiles every wave of a workgroup needs the same
// token fragments; loading them per wave makes the per-CU load path (not
// HBM) the limit.  Here the workgroup copies each 16 NB x 128 token unit into
// LDS once, with full 256-byte row segments per load, already in MFMA
// fragment order, and the waves read their A fragments from LDS; weights
// still stream from HBM straight into registers.  Two LDS buffers: the next
// unit is loaded into registers while the current one is multiplied, then
// stored.  After the k loop the same buffers stage the output tile.

// The k loop of the LDS-staged kernels.  Unit u multiplies the weights in
// registers with the token unit in LDS buffer u & 1, while the token unit
// u+1 travels through registers into the other buffer; one barrier per
// unit.  load(w, u, f) issues the loads of weight fragment group f (of NF)
// of unit u, compute(w, buf, f) consumes group f.  With ROLL, group f of
// unit u+1 is loaded into the same registers as soon as group f of unit u
// has been consumed, so the weight loads run a unit ahead at no register
// cost.  Without it a unit's loads are issued together and waited for
// before its multiplies (the other waves of the SIMD hide the latency).
// Unit 0 of the token rows is staged here, after the first weight loads.
template <bool ROLL, int NF, typename Stage, int NB, typename XU, typename Load, typename Compute>
__device__ __forceinline__ void staged_loop(int units, XU& xu, char (*xs)[NB * 4096], Load&& load,
                                            Compute&& compute) {
  if constexpr (!ROLL) {
    xu.load(0);
    xu.store(xs[0]);
    __syncthreads();
    for (int u = 0; u < units; ++u) {
      Stage w;
#pragma unroll
      for (int f = 0; f < NF; ++f) load(w, u, f);
      if (u + 1 < units) xu.load(u + 1);
      SCHED_FENCE();
#pragma unroll
      for (int f = 0; f < NF; ++f) compute(w, xs[u & 1], f);
      if (u + 1 < units) xu.store(xs[(u + 1) & 1]);
      __syncthreads();
    }
  } else {
    Stage w;
#pragma unroll
    for (int f = 0; f < NF; ++f) load(w, 0, f);
    xu.load(0);
    xu.store(xs[0]);
    __syncthreads();
    // the last unit is peeled off, so that every load of the loop body is
    // unconditional: a load under a branch makes the compiler wait for all
    // outstanding loads where it needs any of them
    for (int u = 0; u + 1 < units; ++u) {
      xu.load(u + 1);
      SCHED_FENCE();
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        compute(w, xs[u & 1], f);
        SCHED_FENCE();
        load(w, u + 1, f);
        SCHED_FENCE();
      }
      xu.store(xs[(u + 1) & 1]);
      __syncthreads();
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) compute(w, xs[(units - 1) & 1], f);
  }
}

// gate/up + SwiGLU, KSPLIT = 1: each wave owns MB 16-row blocks of gate and
// of up (64 MB rows per workgroup) over the full K = H.  1-D grid over
// (tile, slice) items, block 256.
template <int WF, int NB, int MB, int AUX, bool ROLL>
__device__ __forceinline__ void gateup_x_body(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su, const Tile tl, int sl,
    const int32_t* __restrict__ sorted_pair, int k, int H, int I, int P,
    uint16_t* __restrict__ h, char (*xs)[NB * 4096]) {
  // wave index as a uniform value (the slab base below must live in SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15;
  const Dq dq = dq_consts<WF>();
  const int i0 = (sl * 4 + wave) * 16 * MB;
  const int units = H / 128;
  const size_t nb0 = (static_cast<size_t>(tl.e) * I + i0) / 16;
  const Slab<WF> Sg(wg, sg, nb0, MB, H), Su(wu, su, nb0, MB, H);

  // token rows through a raw buffer: T * H < 2^31 elements (an ABI limit),
  // so the byte offsets fit 32 bits
  XUnitBuf<NB> xu;
  xu.init(x, static_cast<uint32_t>(static_cast<size_t>(P / k) * H * 2), [&](int R) {
    int p = sorted_pair[tl.row0 + min(R, tl.rows - 1)];
    p = min(max(p, 0), P - 1);
    return static_cast<size_t>(p / k) * H;
  });

  f32x4_t acc[MB][2][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int gu = 0; gu < 2; ++gu)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[mb][gu][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    TScales sc[MB][2];
    TRaw<WF> raw[MB][2];
  };
  // bf16: group f = fragment f (k chunk f) of every block; low-bit: one
  // group (a unit is one load per block)
  constexpr int NF = WF == WF_BF16 ? 4 : 1;
  staged_loop<ROLL, NF, Stage, NB>(units, xu, xs, [&](Stage& w, int u, int f) {
    if constexpr (WF == WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        w.raw[mb][0].v[f] = tload_frag<AUX>(Sg, mb, u, f, lane);
        w.raw[mb][1].v[f] = tload_frag<AUX>(Su, mb, u, f, lane);
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        w.sc[mb][0] = tscales<WF, AUX>(Sg, mb, u, r);
        w.sc[mb][1] = tscales<WF, AUX>(Su, mb, u, r);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        w.raw[mb][0] = tload<WF, AUX>(Sg, mb, u, lane);
        w.raw[mb][1] = tload<WF, AUX>(Su, mb, u, lane);
      }
    }
  }, [&](const Stage& w, const char* buf, int f) {
    if constexpr (WF == WF_BF16) {
      // k chunk f, token blocks outer: one token fragment is live at a time
      // (what lets 128-row tiles fit 256 VGPRs)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4_t xa = xfrag<NB>(buf, f, b, lane);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int gu = 0; gu < 2; ++gu)
            acc[mb][gu][b] = mfma_bf16(xa, w.raw[mb][gu].v[f], acc[mb][gu][b]);
      }
      return;
    }
    // low-bit: all four k chunks of the unit
    constexpr int NS = 4;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      u32x4_t xa[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) xa[b] = xfrag<NB>(buf, st, b, lane);
      f32x4_t corr[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        corr[b] = mfma_bf16(xa[b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
          const u32x4_t wv = tdecode<WF>(w.raw[mb][gu], st, dq);
          const float sv = w.sc[mb][gu].f32(st);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t pp = mfma_bf16(xa[b], wv, corr[b]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mb][gu][b][j] = fmaf(sv, pp[j], acc[mb][gu][b][j]);
          }
        }
      }
    }
  });

  static_assert(out_tile_bytes<NB, MB>() <= 2 * NB * 4096, "output tile exceeds the token buffers");
  store_tile<NB, MB>(
      xs[0], [&](int mb, int b, int j) { return silu(acc[mb][0][b][j]) * acc[mb][1][b][j]; },
      tl.rows, h + static_cast<size_t>(tl.row0) * I, I, sl * 64 * MB);
}

template <int WF, int NB, int MB, bool ROLL>
__global__ __launch_bounds__(256) void k_gateup_x(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ wg, const uint8_t* __restrict__ wu,
    const uint16_t* __restrict__ sg, const uint16_t* __restrict__ su,
    const int32_t* __restrict__ tiles, int max_tiles, const int32_t* __restrict__ sorted_pair,
    int k, int H, int I, int P, uint16_t* __restrict__ h, int band, int xcd) {
  __shared__ __align__(16) char xs[2][NB * 4096];
  int ti, sl;
  if (!tile_item(tiles[3 * max_tiles], I / (64 * MB), band, xcd != 0, ti, sl)) return;
  const Tile tl = read_tile(tiles, ti);
  if (tl.rows <= 0) return;
  if (single_tile(tiles, max_tiles, ti, tl.e))
    gateup_x_body<WF, NB, MB, kWeightAux, ROLL>(x, wg, wu, sg, su, tl, sl, sorted_pair, k, H, I,
                                                P, h, xs);
  else
    gateup_x_body<WF, NB, MB, 0, ROLL>(x, wg, wu, sg, su, tl, sl, sorted_pair, k, H, I, P, h, xs);
}

// down with the intermediate rows staged through LDS (same scheme, K = I).
template <int WF, int NB, int MB, int AUX, bool ROLL>
__device__ __forceinline__ void down_x_body(const uint16_t* __restrict__ h,
                                            const uint8_t* __restrict__ wd,
                                            const uint16_t* __restrict__ sd, const Tile tl, int sl,
                                            int H, int I, uint16_t* __restrict__ y,
                                            char (*xs)[NB * 4096]) {
  // wave index as a uniform value (the slab base below must live in SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15;
  const Dq dq = dq_consts<WF>();
  const int n0 = (sl * 4 + wave) * 16 * MB;
  const int units = I / 128;
  const size_t nb0 = (static_cast<size_t>(tl.e) * H + n0) / 16;
  const Slab<WF> Sd(wd, sd, nb0, MB, I);

  XUnit<NB> xu;
  xu.init(h, [&](int R) { return static_cast<size_t>(tl.row0 + min(R, tl.rows - 1)) * I; });

  f32x4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mb][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    TScales sc[MB];
    TRaw<WF> raw[MB];
  };
  constexpr int NF = WF == WF_BF16 ? 4 : 1;
  staged_loop<ROLL, NF, Stage, NB>(units, xu, xs, [&](Stage& w, int u, int f) {
    if constexpr (WF == WF_BF16) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) w.raw[mb].v[f] = tload_frag<AUX>(Sd, mb, u, f, lane);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) w.sc[mb] = tscales<WF, AUX>(Sd, mb, u, r);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) w.raw[mb] = tload<WF, AUX>(Sd, mb, u, lane);
    }
  }, [&](const Stage& w, const char* buf, int f) {
    constexpr int NS = WF == WF_BF16 ? 1 : 4;
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
      const int st = WF == WF_BF16 ? f : s4;
      u32x4_t ha[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) ha[b] = xfrag<NB>(buf, st, b, lane);
      f32x4_t corr[NB];
      if constexpr (WF != WF_BF16) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          corr[b] = mfma_bf16(ha[b], neg_offset_fragment<WF>(), f32x4_t{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const u32x4_t wv = tdecode<WF>(w.raw[mb], st, dq);
        if constexpr (WF == WF_BF16) {
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[mb][b] = mfma_bf16(ha[b], wv, acc[mb][b]);
        } else {
          const float sv = w.sc[mb].f32(st);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t pp = mfma_bf16(ha[b], wv, corr[b]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mb][b][j] = fmaf(sv, pp[j], acc[mb][b][j]);
          }
        }
      }
    }
  });
  static_assert(out_tile_bytes<NB, MB>() <= 2 * NB * 4096, "output tile exceeds the token buffers");
  store_tile<NB, MB>(
      xs[0], [&](int mb, int b, int j) { return acc[mb][b][j]; }, tl.rows,
      y + static_cast<size_t>(tl.row0) * H, H, sl * 64 * MB);
}

// float32 path (act and weights float32): one thread per output, float32
// fused multiply-adds in ascending k.  grid (max_tiles, ceil(N/16)),
template <int WF, int NB, int MB, bool ROLL>
__global__ __launch_bounds__(256) void k_down_x(const uint16_t* __restrict__ h,
                                                const uint8_t* __restrict__ wd,
                                                const uint16_t* __restrict__ sd,
                                                const int32_t* __restrict__ tiles, int max_tiles,
                                                int H, int I, uint16_t* __restrict__ y, int band,
                                                int xcd, int split) {
  __shared__ __align__(16) char xs[2][NB * 4096];
  int vt, sl;
  if (!tile_item(tiles[3 * max_tiles] * split, H / (64 * MB), band, xcd != 0, vt, sl)) return;
  // plan tiles taller than 16 NB rows are taken in `split` parts of 16 NB rows
  const int ti = vt / split, part = vt % split;
  Tile tl = read_tile(tiles, ti);
  // non-temporal weight loads only where this item is the expert's only one
  const bool single = single_tile(tiles, max_tiles, ti, tl.e) && tl.rows <= 16 * NB;
  tl.row0 += part * 16 * NB;
  tl.rows = min(tl.rows - part * 16 * NB, 16 * NB);
  if (tl.rows <= 0) return;
  if (single)
    down_x_body<WF, NB, MB, kWeightAux, ROLL>(h, wd, sd, tl, sl, H, I, y, xs);
  else
    down_x_body<WF, NB, MB, 0, ROLL>(h, wd, sd, tl, sl, H, I, y, xs);
}

// block 256 = 16 rows x 16 outputs.
__global__ __launch_bounds__(256) void k_gateup_f32(const float* __restrict__ x,
                                                    const float* __restrict__ wg,
                                                    const float* __restrict__ wu,
                                                    const int32_t* __restrict__ tiles, int max_tiles,
                                                    const int32_t* __restrict__ sorted_pair, int k,
                                                    int H, int I, int P, float* __restrict__ h) {
  const int n_tiles = tiles[3 * max_tiles];
  if (static_cast<int>(blockIdx.x) >= n_tiles) return;
  const Tile tl = read_tile(tiles, blockIdx.x);
  const int rr = threadIdx.x >> 4, i = blockIdx.y * 16 + (threadIdx.x & 15);
  if (rr >= tl.rows || i >= I) return;
  const int p = min(max(sorted_pair[tl.row0 + rr], 0), P - 1);
  const float* xp = x + static_cast<size_t>(p / k) * H;
  const float* gp = wg + (static_cast<size_t>(tl.e) * I + i) * H;
  const float* up = wu + (static_cast<size_t>(tl.e) * I + i) * H;
  float g = 0.f, u = 0.f;
  for (int c = 0; c < H; ++c) {
    g = fmaf(gp[c], xp[c], g);
    u = fmaf(up[c], xp[c], u);
  }
  h[static_cast<size_t>(tl.row0 + rr) * I + i] = silu(g) * u;
}

__global__ __launch_bounds__(256) void k_down_f32(const float* __restrict__ h,
                                                  const float* __restrict__ wd,
                                                  const int32_t* __restrict__ tiles, int max_tiles,
                                                  int H, int I, float* __restrict__ y) {
  const int n_tiles = tiles[3 * max_tiles];
  if (static_cast<int>(blockIdx.x) >= n_tiles) return;
  const Tile tl = read_tile(tiles, blockIdx.x);
  const int rr = threadIdx.x >> 4, n = blockIdx.y * 16 + (threadIdx.x & 15);
  if (rr >= tl.rows || n >= H) return;
  const float* hp = h + static_cast<size_t>(tl.row0 + rr) * I;
  const float* dp = wd + (static_cast<size_t>(tl.e) * H + n) * I;
  float acc = 0.f;
  for (int c = 0; c < I; ++c) acc = fmaf(dp[c], hp[c], acc);
  y[static_cast<size_t>(tl.row0 + rr) * H + n] = acc;
}

template <int WF, int NB>
static void launch_gateup_wf(const moe_shape& s, const Plan& pl, const void* x,
                             const moe_experts& ex, const int32_t* sorted_pair,
                             const int32_t* tiles, void* h, hipStream_t st) {
  const int P = s.T * s.top_k;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint16_t* hb = static_cast<uint16_t*>(h);
  const uint8_t* g8 = static_cast<const uint8_t*>(ex.gate);
  const uint8_t* u8 = static_cast<const uint8_t*>(ex.up);
  if (NB <= 2 || s.I % 128 != 0) {
    const dim3 grid(s.I / 32, pl.max_tiles);
    if ((s.H / 4) % 128 == 0)
      hipLaunchKernelGGL((k_gateup<WF, NB, 4, 4>), grid, dim3(256), 0, st, xb, g8, u8, ex.gate_scale,
                         ex.up_scale, tiles, pl.max_tiles, sorted_pair, s.top_k, s.H, s.I, P, hb);
    else
      hipLaunchKernelGGL((k_gateup<WF, NB, 4, 1>), grid, dim3(256), 0, st, xb, g8, u8, ex.gate_scale,
                         ex.up_scale, tiles, pl.max_tiles, sorted_pair, s.top_k, s.H, s.I, P, hb);
  } else {
    const dim3 grid(s.I / 128, pl.max_tiles);
    if (s.H % 128 == 0)
      hipLaunchKernelGGL((k_gateup<WF, NB, 1, 4>), grid, dim3(256), 0, st, xb, g8, u8, ex.gate_scale,
                         ex.up_scale, tiles, pl.max_tiles, sorted_pair, s.top_k, s.H, s.I, P, hb);
  }
}

template <int WF, int NB>
static void launch_down_wf(const moe_shape& s, const Plan& pl, const void* h,
                           const moe_experts& ex, const int32_t* tiles, void* y, hipStream_t st) {
  const dim3 grid(s.H / 128, pl.max_tiles);
  if (s.I % 128 == 0)
    hipLaunchKernelGGL((k_down<WF, NB, 4>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h),
                       static_cast<const uint8_t*>(ex.down), ex.down_scale, tiles, pl.max_tiles, s.H,
                       s.I, static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL((k_down<WF, NB, 1>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(h),
                       static_cast<const uint8_t*>(ex.down), ex.down_scale, tiles, pl.max_tiles, s.H,
                       s.I, static_cast<uint16_t*>(y));
}

// Rows per wave (16 MB) for the tiled kernels: bf16 keeps 32 rows (the raw
// fragments are 64 B per lane per row block); low-bit formats take 64 rows
// so that every token fragment feeds more MFMAs, except at 64-row token
// tiles: there gate/up takes 16 rows (of gate and of up) and down 32.
// Measured on MI355X: 128 rows (int2 at 16-row tiles) leaves too few waves
// to hide the dequant work (24 -> 28 us per 48-layer verify gate/up launch);
// the 32-row low-bit gate/up at 64-row tiles needed 256 VGPRs + 150 AGPRs
// (one wave per SIMD), the 16-row one fits 228 (two): 1074 -> 738 us (int4)
// and 954 -> 633 us (int2) per gate/up launch at 4096 tokens; down at 16
// rows was slower (its 32-row form already runs two waves per SIMD).
template <int WF, int NB, bool GATEUP>
constexpr int tiled_mb_max() {
  return WF == WF_BF16 ? 2 : (NB >= 4 ? (GATEUP ? 1 : 2) : 4);
}

// bf16 with 16-row tiles (decode): one 16-row block per wave (of gate and
// of up, or of down) with the next k unit's loads issued before the current
// one is multiplied (unit_loop with PF).  Measured on the MI355X at 8 tokens:
// gate/up 77 us against 80 us for two blocks per wave without it (78 us with
// one block alone), the whole step 0.7% faster again with down done the same
// way; the low-bit formats and taller tiles measured slower with it (the
// second register stage halves their occupancy).
template <int WF, int NB>
constexpr bool tile_pf() {
  return WF == WF_BF16 && NB == 1;
}
// LDS-staged kernels: bf16 gate/up issues each weight fragment group a unit
// ahead (staged_loop with ROLL).  Measured on the MI355X at 64-row tiles:
// gate/up 800 -> 769 us at 4096 tokens and 2640 -> 2510 us at 32768;
// down (5 k units) was 9 / 30 us slower with it, the low-bit formats have one
// load per block and unit and nothing to roll.
template <int WF, bool GATEUP>
constexpr bool x_roll() {
  return WF == WF_BF16 && GATEUP;
}
template <int WF, int NB, bool GATEUP>
constexpr int tile_mb_max() {
  return tile_pf<WF, NB>() ? 1 : tiled_mb_max<WF, NB, GATEUP>();
}

// largest MB <= mmax whose workgroup rows (rows_per_mb1 * MB) divide N
template <int WF, int NB>
static int tiled_mb(int N, int rows_per_mb1, int mmax) {
  for (int mb = mmax; mb >= 1; mb >>= 1)
    if (N % (rows_per_mb1 * mb) == 0) return mb;
  return 1;
}

struct TileOrder {
  int band, xcd;
};

// Item order of the tiled FFN grids.  Small batches have about one tile per
// expert and keep the plain order (the slices of one tile adjacent).  Large
// batches give hot experts many tiles: gate/up then walks all tiles of one
// slice on one XCD so the slice is read into its L2 once (measured: 6.4 ->
// 4.0 GB of L2 fills at 4096 tokens); down measured best in plain order.
static TileOrder tile_order(const Plan& pl, bool gateup) {
  if (gateup && pl.nb >= 4) return TileOrder{pl.max_tiles, 1};
  return TileOrder{1, 0};
}

// 1-D grid over (tile, slice) items, rounded up to a multiple of 8
static dim3 item_grid(const Plan& pl, int nslices) {
  const int64_t n = static_cast<int64_t>(pl.max_tiles) * nslices;
  return dim3(static_cast<unsigned>((n + 7) / 8 * 8));
}

template <int WF, int NB, int KSPLIT, int MB>
static void gateup_tiled_launch(const moe_shape& s, const Plan& pl, const void* x,
                                const moe_experts& ex, const int32_t* sorted_pair,
                                const int32_t* tiles, void* h, hipStream_t st) {
  const int nslices = s.I / (16 * MB * (4 / KSPLIT));
  const TileOrder o = tile_order(pl, true);
  if constexpr (KSPLIT == 1 && NB >= 4) {
    // large batches: token tile staged through LDS once per workgroup
    hipLaunchKernelGGL((k_gateup_x<WF, NB, MB, x_roll<WF, true>()>), item_grid(pl, nslices), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(ex.gate),
                       static_cast<const uint8_t*>(ex.up), ex.gate_scale, ex.up_scale, tiles,
                       pl.max_tiles, sorted_pair, s.top_k, s.H, s.I, s.T * s.top_k,
                       static_cast<uint16_t*>(h), min(o.band, pl.max_tiles), o.xcd);
  } else {
    hipLaunchKernelGGL((k_gateup_t<WF, NB, KSPLIT, MB, tile_pf<WF, NB>()>), item_grid(pl, nslices),
                       dim3(256), 0, st, static_cast<const uint16_t*>(x),
                       static_cast<const uint8_t*>(ex.gate), static_cast<const uint8_t*>(ex.up),
                       ex.gate_scale, ex.up_scale, tiles, pl.max_tiles, sorted_pair, s.top_k, s.H,
                       s.I, s.T * s.top_k, static_cast<uint16_t*>(h), min(o.band, pl.max_tiles),
                       o.xcd);
  }
}

template <int WF, int NB, int KSPLIT>
static void gateup_tiled_mb(const moe_shape& s, const Plan& pl, const void* x,
                            const moe_experts& ex, const int32_t* sp, const int32_t* tiles,
                            void* h, hipStream_t st) {
  constexpr int M = tile_mb_max<WF, NB, true>();
  switch (tiled_mb<WF, NB>(s.I, 16 * (4 / KSPLIT), M)) {
    case M: gateup_tiled_launch<WF, NB, KSPLIT, M>(s, pl, x, ex, sp, tiles, h, st); break;
    case (M > 1 ? M / 2 : 0):
      gateup_tiled_launch<WF, NB, KSPLIT, (M > 1 ? M / 2 : 1)>(s, pl, x, ex, sp, tiles, h, st); break;
    default: gateup_tiled_launch<WF, NB, KSPLIT, 1>(s, pl, x, ex, sp, tiles, h, st); break;
  }
}

template <int WF, int NB>
static void launch_gateup_tiled(const moe_shape& s, const Plan& pl, const void* x,
                                const moe_experts& ex, const int32_t* sorted_pair,
                                const int32_t* tiles, void* h, hipStream_t st) {
  // k split across the waves of a workgroup: 4 parts for small batches when
  // H allows (more workgroups stream at once), fewer otherwise
  const int ksplit = (NB <= 2 && s.H % 512 == 0) ? 4 : ((NB <= 2 && s.H % 256 == 0) ? 2 : 1);
  if (ksplit == 4) gateup_tiled_mb<WF, NB, 4>(s, pl, x, ex, sorted_pair, tiles, h, st);
  else if (ksplit == 2) gateup_tiled_mb<WF, NB, 2>(s, pl, x, ex, sorted_pair, tiles, h, st);
  else gateup_tiled_mb<WF, NB, 1>(s, pl, x, ex, sorted_pair, tiles, h, st);
}

template <int WF>
static void gateup_nb(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                      const int32_t* sp, const int32_t* tiles, void* h, hipStream_t st) {
  if constexpr (WF == WF_BF16) {
    if (pl.nb == 8) {   // bf16 tiled only (plan_nb)
      launch_gateup_tiled<WF, 8>(s, pl, x, ex, sp, tiles, h, st);
      return;
    }
  }
  if (s.flags & MOE_F_TILED_WEIGHTS) {
    switch (pl.nb) {
      case 1: launch_gateup_tiled<WF, 1>(s, pl, x, ex, sp, tiles, h, st); break;
      case 2: launch_gateup_tiled<WF, 2>(s, pl, x, ex, sp, tiles, h, st); break;
      default: launch_gateup_tiled<WF, 4>(s, pl, x, ex, sp, tiles, h, st); break;
    }
    return;
  }
  switch (pl.nb) {
    case 1: launch_gateup_wf<WF, 1>(s, pl, x, ex, sp, tiles, h, st); break;
    case 2: launch_gateup_wf<WF, 2>(s, pl, x, ex, sp, tiles, h, st); break;
    default: launch_gateup_wf<WF, 4>(s, pl, x, ex, sp, tiles, h, st); break;
  }
}

template <int WF, int NB, int MB>
static void down_tiled_launch(const moe_shape& s, const Plan& pl, const void* h,
                              const moe_experts& ex, const int32_t* tiles, void* y,
                              const int32_t* pairy, hipStream_t st) {
  const TileOrder o = tile_order(pl, false);
  if constexpr (NB >= 4) {
    // 128-row plan tiles run as two 64-row halves (measured: the 128-row down
    // kernel, 188 VGPRs, was slower than two 64-row items)
    const int split = pl.nb / NB;
    const int64_t n = static_cast<int64_t>(pl.max_tiles) * split * (s.H / (64 * MB));
    hipLaunchKernelGGL((k_down_x<WF, NB, MB, x_roll<WF, false>()>),
                       dim3(static_cast<unsigned>((n + 7) / 8 * 8)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(h), static_cast<const uint8_t*>(ex.down),
                       ex.down_scale, tiles, pl.max_tiles, s.H, s.I, static_cast<uint16_t*>(y),
                       min(o.band, pl.max_tiles * split), o.xcd, split);
  } else {
    // low-bit single-block tiles stage their intermediate rows in LDS
    const size_t lds = static_cast<size_t>(16 * NB) * (2 * s.I + 16);
    const bool sh = WF != WF_BF16 && NB == 1 && lds <= 64 * 1024;
    auto kern = pairy ? (sh ? k_down_t<WF, NB, MB, tile_pf<WF, NB>(), true, true>
                            : k_down_t<WF, NB, MB, tile_pf<WF, NB>(), false, true>)
                      : (sh ? k_down_t<WF, NB, MB, tile_pf<WF, NB>(), true, false>
                            : k_down_t<WF, NB, MB, tile_pf<WF, NB>(), false, false>);
    hipLaunchKernelGGL(kern, item_grid(pl, s.H / (64 * MB)), dim3(256), sh ? lds : 0, st,
                       static_cast<const uint16_t*>(h), static_cast<const uint8_t*>(ex.down),
                       ex.down_scale, tiles, pl.max_tiles, s.H, s.I, static_cast<uint16_t*>(y),
                       min(o.band, pl.max_tiles), o.xcd, pairy, s.T * s.top_k);
  }
}

template <int WF, int NB>
static void launch_down_tiled(const moe_shape& s, const Plan& pl, const void* h,
                              const moe_experts& ex, const int32_t* tiles, void* y,
                              const int32_t* pairy, hipStream_t st) {
  constexpr int M = tile_mb_max<WF, NB, false>();
  switch (tiled_mb<WF, NB>(s.H, 64, M)) {
    case M: down_tiled_launch<WF, NB, M>(s, pl, h, ex, tiles, y, pairy, st); break;
    case (M > 1 ? M / 2 : 0):
      down_tiled_launch<WF, NB, (M > 1 ? M / 2 : 1)>(s, pl, h, ex, tiles, y, pairy, st); break;
    default: down_tiled_launch<WF, NB, 1>(s, pl, h, ex, tiles, y, pairy, st); break;
  }
}

template <int WF>
static void down_nb(const moe_shape& s, const Plan& pl, const void* h, const moe_experts& ex,
                    const int32_t* tiles, void* y, hipStream_t st, const int32_t* pairy = nullptr) {
  if constexpr (WF == WF_BF16) {
    if (pl.nb == 8) {   // bf16 tiled only (plan_nb): 64-row halves of the 128-row tiles
      launch_down_tiled<WF, 4>(s, pl, h, ex, tiles, y, nullptr, st);
      return;
    }
  }
  if (s.flags & MOE_F_TILED_WEIGHTS) {
    switch (pl.nb) {
      case 1: launch_down_tiled<WF, 1>(s, pl, h, ex, tiles, y, pairy, st); break;
      case 2: launch_down_tiled<WF, 2>(s, pl, h, ex, tiles, y, nullptr, st); break;
      default: launch_down_tiled<WF, 4>(s, pl, h, ex, tiles, y, nullptr, st); break;
    }
    return;
  }
  switch (pl.nb) {
    case 1: launch_down_wf<WF, 1>(s, pl, h, ex, tiles, y, st); break;
    case 2: launch_down_wf<WF, 2>(s, pl, h, ex, tiles, y, st); break;
    default: launch_down_wf<WF, 4>(s, pl, h, ex, tiles, y, st); break;
  }
}

hipError_t launch_gateup(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                         const int32_t* sorted_pair, const int32_t* tiles, void* h,
                         hipStream_t st) {
  if (s.act == MOE_DT_F32) {
    const int P = s.T * s.top_k;
    hipLaunchKernelGGL(k_gateup_f32, dim3(pl.max_tiles, (s.I + 15) / 16), dim3(256), 0, st,
                       static_cast<const float*>(x), static_cast<const float*>(ex.gate),
                       static_cast<const float*>(ex.up), tiles, pl.max_tiles, sorted_pair, s.top_k,
                       s.H, s.I, P, static_cast<float*>(h));
  } else if (s.wfmt == MOE_WF_DENSE) {
    gateup_nb<WF_BF16>(s, pl, x, ex, sorted_pair, tiles, h, st);
  } else if (s.wfmt == MOE_WF_INT4_G32) {
    gateup_nb<WF_INT4>(s, pl, x, ex, sorted_pair, tiles, h, st);
  } else {
    gateup_nb<WF_INT2>(s, pl, x, ex, sorted_pair, tiles, h, st);
  }
  return hipGetLastError();
}

hipError_t launch_down(const moe_shape& s, const Plan& pl, const void* h, const moe_experts& ex,
                       const int32_t* tiles, void* y, hipStream_t st) {
  if (s.act == MOE_DT_F32) {
    hipLaunchKernelGGL(k_down_f32, dim3(pl.max_tiles, (s.H + 15) / 16), dim3(256), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(ex.down), tiles,
                       pl.max_tiles, s.H, s.I, static_cast<float*>(y));
  } else if (s.wfmt == MOE_WF_DENSE) {
    down_nb<WF_BF16>(s, pl, h, ex, tiles, y, st);
  } else if (s.wfmt == MOE_WF_INT4_G32) {
    down_nb<WF_INT4>(s, pl, h, ex, tiles, y, st);
  } else {
    down_nb<WF_INT2>(s, pl, h, ex, tiles, y, st);
  }
  return hipGetLastError();
}

// Down followed by the combine.  With 16-row tiles of tiled bf16-activation
// weights the down kernel writes each y row to its pair slot and the
// combine reads a token's k slots directly (one memory round trip instead
// of two); otherwise y in permuted row order and the combine through
// pair_row.
bool down_pair_order(const moe_shape& s, const Plan& pl) {
  return s.act == MOE_DT_BF16 && (s.flags & MOE_F_TILED_WEIGHTS) && pl.nb == 1;
}

hipError_t launch_down_combine(const moe_shape& s, const Plan& pl, const void* h,
                               const moe_experts& ex, const int32_t* tiles,
                               const int32_t* sorted_pair, const int32_t* pair_row, const float* w,
                               const void* residual, void* out, void* y, hipStream_t st) {
  if (!down_pair_order(s, pl)) {
    hipError_t e = launch_down(s, pl, h, ex, tiles, y, st);
    if (e == hipSuccess) e = launch_combine(s, y, pair_row, w, residual, out, st);
    return e;
  }
  if (s.wfmt == MOE_WF_DENSE) down_nb<WF_BF16>(s, pl, h, ex, tiles, y, st, sorted_pair);
  else if (s.wfmt == MOE_WF_INT4_G32) down_nb<WF_INT4>(s, pl, h, ex, tiles, y, st, sorted_pair);
  else down_nb<WF_INT2>(s, pl, h, ex, tiles, y, st, sorted_pair);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_combine(s, y, nullptr, w, residual, out, st);
  return e;
}

hipError_t launch_ffn(const moe_shape& s, const Plan& pl, const void* x, const moe_experts& ex,
                      const int32_t* sorted_pair, const int32_t* tiles, void* h, void* y,
                      hipStream_t st) {
  hipError_t e = launch_gateup(s, pl, x, ex, sorted_pair, tiles, h, st);
  if (e == hipSuccess) e = launch_down(s, pl, h, ex, tiles, y, st);
  return e;
}

}  // namespace moe
