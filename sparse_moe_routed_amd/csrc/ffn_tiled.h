// Device pieces shared by the grouped-FFN kernels on tiled expert weights:
// the weight-format tags, the tile plan record and work-item mapping, and the
// raw-buffer slab readers and decoders of the tiled layout.
#pragma once

#include "moe_device.h"

namespace moe {

enum { WF_BF16 = 0, WF_INT4 = 1, WF_INT2 = 2 };

template <int WF>
__device__ __forceinline__ size_t row_bytes(int K) {
  return WF == WF_BF16 ? static_cast<size_t>(K) * 2 : (WF == WF_INT4 ? K / 2 : K / 4);
}

// fp16 scales of groups g .. g+U-1 of one weight row (U = 1 or 4; 4 requires
// g % 4 == 0, so the 8-byte load is aligned).
template <int U>
struct Scales {
  uint16_t s[U];
};

struct Tile {
  int e, row0, rows;
};

// Keeps the compiler from interleaving a k unit's loads with its MFMAs: left
// alone it reuses a few registers for successive loads and waits on each, so
// one unit pays the memory latency several times over.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// The k loop over units u0 .. u1-1 of one wave: load(stage, u) issues a
// unit's loads, compute(stage) consumes them.  With PF the loads of unit
// u+1 are issued before unit u is multiplied (two register stages), so a
// wave always has one unit in flight; without it, load and compute
// alternate and the other waves of the SIMD hide the latency.
template <bool PF, typename Stage, typename Load, typename Compute>
__device__ __forceinline__ void unit_loop(int u0, int u1, Load&& load, Compute&& compute) {
  if constexpr (!PF) {
    for (int u = u0; u < u1; ++u) {
      Stage s;
      load(s, u);
      SCHED_FENCE();
      compute(s);
    }
  } else {
    Stage a, b;
    load(a, u0);
    int u = u0;
    for (; u + 1 < u1; u += 2) {
      load(b, u + 1);
      SCHED_FENCE();
      compute(a);
      SCHED_FENCE();
      if (u + 2 < u1) load(a, u + 2);
      SCHED_FENCE();
      compute(b);
      SCHED_FENCE();
    }
    if (u < u1) compute(a);
  }
}

__device__ __forceinline__ Tile read_tile(const int32_t* tiles, int t) {
  return Tile{tiles[3 * t], tiles[3 * t + 1], tiles[3 * t + 2]};
}

// Work item (tile, weight slice) of a 1-D tiled-FFN grid whose size is a
// multiple of 8.  Items are numbered in bands of `band` tiles, slice-major
// inside a band, so neighbouring items read the same weight slice of one
// expert for consecutive token tiles.  With `xcd` set, each run of
// neighbouring items goes to workgroups of a single XCD (workgroups are
// handed to the 8 XCDs round-robin by linear id), so the slice that the
// tiles of a hot expert share is fetched into that XCD's L2 once.
__device__ __forceinline__ bool tile_item(int n_tiles, int nslices, int band, bool xcd, int& tile,
                                          int& slice) {
  const int n = n_tiles * nslices;
  int L = static_cast<int>(blockIdx.x);
  if (xcd) {
    const int per = (n + 7) >> 3;
    const int j = L >> 3;
    if (j >= per) return false;
    L = (L & 7) * per + j;
  }
  if (L >= n) return false;
  const int b0 = L / (band * nslices) * band;
  const int nt = min(band, n_tiles - b0);
  const int idx = L - b0 * nslices;
  slice = idx / nt;
  tile = b0 + idx % nt;
  return true;
}

// The weight cache policy per tile: an expert with a single tile reads its
// records once in this call, so they stream non-temporal like the small-tile
// kernels' loads; the tiles of experts with several tiles keep the default
// policy, so their shared slices stay in L2 for the neighbouring items.
__device__ __forceinline__ bool single_tile(const int32_t* __restrict__ tiles, int max_tiles, int ti,
                                            int e) {
  const int n = tiles[3 * max_tiles];
  return (ti == 0 || tiles[3 * (ti - 1)] != e) && (ti + 1 >= n || tiles[3 * (ti + 1)] != e);
}

// The 4-row layout of a 16-row token block holding at most 4 rows (low-bit
// kernels): token t feeds the MFMA's A rows 4t .. 4t+3, so output component
// 0 of lane quarter q is token q and each product needs one scale FMA
// instead of four (in the 16-row layout A row r is token r and all four
// components of a lane are distinct rows).  The tile row that accumulator
// component j of lane quarter q belongs to, in either layout:
__device__ __forceinline__ int acc_row(bool spread, int q, int j) {
  return spread ? 4 * j + q : 4 * q + j;
}

// The bf16 output tile of a 256-thread item -- rows 0 .. 16 NB - 1 of the
// tile, columns col0 .. col0 + 64 MB - 1 -- written through LDS: value(mb, b,
// j) of lane (r, q) in wave w is row 16 b + 4 q + j, column 16 (MB w + mb) +
// r, so direct stores would be 2-byte scatters (4 MB NB per lane); staged,
// each thread stores 16 contiguous bytes.  `lds` holds out_tile_bytes<NB,
// MB>() bytes that no wave still reads.
template <int NB, int MB>
constexpr int out_tile_bytes() {
  return 16 * NB * (128 * MB + 16);
}
// With a store functor: store(row, col, v) writes the 16 bytes v of tile row
// `row` at column `col` (8 values) wherever the caller keeps them.
template <int NB, int MB, typename Val, typename Store>
__device__ __forceinline__ void store_tile_rows(char* lds, Val&& val, int rows, Store store,
                                                int col0) {
  constexpr int pitch = 128 * MB + 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  __syncthreads();   // every wave is done with the buffer
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint16_t*>(lds + (16 * b + 4 * q + j) * pitch +
                                     (16 * (MB * wave + mb) + r) * 2) = f32_to_bf16(val(mb, b, j));
  __syncthreads();
  constexpr int segs = 8 * MB;          // 16-byte segments per row
  constexpr int total = 16 * NB * segs;  // segments in the tile (128 at NB = MB = 1)
#pragma unroll
  for (int it = 0; it < (total + 255) / 256; ++it) {
    const int g = it * 256 + static_cast<int>(threadIdx.x);
    const int row = g / segs, cs = g % segs;
    if (g < total && row < rows)
      store(row, col0 + cs * 8, *reinterpret_cast<const u32x4_t*>(lds + row * pitch + cs * 16));
  }
}

template <int NB, int MB, typename Val>
__device__ __forceinline__ void store_tile(char* lds, Val&& val, int rows,
                                           uint16_t* __restrict__ dst, size_t ld, int col0) {
  store_tile_rows<NB, MB>(
      lds, val, rows,
      [&](int row, int col, u32x4_t v) {
        *reinterpret_cast<u32x4_t*>(dst + static_cast<size_t>(row) * ld + col) = v;
      },
      col0);
}

// ---------------------------------------------------------------------------
// Tiled weights (MOE_F_TILED_WEIGHTS).  The unit of the k loop is 128 k = 4
// MFMA chunks; for one 16-row block a lane fetches, per unit, 4 x 16 B (bf16:
// four consecutive 1 KB fragments), 16 B (int4) or 8 B (int2), plus 8 B of
// scales, so every load instruction of a wave reads one contiguous block.
// ---------------------------------------------------------------------------
// Raw weight bits of one 16-row block and k unit held by a lane: bf16 four
// 16-byte fragments, int4 16 bytes, int2 8 bytes.
template <int WF>
struct TRaw {
  u32x4_t v[4];
};
template <>
struct TRaw<WF_INT4> {
  u32x4_t v[1];
};
template <>
struct TRaw<WF_INT2> {
  u32x2_t v[1];
};

// The four fp16 group scales (k chunks 0..3 of a unit) of one weight row,
// kept packed in two registers.
struct TScales {
  u32x2_t v;
  __device__ __forceinline__ float f32(int st) const {
    return fp16_to_f32(static_cast<uint16_t>(v[st >> 1] >> (16 * (st & 1))));
  }
};

// Cache policy of the weight loads (the aux operand of the raw buffer loads).
// With tiles of 16 or 32 token rows an expert record streams through about
// once per call, so it is read non-temporal (bit 1 -> `nt` on gfx950): a
// streaming read of 4 GiB measured 7.0 TB/s with `nt` against 6.2 TB/s
// without, and the decode FFN gained 6%.  With 64-row tiles (large batches)
// hot experts' slices are read again by their other tiles from L2; `nt` on
// every tile there cost 12% (4096 tokens) to 31% (32768 tokens), so the
// large-batch kernels choose per tile: `nt` only for an expert with a single
// tile (single_tile in the FFN kernels; +2.6% at 4096 tokens).
constexpr int kWeightAux = 2;
template <int NB>
constexpr int weight_aux() {
  return NB >= 4 ? 0 : kWeightAux;
}

// Raw-buffer resource word 3 for gfx9 untyped dword access.
constexpr int kRawBufferWord3 = 0x00020000;

// The row blocks nb0 .. nb0+nblk-1 of one tiled matrix (and of its scales)
// that a workgroup reads, addressed as raw buffers: the base sits in SGPRs,
// a lane supplies one 32-bit offset and each load adds a uniform offset, so
// no 64-bit per-lane address is kept per load.  Loads beyond the slab
// return 0.
template <int WF>
struct Slab {
  __amdgpu_buffer_rsrc_t w, s;
  int K;
  __device__ __forceinline__ Slab(const uint8_t* mat, const uint16_t* sc, size_t nb0, int nblk,
                                  int K_)
      : K(K_) {
    const size_t blk = 16 * row_bytes<WF>(K_);
    w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(mat + nb0 * blk), 0,
                                          static_cast<int>(nblk * blk), kRawBufferWord3);
    if constexpr (WF != WF_BF16) {
      const size_t sblk = static_cast<size_t>(K_ / 128) * 128;   // bytes of scales per block
      s = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(sc) + nb0 * sblk), 0,
          static_cast<int>(nblk * sblk), kRawBufferWord3);
    }
  }
};

// Row block mb of the slab, k unit kb.
template <int WF, int AUX>
__device__ __forceinline__ TRaw<WF> tload(const Slab<WF>& S, int mb, int kb, int lane) {
  TRaw<WF> t;
  if constexpr (WF == WF_BF16) {
    const int soff = (mb * (S.K / 32) + 4 * kb) * 1024;
#pragma unroll
    for (int f = 0; f < 4; ++f)
      t.v[f] = __builtin_amdgcn_raw_buffer_load_b128(S.w, lane * 16 + f * 1024, soff, AUX);
  } else if constexpr (WF == WF_INT4) {
    t.v[0] = __builtin_amdgcn_raw_buffer_load_b128(S.w, lane * 16, (mb * (S.K / 128) + kb) * 1024,
                                                   AUX);
  } else {
    t.v[0] =
        __builtin_amdgcn_raw_buffer_load_b64(S.w, lane * 8, (mb * (S.K / 128) + kb) * 512, AUX);
  }
  return t;
}

// bf16: fragment f (k chunk f) of row block mb, k unit kb.
template <int AUX>
__device__ __forceinline__ u32x4_t tload_frag(const Slab<WF_BF16>& S, int mb, int kb, int f,
                                              int lane) {
  return __builtin_amdgcn_raw_buffer_load_b128(S.w, lane * 16 + f * 1024,
                                               (mb * (S.K / 32) + 4 * kb) * 1024, AUX);
}

template <int WF>
__device__ __forceinline__ Dq dq_consts() {
  if constexpr (WF == WF_BF16) return Dq{0u, 0u};   // unused
  else return Dq{in_vgpr(WF == WF_INT4 ? 0x000F000Fu : 0x00030003u), in_vgpr(0x43004300u)};
}

template <int WF>
__device__ __forceinline__ u32x4_t tdecode(const TRaw<WF>& t, int s, Dq d) {
  if constexpr (WF == WF_BF16) {
    return t.v[s];
  } else if constexpr (WF == WF_INT4) {
    return dequant_int4_tiled(t.v[0][s], d);
  } else {
    const uint32_t w = t.v[0][s >> 1];
    return (s & 1) ? dequant_int2_tiled<1>(w, d) : dequant_int2_tiled<0>(w, d);
  }
}

// fp16 scales of groups 4 kb .. 4 kb + 3 of row r of block mb.
template <int WF, int AUX>
__device__ __forceinline__ TScales tscales(const Slab<WF>& S, int mb, int kb, int r) {
  return TScales{
      __builtin_amdgcn_raw_buffer_load_b64(S.s, r * 8, (mb * (S.K / 128) + kb) * 128, AUX)};
}

// Prescaled int2 decode (the rolled 16-row-tile kernels).  Dword m of a
// chunk's B fragment holds stored codes 2m and 2m+1 (low and high bf16
// half).  For m = 0, 1, 2 the code is masked where it lies in the byte of
// its chunk (bits 2m of each half) instead of being shifted down, which
// gives the exact bf16 value 128 + 4^m c (c = stored code); dword 3 is
// shifted as before (128 + c).  Token dword m of the A fragment is divided
// by 4^m beforehand (prescale_x_int2), so each product x 4^-m (128 + 4^m c)
// = 128 x 4^-m + x c still carries the code once, and the correction
// fragment (neg_offset_fragment_ps) holds -(128 + 4^m 2) per dword, making
// the sum exactly x (c - 2) per term up to the MFMA's float32 rounding.
// Five VALU per chunk of 8 codes instead of seven (sub-chunk 0), six
// instead of eight (sub-chunk 1).
struct DqPs {
  uint32_t m0, m1, m2, magic;
};
__device__ __forceinline__ DqPs dq_ps_consts() {
  return DqPs{in_vgpr(0x00030003u), in_vgpr(0x000C000Cu), in_vgpr(0x00300030u),
              in_vgpr(0x43004300u)};
}
__device__ __forceinline__ u32x4_t tdecode_int2_ps(const TRaw<WF_INT2>& t, int s, DqPs d) {
  const uint32_t w = t.v[0][s >> 1];
  const uint32_t ws = (s & 1) ? (w >> 8) : w;
  u32x4_t r;
  r[0] = (ws & d.m0) | d.magic;
  r[1] = (ws & d.m1) | d.magic;
  r[2] = (ws & d.m2) | d.magic;
  r[3] = ((w >> ((s & 1) ? 14 : 6)) & d.m0) | d.magic;
  return r;
}
__device__ __forceinline__ u32x4_t neg_offset_fragment_ps() {
  // bf16 pairs (-130), (-136), (-160), (-130)
  return u32x4_t{kNegOffset2, 0xC308C308u, 0xC320C320u, kNegOffset2};
}
// Both bf16 halves of w divided by 2^(2 e) (e = 1 or 2): the exponent field
// lowered by 2 e with a saturating 16-bit subtraction on the magnitude, the
// sign kept.  Exact for |x| >= 2^-122; zeros stay zero, smaller magnitudes
// flush towards zero.  An infinity or NaN becomes a finite value of
// magnitude >= 2^124; its products with the decoded codes (>= 128) and with
// the correction fragment overflow float32 with opposite signs, so a
// non-finite token still makes the MFMA result NaN.
__device__ __forceinline__ uint32_t bf16x2_div_pow4(uint32_t w, uint16_t exp_step) {
  typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
  const u16x2_t m = __builtin_bit_cast(u16x2_t, w & 0x7fff7fffu);
  const u16x2_t r = __builtin_elementwise_sub_sat(m, u16x2_t{exp_step, exp_step});
  return __builtin_bit_cast(uint32_t, r) | (w & 0x80008000u);
}
// A token fragment prepared for tdecode_int2_ps: dword 1 / 4, dword 2 / 16.
__device__ __forceinline__ u32x4_t prescale_x_int2(u32x4_t v) {
  v[1] = bf16x2_div_pow4(v[1], 0x0100);
  v[2] = bf16x2_div_pow4(v[2], 0x0200);
  return v;
}

template <int WF>
__device__ __forceinline__ u32x4_t neg_offset_fragment() {
  const uint32_t c = (WF == WF_INT4) ? kNegOffset4 : kNegOffset2;
  return u32x4_t{c, c, c, c};
}

}  // namespace moe
