// Plain, slow CPU oracle of the routed sparse-MoE layer in C++ (TEST
// INFRASTRUCTURE ONLY).
//
// Only tests/, __graft_entry__.smoke() and the CPU-baseline legs of bench.py
// may load it; the product library never does, and it shares no code, table
// or helper with the HIP path (nor with the numpy oracle beside it, which it
// is checked against).  Everything is float64 on the exact stored values:
// bf16 and fp16 bit patterns and small integer codes convert exactly.
// Each output element is computed by one thread in a fixed order, so the
// results do not depend on the thread count.
//
// Sources (page title, note, section):
//  [P-019] "Agent Field Notes -- full corpus", AFN-019 "Hide SSD misses before
//          the router knows they exist": section "Why overlap alone cannot
//          defeat the byte roofline" (expert = gate [I x H] + up [I x H] +
//          down [H x I]; low-bit storage; grouping rows by expert), section
//          "Hypothesis H4: ExpertMajor should stream as a wavefront, not a
//          barrier" (gate and up feed the SwiGLU intermediate before down;
//          separate result slots; the weighted sum in route-rank order).
//  [P-001] same page, AFN-001, section "Phase 1: separate math from
//          acceleration" (float32 router softmax, normalized top-10).
//  [P-017] same page, AFN-017, section "Tie handling belongs to membership"
//          (equal scores: the smaller expert index is chosen).
//  [P-021] same page, AFN-021, section "The key equivalence -- and where it
//          breaks" (expert IDs in rank order).
// Readings where the pages leave a step open: the optional router bias is
// added before selection and softmax; selection uses the logits (softmax is
// monotone); the renormalized weights are the softmax probabilities of the
// selected experts divided by their sum; int4 / int2 codes are signed
// two's complement packed little-endian along the reduction axis, one fp16
// scale per 32 of them (w = q * s).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

double bf16_to_double(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// IEEE binary16 -> double, from the bit fields (exact).
double fp16_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1, exp = (h >> 10) & 0x1f, man = h & 0x3ff;
  double v;
  if (exp == 0) v = std::ldexp(static_cast<double>(man), -24);   // subnormal / zero
  else if (exp == 31) v = man ? NAN : INFINITY;
  else v = std::ldexp(static_cast<double>(man + 1024), exp - 25);
  return sign ? -v : v;
}

// Run f(i) for i in [0, n) on `threads` threads, each i on one thread.
template <typename F>
void parallel_for(int n, int threads, F f) {
  if (threads <= 1 || n <= 1) {
    for (int i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int w = 0; w < threads; ++w)
    pool.emplace_back([=, &f] {
      for (int i = w; i < n; i += threads) f(i);
    });
  for (auto& th : pool) th.join();
}

// Row `r` of one expert matrix with K columns, decoded to doubles.
// wfmt 0: dense values (act 0: float32, act 1: bf16 bit patterns);
// wfmt 1 / 2: packed int4 / int2 codes (element c at byte c*bits/8, bit
// (c*bits)%8) times the fp16 scale of its group of 32 ([P-019] "Why overlap
// alone cannot defeat the byte roofline": low-bit storage).
void decode_row(int wfmt, int act, const void* mat, const uint16_t* scales, int r, int K,
                double* out) {
  if (wfmt == 0) {
    if (act == 0) {
      const float* m = static_cast<const float*>(mat) + static_cast<size_t>(r) * K;
      for (int c = 0; c < K; ++c) out[c] = static_cast<double>(m[c]);
    } else {
      const uint16_t* m = static_cast<const uint16_t*>(mat) + static_cast<size_t>(r) * K;
      for (int c = 0; c < K; ++c) out[c] = bf16_to_double(m[c]);
    }
    return;
  }
  const int bits = wfmt == 1 ? 4 : 2;
  const int row_bytes = K * bits / 8;
  const uint8_t* m = static_cast<const uint8_t*>(mat) + static_cast<size_t>(r) * row_bytes;
  const uint16_t* s = scales + static_cast<size_t>(r) * (K / 32);
  for (int c = 0; c < K; ++c) {
    const int bit = c * bits;
    int q = (m[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
    if (q >= (1 << (bits - 1))) q -= (1 << bits);   // two's complement
    out[c] = static_cast<double>(q) * fp16_to_double(s[c / 32]);
  }
}

}  // namespace

extern "C" {

// Activation storage -> double: act 0 float32 values, act 1 bf16 bit
// patterns (exact in both cases).
void oc_decode_act(int act, int64_t n, const void* src, double* dst) {
  for (int64_t i = 0; i < n; ++i)
    dst[i] = act == 0 ? static_cast<double>(static_cast<const float*>(src)[i])
                      : bf16_to_double(static_cast<const uint16_t*>(src)[i]);
}

// double -> bf16 bit pattern, one rounding to nearest with ties to even (the
// storage step between stacked layers: x_{l+1} is stored in the activation
// type).  bf16 keeps 8 significant bits and float32's exponent range: the
// value is rounded on the grid of its binade (ulp 2^(e-7) for 2^e <= |v| <
// 2^(e+1), e >= -126; ulp 2^-133 below), then written through float32,
// which holds every bf16 value exactly.  Finite inputs only; values that
// round beyond the largest bf16 become infinity.
void oc_round_bf16(int64_t n, const double* src, uint16_t* dst) {
  for (int64_t i = 0; i < n; ++i) {
    const double v = src[i];
    double r = 0.0;
    if (v != 0.0) {
      int e = std::ilogb(v);
      if (e < -126) e = -126;
      const double q = std::nearbyint(std::ldexp(v, 7 - e));   // default mode: ties to even
      r = std::ldexp(q, e - 7);
    } else {
      r = v;   // keeps the sign of zero
    }
    float f = static_cast<float>(r);   // exact unless it overflows
    if (std::fabs(r) > 3.3895313892515355e38) f = r > 0 ? INFINITY : -INFINITY;
    uint32_t u;
    std::memcpy(&u, &f, sizeof u);
    dst[i] = static_cast<uint16_t>(u >> 16);
  }
}

// logits[t][e] = sum_{h ascending} x[t][h] * wr[e][h] (+ bias[e])
// ([P-001] "Phase 1"; the bias is a reading of the pages).
void oc_router_logits(int T, int H, int E, const double* x, const double* wr, const double* bias,
                      int threads, double* logits) {
  parallel_for(T, threads, [&](int t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += x[static_cast<size_t>(t) * H + h] * wr[static_cast<size_t>(e) * H + h];
      if (bias) s += bias[e];
      logits[static_cast<size_t>(t) * E + e] = s;
    }
  });
}

// Exact top-k by the rank-count definition: rank(e) = #{e' : l[e'] > l[e]}
// + #{e' < e : l[e'] == l[e]}; e is selected iff rank < k, at position rank
// ([P-017] "Tie handling belongs to membership", [P-021] "The key
// equivalence").  Returns 0, or -1 on a non-finite logit.
int oc_select_topk(int T, int E, int k, const double* logits, int threads, int32_t* ids) {
  int bad = 0;
  for (size_t i = 0; i < static_cast<size_t>(T) * E; ++i)
    if (!std::isfinite(logits[i])) bad = 1;
  if (bad) return -1;
  parallel_for(T, threads, [&](int t) {
    const double* l = logits + static_cast<size_t>(t) * E;
    for (int e = 0; e < E; ++e) {
      int rank = 0;
      for (int f = 0; f < E; ++f)
        if (l[f] > l[e] || (l[f] == l[e] && f < e)) ++rank;
      if (rank < k) ids[static_cast<size_t>(t) * k + rank] = e;
    }
  });
  return 0;
}

// Softmax over all E experts, then the selected probabilities divided by
// their sum ([P-001] "Phase 1": float32 router softmax, normalized top-k).
void oc_route_weights(int T, int E, int k, const double* logits, const int32_t* ids,
                      double* w) {
  for (int t = 0; t < T; ++t) {
    const double* l = logits + static_cast<size_t>(t) * E;
    double m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += std::exp(l[e] - m);
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += std::exp(l[ids[static_cast<size_t>(t) * k + j]] - m) / z;
    for (int j = 0; j < k; ++j)
      w[static_cast<size_t>(t) * k + j] =
          (std::exp(l[ids[static_cast<size_t>(t) * k + j]] - m) / z) / sel;
  }
}

// Stable counting sort of the pairs p = t*k + j by expert ([P-019] "Why
// overlap alone cannot defeat the byte roofline": rows grouped by expert):
// counts, offsets (exclusive scan), row -> pair, pair -> row, the active
// experts ascending.  Returns the number of active experts, or -1 (nothing
// written) if an id is outside [0, E).
int oc_permutation(int P, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_pair, int32_t* pair_row, int32_t* active) {
  for (int p = 0; p < P; ++p)
    if (ids[p] < 0 || ids[p] >= E) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int p = 0; p < P; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(E, 0);
  for (int p = 0; p < P; ++p) {
    const int e = ids[p];
    const int row = offsets[e] + fill[e]++;
    sorted_pair[row] = p;
    pair_row[p] = row;
  }
  int n = 0;
  for (int e = 0; e < E; ++e)
    if (counts[e] > 0) active[n++] = e;
  return n;
}

// Y[row] = W_down (silu(W_gate x_t) * (W_up x_t)) for the expert and token of
// every row ([P-019] "Hypothesis H4": gate and up feed the intermediate,
// down only after it exists, one result slot per pair).  Weight layouts:
// gate/up [E][I][H], down [E][H][I] (values, or packed codes with fp16
// scales [E][rows][K/32]).  Each active expert's matrices are decoded once.
void oc_grouped_ffn(int T, int H, int E, int I, int k, int wfmt, int act, const double* x,
                    const void* gate, const void* up, const void* down, const uint16_t* gs,
                    const uint16_t* us, const uint16_t* ds, const int32_t* offsets,
                    const int32_t* sorted_pair, const int32_t* active, int n_active, int threads,
                    double* Y) {
  (void)T;
  (void)E;
  const int bits = wfmt == 1 ? 4 : (wfmt == 2 ? 2 : 0);
  const size_t esz = act == 0 ? 4 : 2;
  auto mat_at = [&](const void* base, int e, int rows, int K) -> const void* {
    const size_t per = wfmt == 0 ? static_cast<size_t>(rows) * K * esz
                                 : static_cast<size_t>(rows) * K * bits / 8;
    return static_cast<const uint8_t*>(base) + static_cast<size_t>(e) * per;
  };
  auto sc_at = [&](const uint16_t* base, int e, int rows, int K) -> const uint16_t* {
    return base ? base + static_cast<size_t>(e) * rows * (K / 32) : nullptr;
  };
  std::vector<double> wg(static_cast<size_t>(I) * H), wu(static_cast<size_t>(I) * H),
      wd(static_cast<size_t>(H) * I);
  for (int a = 0; a < n_active; ++a) {
    const int e = active[a];
    for (int i = 0; i < I; ++i) {
      decode_row(wfmt, act, mat_at(gate, e, I, H), sc_at(gs, e, I, H), i, H, &wg[static_cast<size_t>(i) * H]);
      decode_row(wfmt, act, mat_at(up, e, I, H), sc_at(us, e, I, H), i, H, &wu[static_cast<size_t>(i) * H]);
    }
    for (int n = 0; n < H; ++n)
      decode_row(wfmt, act, mat_at(down, e, H, I), sc_at(ds, e, H, I), n, I, &wd[static_cast<size_t>(n) * I]);
    const int r0 = offsets[e], r1 = offsets[e + 1];
    parallel_for(r1 - r0, threads, [&](int rr) {
      const int row = r0 + rr;
      const double* xt = x + static_cast<size_t>(sorted_pair[row] / k) * H;
      std::vector<double> a_(I);
      for (int i = 0; i < I; ++i) {
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
          g += wg[static_cast<size_t>(i) * H + h] * xt[h];
          u += wu[static_cast<size_t>(i) * H + h] * xt[h];
        }
        a_[i] = g / (1.0 + std::exp(-g)) * u;   // silu(g) * u
      }
      for (int n = 0; n < H; ++n) {
        double y = 0.0;
        for (int i = 0; i < I; ++i) y += wd[static_cast<size_t>(n) * I + i] * a_[i];
        Y[static_cast<size_t>(row) * H + n] = y;
      }
    });
  }
}

// out[t] = residual[t] + sum_{j ascending} w[t][j] * Y[pair_row[t*k + j]]
// ([P-019] "Hypothesis H4": the weighted sum in route-rank order).
void oc_combine(int T, int H, int k, const double* Y, const int32_t* pair_row, const double* w,
                const double* residual, double* out) {
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < H; ++n) {
      double s = residual ? residual[static_cast<size_t>(t) * H + n] : 0.0;
      for (int j = 0; j < k; ++j)
        s += w[static_cast<size_t>(t) * k + j] *
             Y[static_cast<size_t>(pair_row[static_cast<size_t>(t) * k + j]) * H + n];
      out[static_cast<size_t>(t) * H + n] = s;
    }
}

}  // extern "C"
