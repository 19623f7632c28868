// Host-only validation battery of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the real validation layer (moe_abi.cpp,
// plan.cpp) and launchers that abort if reached.  Every call below is one the
// library must reject (or a T = 0 no-op): it must return the expected status,
// reach no launcher and leave every sentinel buffer untouched.  Workspace
// sizes are also computed over the whole shape domain, including its corners,
// so that UBSan sees every size computation.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe.h"

namespace {

int g_fail = 0;

#define EXPECT_EQ(got, want)                                                              \
  do {                                                                                    \
    const long long g_ = static_cast<long long>(got), w_ = static_cast<long long>(want); \
    if (g_ != w_) {                                                                       \
      std::fprintf(stderr, "FAIL %s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #got, \
                   g_, w_);                                                               \
      ++g_fail;                                                                           \
    }                                                                                     \
  } while (0)

// Host buffer with a sentinel fill standing in for device memory; the
// address handed out is 256-byte aligned.
struct Buf {
  std::vector<unsigned char> a;
  unsigned char* p;
  explicit Buf(size_t n) : a(n + 512, 0xA5) {
    p = a.data() + (256 - reinterpret_cast<uintptr_t>(a.data()) % 256) % 256;
  }
  bool untouched() const {
    for (unsigned char c : a)
      if (c != 0xA5) return false;
    return true;
  }
};

moe_shape shape(int T, int H, int E, int I, int k, int act = MOE_DT_BF16, int wfmt = MOE_WF_DENSE,
                unsigned flags = 0) {
  moe_shape s;
  s.T = T;
  s.H = H;
  s.E = E;
  s.I = I;
  s.top_k = k;
  s.act = static_cast<moe_dtype>(act);
  s.wfmt = static_cast<moe_wformat>(wfmt);
  s.flags = flags;
  return s;
}

}  // namespace

int main() {
  // small shape whose buffers fit the 64 KiB sentinels: E=4, k=2, H=128, I=128, T=8
  const moe_shape s = shape(8, 128, 4, 128, 2);
  const size_t N = 1 << 16;
  Buf x(N), wr(N), ids(N), w(N), lg(N), ws(N), out(N), res(N), y(N), h(N), g(N), u(N), d(N),
      gs(N), us(N), ds(N), pm[6] = {Buf(N), Buf(N), Buf(N), Buf(N), Buf(N), Buf(N)}, clk(N);
  moe_experts ex{g.p, u.p, d.p, nullptr, nullptr, nullptr};
  moe_experts ex2{gs.p, us.p, ds.p, nullptr, nullptr, nullptr};
  moe_perm perm{reinterpret_cast<int32_t*>(pm[0].p), reinterpret_cast<int32_t*>(pm[1].p),
                reinterpret_cast<int32_t*>(pm[2].p), reinterpret_cast<int32_t*>(pm[3].p),
                reinterpret_cast<int32_t*>(pm[4].p), reinterpret_cast<int32_t*>(pm[5].p)};
  int32_t* pids = reinterpret_cast<int32_t*>(ids.p);
  float* pw = reinterpret_cast<float*>(w.p);
  float* plg = reinterpret_cast<float*>(lg.p);
  const size_t big = size_t{1} << 40;

  // ---- shape domain ---------------------------------------------------------
  const long long bad[][9] = {
      // T, H, E, I, k, act, wfmt, flags, expected
      {8, 100, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 0, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 128, 4, 48, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 128, 2000, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 128, 4, 128, 0, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 128, 4, 128, 5, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {-1, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {131073, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0, MOE_E_SHAPE},
      {8, 128, 4, 128, 2, 7, MOE_WF_DENSE, 0, MOE_E_DTYPE},
      {8, 128, 4, 128, 2, MOE_DT_BF16, 9, 0, MOE_E_FORMAT},
      {8, 128, 4, 128, 2, MOE_DT_F32, MOE_WF_INT4_G32, 0, MOE_E_FORMAT},
      {8, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, 0x80000000u, MOE_E_FLAGS},
      {8, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, MOE_F_FUSED_FFN, MOE_E_FLAGS},
      {8, 128, 4, 96, 2, MOE_DT_BF16, MOE_WF_DENSE, MOE_F_TILED_WEIGHTS, MOE_E_SHAPE},
      {8, 128, 4, 128, 2, MOE_DT_F32, MOE_WF_DENSE, MOE_F_TILED_WEIGHTS, MOE_E_FORMAT},
      {1639, 2560, 512, 640, 10, MOE_DT_BF16, MOE_WF_DENSE,
       MOE_F_TILED_WEIGHTS | MOE_F_FUSED_FFN, MOE_E_LIMIT},
  };
  for (const auto& b : bad) {
    const moe_shape sb = shape(static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]),
                               static_cast<int>(b[3]), static_cast<int>(b[4]), static_cast<int>(b[5]),
                               static_cast<int>(b[6]), static_cast<unsigned>(b[7]));
    EXPECT_EQ(moe_route(&sb, x.p, wr.p, nullptr, pids, pw, plg, ws.p, big, nullptr), b[8]);
    EXPECT_EQ(moe_workspace_size(&sb), 0);
  }
  // workspace sizes over the domain, corners included
  const int Ts[] = {1, 16, 64, 65, 1024, 1025, 4096, 16384, 131072};
  const int Es[] = {1, 16, 512, 1024};
  const int Hs[] = {128, 2560, 65536 - 128};
  const int Is[] = {128, 640, 65536 - 128};
  for (int T : Ts)
    for (int E : Es)
      for (int H : Hs)
        for (int I : Is)
          for (int wf = 0; wf < 3; ++wf)
            for (unsigned fl : {0u, 1u, 3u, 5u, 7u}) {
              const moe_shape sz = shape(T, H, E, I, E < 10 ? E : 10, MOE_DT_BF16, wf, fl);
              const size_t n = moe_workspace_size(&sz);
              (void)n;
              (void)moe_ffn_fused_items(&sz);
            }
  for (int T : Ts) (void)moe_route_locality_blocks(T);
  for (int st = -1; st <= 13; ++st) EXPECT_EQ(moe_status_str(st) != nullptr, 1);

  // ---- pointers, alignment, aliasing, workspace --------------------------
  EXPECT_EQ(moe_route(nullptr, x.p, wr.p, nullptr, pids, pw, plg, ws.p, big, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_route(&s, nullptr, wr.p, nullptr, pids, pw, plg, ws.p, big, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_route(&s, x.p + 2, wr.p, nullptr, pids, pw, plg, ws.p, big, nullptr), MOE_E_ALIGN);
  EXPECT_EQ(moe_route(&s, x.p, wr.p, nullptr, pids, pw, plg + 1, ws.p, big, nullptr), MOE_E_ALIGN);
  EXPECT_EQ(moe_route(&s, x.p, wr.p, nullptr, pids, reinterpret_cast<float*>(ids.p + 16), plg, ws.p,
                      big, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_route(&s, x.p, wr.p, nullptr, pids, pw, reinterpret_cast<float*>(x.p), ws.p, big,
                      nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_route(&s, x.p, wr.p, nullptr, pids, pw, plg, ws.p, moe_workspace_size(&s) - 1,
                      nullptr), MOE_E_WORKSPACE);
  EXPECT_EQ(moe_route(&s, x.p, wr.p, nullptr, pids, pw, plg, nullptr, big, nullptr), MOE_E_WORKSPACE);
  EXPECT_EQ(moe_permute(&s, pids, nullptr, ws.p, big, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_permute(&s, pids, &perm, ws.p, 16, nullptr), MOE_E_WORKSPACE);
  EXPECT_EQ(moe_permute(&s, reinterpret_cast<int32_t*>(pm[0].p), &perm, ws.p, big, nullptr),
            MOE_E_ALIAS);
  // experts: scales with dense weights, low-bit without scales
  moe_experts dense_sc{g.p, u.p, d.p, reinterpret_cast<uint16_t*>(gs.p), nullptr, nullptr};
  EXPECT_EQ(moe_grouped_ffn(&s, x.p, &dense_sc, &perm, y.p, ws.p, big, nullptr), MOE_E_FORMAT);
  const moe_shape s4 = shape(8, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_INT4_G32);
  EXPECT_EQ(moe_grouped_ffn(&s4, x.p, &ex, &perm, y.p, ws.p, big, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_grouped_ffn(&s, x.p, &ex, &perm, g.p, ws.p, big, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_ffn_gate_up(&s, x.p, &ex, &perm, nullptr, ws.p, big, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_ffn_down(&s, h.p, &ex, h.p + 64, ws.p, big, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_combine(&s, y.p, pids, pw, res.p, res.p + 32, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_combine(&s, y.p, pids, nullptr, res.p, out.p, nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_layer(&s, x.p, wr.p, nullptr, &ex, nullptr, x.p + 64, pids, pw, nullptr, ws.p, big,
                      nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_layer(&s, x.p, wr.p, nullptr, nullptr, nullptr, out.p, pids, pw, nullptr, ws.p, big,
                      nullptr), MOE_E_NULL);
  // layout conversion and staging
  const moe_shape st1 = shape(8, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, MOE_F_TILED_WEIGHTS);
  EXPECT_EQ(moe_tile_experts(&st1, &ex, &ex2, nullptr), MOE_E_FLAGS);
  EXPECT_EQ(moe_tile_experts(&s, &ex, &ex, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_stage_experts(&s, &ex, &ex, &perm, MOE_STAGE_GATE_UP, nullptr), MOE_E_ALIAS);
  EXPECT_EQ(moe_stage_experts(&s, &ex, &ex2, &perm, 0, nullptr), MOE_E_FLAGS);
  EXPECT_EQ(moe_stage_experts(&s, &ex, &ex2, &perm, 4, nullptr), MOE_E_FLAGS);
  // pageable host memory is not device-readable (no launch either way);
  // I = 32 keeps the expert records inside the 64 KiB buffers
  const moe_shape ss = shape(8, 128, 4, 32, 2);
  EXPECT_EQ(moe_stage_experts(&ss, &ex, &ex2, &perm, MOE_STAGE_GATE_UP | MOE_STAGE_DOWN, nullptr),
            MOE_E_MEMORY);
  // fused FFN
  const moe_shape sf =
      shape(8, 128, 4, 128, 2, MOE_DT_BF16, MOE_WF_DENSE, MOE_F_TILED_WEIGHTS | MOE_F_FUSED_FFN);
  EXPECT_EQ(moe_ffn_fused(&st1, x.p, &ex, &perm, y.p, 0, nullptr, ws.p, big, nullptr), MOE_E_FLAGS);
  EXPECT_EQ(moe_ffn_fused(&sf, x.p, &ex, &perm, y.p, -1, nullptr, ws.p, big, nullptr), MOE_E_SHAPE);
  EXPECT_EQ(moe_ffn_fused(&sf, x.p, &ex, &perm, y.p, 0, reinterpret_cast<uint64_t*>(clk.p + 8), ws.p,
                          big, nullptr), MOE_E_ALIGN);
  EXPECT_EQ(moe_ffn_fused(&sf, x.p, &ex, &perm, y.p, 0, reinterpret_cast<uint64_t*>(y.p), ws.p, big,
                          nullptr), MOE_E_ALIAS);
  // measurement helpers
  EXPECT_EQ(moe_stream_read(nullptr, 16, reinterpret_cast<uint32_t*>(out.p), nullptr), MOE_E_NULL);
  EXPECT_EQ(moe_stream_read(x.p, 24, reinterpret_cast<uint32_t*>(out.p), nullptr), MOE_E_SHAPE);
  EXPECT_EQ(moe_route_locality(&s, nullptr, pids, pids, nullptr), MOE_E_NULL);
  // T = 0 is a no-op for every entry point
  const moe_shape s0 = shape(0, 128, 4, 128, 2);
  EXPECT_EQ(moe_route(&s0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
            MOE_OK);
  EXPECT_EQ(moe_layer(&s0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, nullptr, 0, nullptr), MOE_OK);

  const Buf* all[] = {&x, &wr, &ids, &w, &lg, &ws, &out, &res, &y, &h, &g, &u, &d, &gs, &us, &ds,
                      &pm[0], &pm[1], &pm[2], &pm[3], &pm[4], &pm[5], &clk};
  for (const Buf* b : all) EXPECT_EQ(b->untouched(), 1);
  if (g_fail) {
    std::fprintf(stderr, "%d failures\n", g_fail);
    return 1;
  }
  std::printf("validation battery: all passed\n");
  return 0;
}
