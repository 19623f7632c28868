// C ABI of the routed-MoE layer: host-side validation, launch planning and
// dispatch.  Validation is complete before the first HIP call of an entry
// point, so a rejected call enqueues nothing and writes nothing (the
// fail-closed admission rule of "Agent Field Notes -- full corpus", AFN-001,
// section "Phase 3: reject before the GPU exists").
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "moe_internal.h"

namespace moe {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static size_t act_bytes(const moe_shape& s) { return s.act == MOE_DT_F32 ? 4 : 2; }

static size_t wrow_bytes(const moe_shape& s, int K) {
  switch (s.wfmt) {
    case MOE_WF_INT4_G32: return static_cast<size_t>(K) / 2;
    case MOE_WF_INT2_G32: return static_cast<size_t>(K) / 4;
    default: return static_cast<size_t>(K) * act_bytes(s);
  }
}

// average rows per expert from which bf16 tiled layers use 128-token tiles
// (measured on the Zipf-skewed 2560 x 640 layer: the step is 0.6% slower
// at 40 rows per expert, 1.6% faster at 60, 2.3% at 80, 6% at 640)
constexpr int64_t kWideMinRows = 48;

// 16-row token groups per FFN tile, chosen from the batch size.
// Token rows per tile = 16 nb.  One 16-row block while experts average at
// most 12 rows (padding rows cost MFMA and, for low-bit weights, one scale
// FMA per output and group), then 32 up to 1024 tokens, 64 beyond, and 128
// (bf16 tiled weights, staged calls) once experts average 48 rows.
static int plan_nb(const moe_shape& s) {
  if (s.act == MOE_DT_F32 || s.T <= 16) return 1;
  if (static_cast<int64_t>(s.T) * s.top_k <= 12LL * s.E) return 1;
  if (s.T <= 1024) return 2;
  if (tiles128_ok(s) && !(s.flags & MOE_F_FUSED_FFN) &&
      static_cast<int64_t>(s.T) * s.top_k >= kWideMinRows * s.E)
    return 8;
  return 4;
}

// MOE_F_FUSED_FFN: pairs whose float32 partial results the workspace holds
constexpr int64_t kFusedMaxPairs = 16384;

static int64_t plan_max_tiles(const moe_shape& s) {
  const int64_t P = static_cast<int64_t>(s.T) * s.top_k;
  return P / (16 * plan_nb(s)) + std::min<int64_t>(s.E, P);
}

bool make_plan(const moe_shape& s, Plan* p) {
  const int64_t T = s.T, P = static_cast<int64_t>(s.T) * s.top_k;
  std::memset(p, 0, sizeof(*p));
  p->chunks = permute_single_pass(s) ? 0 : permute_chunks(s);
  p->nb = plan_nb(s);
  p->max_tiles = static_cast<int>(plan_max_tiles(s));

  size_t off = 0;
  p->logits_off = off;
  off = align_up(off + static_cast<size_t>(T) * s.E * sizeof(float), 256);
  if (router_gsum(s)) {
    p->gsum_off = off;
    off = align_up(off + static_cast<size_t>(router_groups(s.H)) * T * s.E * sizeof(double), 256);
  }
  p->chunk_off = off;
  off = align_up(off + static_cast<size_t>(p->chunks) * s.E * 2 * sizeof(int32_t), 256);
  p->perm_off = off;
  off = align_up(off + (static_cast<size_t>(s.E) * 3 + 2 + 2 * P) * sizeof(int32_t), 256);
  p->tiles_off = off;
  off = align_up(off + (static_cast<size_t>(p->max_tiles) * 3 + 2) * sizeof(int32_t), 256);
  p->h_off = off;
  off = align_up(off + static_cast<size_t>(P) * s.I * act_bytes(s), 256);
  p->y_off = off;
  off = align_up(off + static_cast<size_t>(P) * s.H * act_bytes(s), 256);
  if (s.flags & MOE_F_CHECK_FINITE) {
    p->ids_off = off;
    off = align_up(off + static_cast<size_t>(P) * 4, 256);
    p->w_off = off;
    off = align_up(off + static_cast<size_t>(P) * 4, 256);
    p->out_off = off;
    off = align_up(off + static_cast<size_t>(T) * s.H * act_bytes(s), 256);
    p->status_off = off;
    off = align_up(off + 4, 256);
  }
  if (s.flags & MOE_F_FUSED_FFN) {
    p->part_off = off;
    off = align_up(off + static_cast<size_t>(fused_slices(s)) * P * s.H * sizeof(float), 256);
  }
  p->total = off;
  return true;
}

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

struct Span {
  const void* p;
  size_t n;
};

static bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Every output must be disjoint from every other output and every input.
static bool any_alias(const Span* outs, int no, const Span* ins, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = i + 1; j < no; ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (int j = 0; j < ni; ++j)
      if (overlap(outs[i], ins[j])) return true;
  }
  return false;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int check_shape(const moe_shape* s) {
  if (!s) return MOE_E_NULL;
  if (s->flags & ~(MOE_F_TILED_WEIGHTS | MOE_F_CHECK_FINITE | MOE_F_FUSED_FFN)) return MOE_E_FLAGS;
  if ((s->flags & MOE_F_FUSED_FFN) && !(s->flags & MOE_F_TILED_WEIGHTS)) return MOE_E_FLAGS;
  if (s->act != MOE_DT_F32 && s->act != MOE_DT_BF16) return MOE_E_DTYPE;
  if (s->wfmt != MOE_WF_DENSE && s->wfmt != MOE_WF_INT4_G32 && s->wfmt != MOE_WF_INT2_G32)
    return MOE_E_FORMAT;
  if (s->act == MOE_DT_F32 && s->wfmt != MOE_WF_DENSE) return MOE_E_FORMAT;
  if (s->T < 0 || s->T > 131072) return MOE_E_SHAPE;
  if (s->E < 1 || s->E > 1024 || s->top_k < 1 || s->top_k > s->E) return MOE_E_SHAPE;
  if (s->H <= 0 || s->H > 65536 || s->H % 128 != 0) return MOE_E_SHAPE;
  if (s->I <= 0 || s->I > 65536 || s->I % 32 != 0) return MOE_E_SHAPE;
  if (s->flags & MOE_F_TILED_WEIGHTS) {
    if (s->act != MOE_DT_BF16) return MOE_E_FORMAT;
    if (s->I % 128 != 0) return MOE_E_SHAPE;
  }
  const int64_t T = s->T;
  if (T * s->top_k >= (int64_t{1} << 31)) return MOE_E_LIMIT;
  if (T * std::max(s->E, s->H) >= (int64_t{1} << 31)) return MOE_E_LIMIT;
  if (plan_max_tiles(*s) > 65535) return MOE_E_LIMIT;   // FFN grid y dimension
  if ((s->flags & MOE_F_FUSED_FFN) && T * s->top_k > kFusedMaxPairs) return MOE_E_LIMIT;
  return MOE_OK;
}

static int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return MOE_E_NULL;
  for (const void* p : ps)
    if (!aligned16(p)) return MOE_E_ALIGN;
  return MOE_OK;
}

static int check_opt_ptr(const void* p) { return (p && !aligned16(p)) ? MOE_E_ALIGN : MOE_OK; }

static int check_ws(const Plan& pl, void* ws, size_t bytes) {
  if (pl.total == 0) return MOE_OK;
  if (!ws || bytes < pl.total) return MOE_E_WORKSPACE;
  if (!aligned16(ws)) return MOE_E_ALIGN;
  return MOE_OK;
}

static int check_perm(const moe_perm* pm) {
  if (!pm) return MOE_E_NULL;
  return check_ptrs({pm->counts, pm->offsets, pm->sorted_pair, pm->pair_row, pm->active, pm->n_active});
}

static int check_experts(const moe_shape& s, const moe_experts* ex) {
  if (!ex) return MOE_E_NULL;
  int st = check_ptrs({ex->gate, ex->up, ex->down});
  if (st) return st;
  const bool q = s.wfmt != MOE_WF_DENSE;
  if (q) return check_ptrs({ex->gate_scale, ex->up_scale, ex->down_scale});
  if (ex->gate_scale || ex->up_scale || ex->down_scale) return MOE_E_FORMAT;
  return MOE_OK;
}

static void expert_spans(const moe_shape& s, const moe_experts& ex, Span* out /*[6]*/) {
  const size_t gu = static_cast<size_t>(s.E) * s.I * wrow_bytes(s, s.H);
  const size_t dn = static_cast<size_t>(s.E) * s.H * wrow_bytes(s, s.I);
  const size_t gs = static_cast<size_t>(s.E) * s.I * (s.H / 32) * 2;
  const size_t ds = static_cast<size_t>(s.E) * s.H * (s.I / 32) * 2;
  out[0] = {ex.gate, gu};
  out[1] = {ex.up, gu};
  out[2] = {ex.down, dn};
  out[3] = {ex.gate_scale, ex.gate_scale ? gs : 0};
  out[4] = {ex.up_scale, ex.up_scale ? gs : 0};
  out[5] = {ex.down_scale, ex.down_scale ? ds : 0};
}

static void perm_spans(const moe_shape& s, const moe_perm& pm, Span* out /*[6]*/) {
  const size_t P = static_cast<size_t>(s.T) * s.top_k;
  out[0] = {pm.counts, s.E * 4u};
  out[1] = {pm.offsets, (s.E + 1) * 4u};
  out[2] = {pm.sorted_pair, P * 4};
  out[3] = {pm.pair_row, P * 4};
  out[4] = {pm.active, s.E * 4u};
  out[5] = {pm.n_active, 4};
}

static PermPtrs perm_ptrs(const moe_perm& pm) {
  return PermPtrs{pm.counts, pm.offsets, pm.sorted_pair, pm.pair_row, pm.active, pm.n_active};
}

static PermPtrs ws_perm(const moe_shape& s, const Plan& pl, void* ws) {
  int32_t* b = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.perm_off);
  const size_t P = static_cast<size_t>(s.T) * s.top_k;
  PermPtrs pp;
  pp.counts = b;
  pp.offsets = b + s.E;
  pp.sorted_pair = b + 2 * s.E + 1;
  pp.pair_row = pp.sorted_pair + P;
  pp.active = pp.pair_row + P;
  pp.n_active = pp.active + s.E;
  return pp;
}

static int32_t* ws_tiles(const Plan& pl, void* ws) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(ws) + pl.tiles_off);
}

static int device_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_DEVICE; }

// MOE_F_CHECK_FINITE: wait for the enqueued work and read the status word.
static int finite_status(const Plan& pl, void* ws, hipStream_t st, hipError_t e) {
  if (e != hipSuccess) return MOE_E_DEVICE;
  uint32_t host = 0;
  const uint32_t* dev = reinterpret_cast<const uint32_t*>(static_cast<char*>(ws) + pl.status_off);
  if (hipMemcpyAsync(&host, dev, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return MOE_E_DEVICE;
  return host ? MOE_E_NONFINITE : MOE_OK;
}

static hipError_t publish(void* dst, const void* src, size_t bytes, hipStream_t st) {
  return bytes ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
}

constexpr uint32_t kBadX = 1u, kBadLogits = 2u, kBadOut = 4u;

// The expert FFN and the combine of moe_layer: gate/up, down, combine of y;
// or, with MOE_F_FUSED_FFN, the fused kernel and the combine of its partial
// results.
static hipError_t ffn_and_combine(const moe_shape& s, const Plan& pl, const void* x,
                                  const moe_experts& ex, const PermPtrs& pp, int32_t* tiles,
                                  const float* w, const void* residual, void* out, void* ws,
                                  hipStream_t st) {
  char* wsb = static_cast<char*>(ws);
  if (s.flags & MOE_F_FUSED_FFN) {
    float* part = reinterpret_cast<float*>(wsb + pl.part_off);
    hipError_t e = launch_ffn_fused(s, pl, x, ex, pp.sorted_pair, tiles, part, 0, nullptr, st);
    if (e == hipSuccess) e = launch_combine_parts(s, part, pp.pair_row, w, residual, out, st);
    return e;
  }
  void* h = wsb + pl.h_off;
  void* y = wsb + pl.y_off;
  hipError_t e = launch_gateup(s, pl, x, ex, pp.sorted_pair, tiles, h, st);
  if (e == hipSuccess)
    e = launch_down_combine(s, pl, h, ex, tiles, pp.sorted_pair, pp.pair_row, w, residual, out, y,
                            st);
  return e;
}

int layer_call(const moe_shape* shape, const void* x, const void* w_router, const float* router_bias,
               const moe_experts* experts, const void* residual, void* out, int32_t* topk_ids,
               float* topk_w, const moe_perm* perm, void* workspace, size_t workspace_bytes,
               hipStream_t stream, ScratchFn scratch) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, w_router, out, topk_ids, topk_w}))) return st;
  if ((st = check_opt_ptr(router_bias)) || (st = check_opt_ptr(residual))) return st;
  if ((st = check_experts(s, experts))) return st;
  if (perm && (st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  // the no-allocation entry point supplies its own scratch once the call is valid
  if (scratch && (st = scratch(pl.total, stream, &workspace, &workspace_bytes))) return st;
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span outs[10];
  outs[0] = {out, static_cast<size_t>(s.T) * s.H * ab};
  outs[1] = {topk_ids, P * 4};
  outs[2] = {topk_w, P * 4};
  outs[3] = {workspace, pl.total};
  int no = 4;
  if (perm) {
    perm_spans(s, *perm, outs + 4);
    no = 10;
  }
  Span ins[10];
  ins[0] = {x, static_cast<size_t>(s.T) * s.H * ab};
  ins[1] = {w_router, static_cast<size_t>(s.E) * s.H * ab};
  ins[2] = {router_bias, router_bias ? s.E * 4u : 0};
  ins[3] = {residual, residual ? static_cast<size_t>(s.T) * s.H * ab : 0};
  expert_spans(s, *experts, ins + 4);
  if (any_alias(outs, no, ins, 10)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  int32_t* tiles = ws_tiles(pl, workspace);
  char* wsb = static_cast<char*>(workspace);
  if (!(s.flags & MOE_F_CHECK_FINITE)) {
    const PermPtrs pp = perm ? perm_ptrs(*perm) : ws_perm(s, pl, workspace);
    hipError_t e = launch_route_permute(s, pl, x, w_router, router_bias, topk_ids, topk_w, nullptr,
                                        pp, tiles, workspace, stream);
    if (e == hipSuccess) e = ffn_and_combine(s, pl, x, *experts, pp, tiles, topk_w, residual, out, workspace, stream);
    return device_status(e);
  }
  // private results (ids, weights, permutation, output), checked, then published
  const PermPtrs wp = ws_perm(s, pl, workspace);
  int32_t* pids = reinterpret_cast<int32_t*>(wsb + pl.ids_off);
  float* pw = reinterpret_cast<float*>(wsb + pl.w_off);
  void* pout = wsb + pl.out_off;
  uint32_t* status = reinterpret_cast<uint32_t*>(wsb + pl.status_off);
  const bool bf = s.act == MOE_DT_BF16;
  const size_t TH = static_cast<size_t>(s.T) * s.H;
  hipError_t e = launch_zero_status(status, stream);
  if (e == hipSuccess) e = launch_check_finite(x, TH, bf, kBadX, status, stream);
  if (e == hipSuccess)
    e = launch_route(s, pl, x, w_router, router_bias, pids, pw, nullptr, workspace, stream);
  if (e == hipSuccess)
    e = launch_check_finite(wsb + pl.logits_off, static_cast<size_t>(s.T) * s.E, false, kBadLogits,
                            status, stream);
  if (e == hipSuccess) e = launch_permute(s, pl, pids, wp, tiles, workspace, stream);
  if (e == hipSuccess) e = ffn_and_combine(s, pl, x, *experts, wp, tiles, pw, residual, pout, workspace, stream);
  if (e == hipSuccess) e = launch_check_finite(pout, TH, bf, kBadOut, status, stream);
  if ((st = finite_status(pl, workspace, stream, e))) return st;
  e = publish(out, pout, TH * ab, stream);
  if (e == hipSuccess) e = publish(topk_ids, pids, P * 4, stream);
  if (e == hipSuccess) e = publish(topk_w, pw, P * 4, stream);
  if (e == hipSuccess && perm) {
    const PermPtrs cp = perm_ptrs(*perm);
    e = publish(cp.counts, wp.counts, s.E * 4u, stream);
    if (e == hipSuccess) e = publish(cp.offsets, wp.offsets, (s.E + 1) * 4u, stream);
    if (e == hipSuccess) e = publish(cp.sorted_pair, wp.sorted_pair, P * 4, stream);
    if (e == hipSuccess) e = publish(cp.pair_row, wp.pair_row, P * 4, stream);
    if (e == hipSuccess) e = publish(cp.active, wp.active, s.E * 4u, stream);
    if (e == hipSuccess) e = publish(cp.n_active, wp.n_active, 4, stream);
  }
  return device_status(e);
}


}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_size(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  if (shape->T == 0) return 0;
  Plan pl;
  make_plan(*shape, &pl);
  return pl.total;
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_E_NULL: return "MOE_E_NULL: a required pointer is NULL";
    case MOE_E_SHAPE: return "MOE_E_SHAPE: dimension outside the supported domain";
    case MOE_E_DTYPE: return "MOE_E_DTYPE: unknown activation type";
    case MOE_E_FORMAT: return "MOE_E_FORMAT: unsupported weight format or combination";
    case MOE_E_ALIGN: return "MOE_E_ALIGN: pointer not 16-byte aligned";
    case MOE_E_ALIAS: return "MOE_E_ALIAS: an output overlaps another buffer";
    case MOE_E_WORKSPACE: return "MOE_E_WORKSPACE: workspace missing or too small";
    case MOE_E_LIMIT: return "MOE_E_LIMIT: index arithmetic would exceed 2^31";
    case MOE_E_DEVICE: return "MOE_E_DEVICE: HIP error while enqueuing";
    case MOE_E_FLAGS: return "MOE_E_FLAGS: unknown flag bit or unsupported flag combination";
    case MOE_E_NONFINITE: return "MOE_E_NONFINITE: NaN or infinity found; outputs not written";
    case MOE_E_MEMORY: return "MOE_E_MEMORY: a source buffer is not device-readable memory";
    default: return "unknown moe status";
  }
}

int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* router_bias,
              int32_t* topk_ids, float* topk_w, float* logits, void* workspace,
              size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, w_router, topk_ids, topk_w}))) return st;
  if ((st = check_opt_ptr(router_bias)) || (st = check_opt_ptr(logits))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  const Span outs[] = {{topk_ids, P * 4}, {topk_w, P * 4},
                       {logits, logits ? static_cast<size_t>(s.T) * s.E * 4 : 0},
                       {workspace, pl.total}};
  const Span ins[] = {{x, static_cast<size_t>(s.T) * s.H * ab},
                      {w_router, static_cast<size_t>(s.E) * s.H * ab},
                      {router_bias, router_bias ? s.E * 4u : 0}};
  if (any_alias(outs, 4, ins, 3)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  if (!(s.flags & MOE_F_CHECK_FINITE))
    return device_status(
        launch_route(s, pl, x, w_router, router_bias, topk_ids, topk_w, logits, workspace, stream));
  // private results, checked, then published
  char* wsb = static_cast<char*>(workspace);
  int32_t* pids = reinterpret_cast<int32_t*>(wsb + pl.ids_off);
  float* pw = reinterpret_cast<float*>(wsb + pl.w_off);
  float* plg = reinterpret_cast<float*>(wsb + pl.logits_off);
  uint32_t* status = reinterpret_cast<uint32_t*>(wsb + pl.status_off);
  const bool bf = s.act == MOE_DT_BF16;
  hipError_t e = launch_zero_status(status, stream);
  if (e == hipSuccess) e = launch_check_finite(x, static_cast<size_t>(s.T) * s.H, bf, kBadX, status, stream);
  if (e == hipSuccess) e = launch_route(s, pl, x, w_router, router_bias, pids, pw, plg, workspace, stream);
  if (e == hipSuccess) e = launch_check_finite(plg, static_cast<size_t>(s.T) * s.E, false, kBadLogits, status, stream);
  if ((st = finite_status(pl, workspace, stream, e))) return st;
  e = publish(topk_ids, pids, P * 4, stream);
  if (e == hipSuccess) e = publish(topk_w, pw, P * 4, stream);
  if (e == hipSuccess && logits) e = publish(logits, plg, static_cast<size_t>(s.T) * s.E * 4, stream);
  return device_status(e);
}

int moe_permute(const moe_shape* shape, const int32_t* topk_ids, const moe_perm* perm,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({topk_ids}))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k;
  Span outs[7];
  perm_spans(s, *perm, outs);
  outs[6] = {workspace, pl.total};
  const Span ins[] = {{topk_ids, P * 4}};
  if (any_alias(outs, 7, ins, 1)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(
      launch_permute(s, pl, topk_ids, perm_ptrs(*perm), ws_tiles(pl, workspace), workspace, stream));
}

int moe_route_permute(const moe_shape* shape, const void* x, const void* w_router,
                      const float* router_bias, int32_t* topk_ids, float* topk_w, float* logits,
                      const moe_perm* perm, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, w_router, topk_ids, topk_w}))) return st;
  if ((st = check_opt_ptr(router_bias)) || (st = check_opt_ptr(logits))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span outs[10];
  outs[0] = {topk_ids, P * 4};
  outs[1] = {topk_w, P * 4};
  outs[2] = {logits, logits ? static_cast<size_t>(s.T) * s.E * 4 : 0};
  outs[3] = {workspace, pl.total};
  perm_spans(s, *perm, outs + 4);
  const Span ins[] = {{x, static_cast<size_t>(s.T) * s.H * ab},
                      {w_router, static_cast<size_t>(s.E) * s.H * ab},
                      {router_bias, router_bias ? s.E * 4u : 0}};
  if (any_alias(outs, 10, ins, 3)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_route_permute(s, pl, x, w_router, router_bias, topk_ids, topk_w,
                                            logits, perm_ptrs(*perm), ws_tiles(pl, workspace),
                                            workspace, stream));
}

int moe_grouped_ffn(const moe_shape* shape, const void* x, const moe_experts* experts,
                    const moe_perm* perm, void* y, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, y}))) return st;
  if ((st = check_experts(s, experts))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span ins[13];
  ins[0] = {x, static_cast<size_t>(s.T) * s.H * ab};
  expert_spans(s, *experts, ins + 1);
  perm_spans(s, *perm, ins + 7);
  const Span outs[] = {{y, P * s.H * ab}, {workspace, pl.total}};
  if (any_alias(outs, 2, ins, 13)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  void* h = static_cast<char*>(workspace) + pl.h_off;
  int32_t* tiles = ws_tiles(pl, workspace);
  hipError_t e = launch_plan_tiles(s, pl, perm_ptrs(*perm), tiles, stream);
  if (e == hipSuccess) e = launch_ffn(s, pl, x, *experts, perm->sorted_pair, tiles, h, y, stream);
  return device_status(e);
}

int moe_ffn_gate_up(const moe_shape* shape, const void* x, const moe_experts* experts,
                    const moe_perm* perm, void* h, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, h}))) return st;
  if ((st = check_experts(s, experts))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span ins[13];
  ins[0] = {x, static_cast<size_t>(s.T) * s.H * ab};
  expert_spans(s, *experts, ins + 1);
  perm_spans(s, *perm, ins + 7);
  const Span outs[] = {{h, P * s.I * ab}, {workspace, pl.total}};
  if (any_alias(outs, 2, ins, 13)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(
      launch_gateup(s, pl, x, *experts, perm->sorted_pair, ws_tiles(pl, workspace), h, stream));
}

int moe_ffn_down(const moe_shape* shape, const void* h, const moe_experts* experts, void* y,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({h, y}))) return st;
  if ((st = check_experts(s, experts))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span ins[7];
  ins[0] = {h, P * s.I * ab};
  expert_spans(s, *experts, ins + 1);
  const Span outs[] = {{y, P * s.H * ab}, {workspace, pl.total}};
  if (any_alias(outs, 2, ins, 7)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_down(s, pl, h, *experts, ws_tiles(pl, workspace), y, stream));
}

int moe_ffn_down_combine(const moe_shape* shape, const void* h, const moe_experts* experts,
                         const moe_perm* perm, const float* topk_w, const void* residual, void* out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({h, topk_w, out}))) return st;
  if ((st = check_opt_ptr(residual))) return st;
  if ((st = check_experts(s, experts))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span ins[15];
  ins[0] = {h, P * s.I * ab};
  expert_spans(s, *experts, ins + 1);
  perm_spans(s, *perm, ins + 7);
  ins[13] = {topk_w, P * 4};
  ins[14] = {residual, residual ? static_cast<size_t>(s.T) * s.H * ab : 0};
  const Span outs[] = {{out, static_cast<size_t>(s.T) * s.H * ab}, {workspace, pl.total}};
  if (any_alias(outs, 2, ins, 15)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  char* wsb = static_cast<char*>(workspace);
  return device_status(launch_down_combine(s, pl, h, *experts, ws_tiles(pl, workspace),
                                           perm->sorted_pair, perm->pair_row, topk_w, residual,
                                           out, wsb + pl.y_off, stream));
}

int moe_ffn_fused(const moe_shape* shape, const void* x, const moe_experts* experts,
                  const moe_perm* perm, void* y, int32_t wave_tiles, uint64_t* item_clock,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (!(s.flags & MOE_F_FUSED_FFN)) return MOE_E_FLAGS;
  if (wave_tiles < 0) return MOE_E_SHAPE;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({x, y}))) return st;
  if ((st = check_opt_ptr(item_clock))) return st;
  if ((st = check_experts(s, experts))) return st;
  if ((st = check_perm(perm))) return st;
  Plan pl;
  make_plan(s, &pl);
  if ((st = check_ws(pl, workspace, workspace_bytes))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  Span ins[13];
  ins[0] = {x, static_cast<size_t>(s.T) * s.H * ab};
  expert_spans(s, *experts, ins + 1);
  perm_spans(s, *perm, ins + 7);
  const size_t items = static_cast<size_t>(pl.max_tiles) * fused_slices(s);
  const Span outs[] = {{y, P * s.H * ab},
                       {workspace, pl.total},
                       {item_clock, item_clock ? 3 * items * sizeof(uint64_t) : 0}};
  if (any_alias(outs, 3, ins, 13)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  int32_t* tiles = ws_tiles(pl, workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_off);
  hipError_t e = launch_plan_tiles(s, pl, perm_ptrs(*perm), tiles, stream);
  if (e == hipSuccess)
    e = launch_ffn_fused(s, pl, x, *experts, perm->sorted_pair, tiles, part, wave_tiles, item_clock,
                         stream);
  if (e == hipSuccess) e = launch_reduce_parts(s, part, y, stream);
  return device_status(e);
}

size_t moe_ffn_fused_items(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK || !(shape->flags & MOE_F_FUSED_FFN)) return 0;
  return static_cast<size_t>(plan_max_tiles(*shape)) * fused_slices(*shape);
}

int moe_device_clock_khz(int32_t* khz) {
  if (!khz) return MOE_E_NULL;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_DEVICE;
  }
  *khz = rate;
  return MOE_OK;
}

int moe_tile_experts(const moe_shape* shape, const moe_experts* src, const moe_experts* dst,
                     hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.flags != 0) return MOE_E_FLAGS;            // describes the row-major source
  if (s.act != MOE_DT_BF16) return MOE_E_FORMAT;
  if (s.I % 128 != 0) return MOE_E_SHAPE;
  if ((st = check_experts(s, src)) || (st = check_experts(s, dst))) return st;
  Span outs[6], ins[6];
  expert_spans(s, *dst, outs);
  expert_spans(s, *src, ins);
  if (any_alias(outs, 6, ins, 6)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_tile_experts(s, *src, *dst, stream));
}

int moe_combine(const moe_shape* shape, const void* y, const int32_t* pair_row,
                const float* topk_w, const void* residual, void* out, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({y, pair_row, topk_w, out}))) return st;
  if ((st = check_opt_ptr(residual))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k, ab = act_bytes(s);
  const Span outs[] = {{out, static_cast<size_t>(s.T) * s.H * ab}};
  const Span ins[] = {{y, P * s.H * ab},
                      {pair_row, P * 4},
                      {topk_w, P * 4},
                      {residual, residual ? static_cast<size_t>(s.T) * s.H * ab : 0}};
  if (any_alias(outs, 1, ins, 4)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_combine(s, y, pair_row, topk_w, residual, out, stream));
}

int moe_layer(const moe_shape* shape, const void* x, const void* w_router, const float* router_bias,
              const moe_experts* experts, const void* residual, void* out, int32_t* topk_ids,
              float* topk_w, const moe_perm* perm, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  return layer_call(shape, x, w_router, router_bias, experts, residual, out, topk_ids, topk_w, perm,
                    workspace, workspace_bytes, stream, nullptr);
}

// Device-usable address of a buffer the kernel will read: device memory as
// is, pinned host memory through its device mapping; nullptr otherwise.
static const char* device_readable(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice) return static_cast<const char*>(p);
  if (a.type == hipMemoryTypeHost && a.devicePointer && a.hostPointer)
    return static_cast<const char*>(a.devicePointer) +
           (static_cast<const char*>(p) - static_cast<const char*>(a.hostPointer));
  return nullptr;
}

int moe_stage_experts(const moe_shape* shape, const moe_experts* src, const moe_experts* dst,
                      const moe_perm* perm, uint32_t parts, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (parts == 0 || (parts & ~(MOE_STAGE_GATE_UP | MOE_STAGE_DOWN))) return MOE_E_FLAGS;
  const moe_shape& s = *shape;
  if ((st = check_experts(s, src)) || (st = check_experts(s, dst)) || (st = check_perm(perm))) return st;
  Span sp[6], dp[6], pp[6];
  expert_spans(s, *src, sp);
  expert_spans(s, *dst, dp);
  perm_spans(s, *perm, pp);
  if (any_alias(dp, 6, sp, 6) || any_alias(dp, 6, pp, 6)) return MOE_E_ALIAS;
  StagePieces pc;
  const size_t E = static_cast<size_t>(s.E);
  for (int m = 0; m < kStagePieces; ++m) {
    pc.src[m] = nullptr;
    pc.dst[m] = static_cast<char*>(const_cast<void*>(dp[m].p));
    pc.bytes[m] = sp[m].n / E;
    // pieces 0, 1, 3, 4 are gate, up and their scales; 2 and 5 are down's
    const bool down = m == 2 || m == 5;
    if (!sp[m].p || !(parts & (down ? MOE_STAGE_DOWN : MOE_STAGE_GATE_UP))) continue;
    if (pc.bytes[m] % 16 != 0) return MOE_E_SHAPE;
    pc.src[m] = device_readable(sp[m].p);
    if (!pc.src[m]) return MOE_E_MEMORY;
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, dp[m].p) != hipSuccess || a.type != hipMemoryTypeDevice) {
      (void)hipGetLastError();
      return MOE_E_MEMORY;
    }
  }
  (void)hipGetLastError();
  return device_status(launch_stage_experts(s, pc, perm->active, perm->n_active, stream));
}

size_t moe_route_locality_blocks(int32_t T) {
  return T <= 0 ? 0 : static_cast<size_t>(locality_blocks(T));
}

int moe_route_locality(const moe_shape* shape, const int32_t* topk_ids, int32_t* overlap_prev,
                       int32_t* block_unique, hipStream_t stream) {
  int st = check_shape(shape);
  if (st) return st;
  const moe_shape& s = *shape;
  if (s.T == 0) return MOE_OK;
  if ((st = check_ptrs({topk_ids, overlap_prev, block_unique}))) return st;
  const size_t P = static_cast<size_t>(s.T) * s.top_k;
  const Span outs[] = {{overlap_prev, static_cast<size_t>(s.T) * 4},
                       {block_unique, moe_route_locality_blocks(s.T) * 4}};
  const Span ins[] = {{topk_ids, P * 4}};
  if (any_alias(outs, 2, ins, 1)) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_route_locality(s, topk_ids, overlap_prev, block_unique, stream));
}

int moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return MOE_E_NULL;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return MOE_E_ALIGN;
  if (bytes == 0 || bytes % 16 != 0) return MOE_E_SHAPE;
  if (overlap(Span{buf, bytes}, Span{sink, 4})) return MOE_E_ALIAS;
  (void)hipGetLastError();
  return device_status(launch_stream_read(buf, bytes, sink, stream));
}

}  // extern "C"
