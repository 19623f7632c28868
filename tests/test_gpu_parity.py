"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Stage tests feed each HIP stage the oracle's upstream outputs (teacher
forcing) and compare element by element; end-to-end tests run the fused
moe_layer free and compare routes (bit-exact except near ties) and outputs
(bf16: max-abs 2e-2 and rel-L2 1e-2; float32: max-abs 1e-5; weights 1e-5).
"""
import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from moe_inputs import CONFIGS, make_x
from oracle import moe_oracle as O
from tests.gpu_util import (DEV, buffers, check_oracles_agree, check_routes, check_values, decode, i32,
                            make_case, np_of, say, tiled_ok, to_act_tensor)

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = (CONFIGS[i] for i in range(1, 6))

# Sizes the oracle finishes in seconds that still span several tiles, ragged
# tails, both permutation paths and every kernel variant.
SMALL = {
    "tiny": C1,                                                              # workload 1, full
    "tiny_ragged": C1.with_(T=37),
    "decode": C2,                                                            # workload 2, full
    "bf16_ragged": C2.with_(T=37, H=256, E=100, I=96, k=7),
    "prefill_chunked": C3.with_(T=1100, H=256, I=128),                       # chunked permute, 64-row tiles
    "int4_small": C4.with_(T=96, H=512, E=64, I=128, k=8, layers=1),
    "int2_small": C5.with_(T=16, H=512, E=64, I=128, layers=1),
    "int4_many_rows": C4.with_(T=1500, H=256, E=16, I=128, k=4, layers=1),
    # 128-row tiles (T*k >= 48 E, bf16 tiled): gate/up at 8 token blocks,
    # down on 64-row halves; ragged tails, experts with 0..1883 rows, 2 and 3
    # gate/up slices, 2 and 5 k units
    "bf16_tiles128": C3.with_(T=2050, H=256, E=16, I=256, k=2),
    "bf16_tiles128_ragged": C3.with_(T=1300, H=640, E=8, I=384, k=2),
    # low-bit 64-row tiles with 6 gate/up slices of 16 rows per wave
    "int2_many_rows": C5.with_(T=1300, H=256, E=16, I=384, k=4, layers=1, bias="none"),
    "int2_ksplit_rows": C5.with_(T=600, H=384, E=24, I=96, k=3, layers=1, bias="none"),
    # LDS-staged router with a ragged expert tile and parts that end inside
    # a 128-wide k unit (H/32 = 20 chunks, 10 parts of 2)
    "router_ragged_parts": C3.with_(T=200, H=640, E=100, I=128, k=6),
    # top-k at the edges of the threshold selection: k = 64 of 64 experts
    # (64 candidates, the most it ranks directly), k = 65 (k rounds)
    "topk_k64": C2.with_(T=20, H=256, E=64, I=128, k=64),
    "topk_k65": C2.with_(T=20, H=256, E=80, I=128, k=65),
}

_cache = {}

LAYOUT_CASES = [(n, lay) for n in SMALL for lay in ("row", "tiled")
                if lay == "row" or tiled_ok(SMALL[n])]


def get(name):
    if name not in _cache:
        cfg = SMALL[name]
        say(f"[case {name}] generate + oracle: {cfg}")
        case = make_case(cfg)
        res = case.x64 if cfg.residual else None
        ref = O.moe_layer(case.x64, case.wr64, case.bias64, case.ex_oracle, cfg.k, residual=res)
        _cache[name] = (case, ref)
    return _cache[name]


def sync():
    torch.cuda.synchronize()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    M.load()
    yield
    _cache.clear()


@pytest.mark.parametrize("name", list(SMALL))
def test_route(name):
    case, ref = get(name)
    cfg = case.cfg
    buf = buffers(cfg)
    say(f"[case {name}] moe_route")
    buf.route(case.li.x, case.li.w_router, case.li.bias)
    sync()
    lg = buf.logits.cpu().numpy().astype(np.float64)
    dl = np.abs(lg - ref.logits)
    assert (dl <= 1e-5 * np.maximum(1.0, np.abs(ref.logits))).all(), f"max |dlogit| {dl.max()}"
    stats, _ = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                            ref.logits, ref.ids, ref.w, cfg.k)
    say(f"[case {name}] routes {stats} max|dlogit| {dl.max():.3g}")


@pytest.mark.parametrize("name", list(SMALL))
def test_permute(name):
    case, ref = get(name)
    cfg = case.cfg
    buf = buffers(cfg)
    say(f"[case {name}] moe_permute on oracle ids")
    buf.permute(topk_ids=i32(ref.ids))
    sync()
    p = ref.perm
    assert np.array_equal(buf.counts.cpu().numpy(), p.counts)
    assert np.array_equal(buf.offsets.cpu().numpy(), p.offsets)
    assert np.array_equal(buf.sorted_pair.cpu().numpy(), p.sorted_pair)
    assert np.array_equal(buf.pair_row.cpu().numpy(), p.pair_row)
    assert int(buf.n_active.item()) == p.n_active
    act = buf.active.cpu().numpy()
    assert np.array_equal(act[:p.n_active], p.active) and (act[p.n_active:] == -1).all()


# Seeded random routes (distinct experts per token) across the permutation
# paths: 32-token kernel, one workgroup (bitmap + prefixes up to 48 KB of
# LDS), chunked beyond it (256-token chunks: one launch up to 4 chunks, count
# + merged scan and placement up to 16, three launches beyond); the boundary
# shapes on both sides of each.
PERM_RANDOM = [(1, 10, 512), (32, 10, 512), (33, 10, 512), (384, 10, 512), (385, 10, 512),
               (1024, 10, 512), (1025, 10, 512), (2000, 10, 512), (4096, 10, 512),
               (4097, 10, 512), (192, 8, 1024), (193, 8, 1024), (700, 1, 16)]


@pytest.mark.parametrize("T,k,E", PERM_RANDOM)
def test_permute_random_routes(T, k, E):
    rng = np.random.default_rng(2000 + T + k + E)
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int64)
    p = O.permutation(ids, E)
    buf = M.MoELayerBuffers(T, 128, E, 64, k, "bf16", "dense", device=DEV)
    say(f"[permute random T={T} k={k} E={E}]")
    buf.permute(topk_ids=i32(ids))
    sync()
    assert np.array_equal(buf.counts.cpu().numpy(), p.counts)
    assert np.array_equal(buf.offsets.cpu().numpy(), p.offsets)
    assert np.array_equal(buf.sorted_pair.cpu().numpy(), p.sorted_pair)
    assert np.array_equal(buf.pair_row.cpu().numpy(), p.pair_row)
    assert int(buf.n_active.item()) == p.n_active
    act = buf.active.cpu().numpy()
    assert np.array_equal(act[:p.n_active], p.active) and (act[p.n_active:] == -1).all()


def _oracle_perm_tensors(p):
    t = [i32(p.counts), i32(p.offsets), i32(p.sorted_pair), i32(p.pair_row),
         i32(np.concatenate([p.active, -np.ones(len(p.counts) - p.n_active)])), i32([p.n_active])]
    return t, M.make_perm(*t)


@pytest.mark.parametrize("name,layout", LAYOUT_CASES)
def test_grouped_ffn(name, layout):
    case, ref = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    buf = buffers(cfg, tiled)
    keep, perm = _oracle_perm_tensors(ref.perm)
    say(f"[case {name} {layout}] moe_grouped_ffn on oracle permutation")
    buf.grouped_ffn(case.li.x, case.experts(tiled), perm=perm)
    sync()
    stats = check_values(decode(buf.y, cfg.act), ref.Y, cfg.act, "Y")
    say(f"[case {name}] Y {stats}")


@pytest.mark.parametrize("name,layout", LAYOUT_CASES)
def test_ffn_components(name, layout):
    """moe_ffn_gate_up (SwiGLU intermediate) and moe_ffn_down separately; the
    tile plan comes from moe_permute run on the oracle's ids."""
    case, ref = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    buf = buffers(cfg, tiled)
    keep, perm = _oracle_perm_tensors(ref.perm)
    say(f"[case {name} {layout}] moe_permute + moe_ffn_gate_up")
    buf.permute(topk_ids=i32(ref.ids))
    buf.ffn_gate_up(case.li.x, case.experts(tiled), perm=perm)
    sync()
    A = O.grouped_intermediate(case.x64, ref.perm, cfg.k, case.ex_oracle)
    hs = check_values(decode(buf.h, cfg.act), A, cfg.act, "h")
    Ar = O.act_round(A, cfg.act)
    say(f"[case {name} {layout}] moe_ffn_down on the oracle intermediate")
    buf.ffn_down(case.experts(tiled), h=to_act_tensor(Ar, cfg.act))
    sync()
    ys = check_values(decode(buf.y, cfg.act), O.grouped_down(Ar, ref.perm, case.ex_oracle), cfg.act, "Y")
    say(f"[case {name}] h {hs} Y {ys}")


@pytest.mark.parametrize("name", list(SMALL))
def test_combine(name):
    case, ref = get(name)
    cfg = case.cfg
    buf = buffers(cfg)
    Yr = O.act_round(ref.Y, cfg.act)
    w32 = ref.w.astype(np.float32)
    res = case.li.x if cfg.residual else None
    say(f"[case {name}] moe_combine on oracle slots")
    buf.combine(residual=res, y=to_act_tensor(Yr, cfg.act), pair_row=i32(ref.perm.pair_row),
                topk_w=torch.from_numpy(w32).to(DEV))
    sync()
    want = O.combine(Yr, ref.perm.pair_row, w32.astype(np.float64), case.x64 if cfg.residual else None)
    stats = check_values(decode(buf.out, cfg.act), want, cfg.act, "out")
    say(f"[case {name}] combine {stats}")


@pytest.mark.parametrize("name,layout", LAYOUT_CASES)
def test_layer_end_to_end(name, layout):
    case, ref = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    buf = buffers(cfg, tiled)
    res = case.li.x if cfg.residual else None
    say(f"[case {name} {layout}] moe_layer")
    buf.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(tiled), residual=res)
    sync()
    stats, same = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                               ref.logits, ref.ids, ref.w, cfg.k)
    got = decode(buf.out, cfg.act)
    vs = check_values(got[same], ref.out[same], cfg.act, "out")
    say(f"[case {name}] layer routes {stats} out {vs}")


CXX_CASES = [("tiny", None), ("decode", None), ("bf16_ragged", None), ("int4_small", None),
             ("int2_small", None), ("bf16_tiles128_ragged", None), ("verify_int2_layer0", C5)]


@pytest.mark.parametrize("name,full", CXX_CASES, ids=[n for n, _ in CXX_CASES])
def test_layer_against_cxx_oracle(name, full):
    """The whole layer (row-major and, where it applies, tiled weights)
    against the plain C++ float64 oracle: routes bit-exact except near ties,
    every output element within the output tolerance."""
    from tests.gpu_util import cxx_oracle_layer
    case = make_case(full) if full is not None else get(name)[0]
    cfg = case.cfg
    say(f"[cxx {name}] C++ oracle: {cfg}")
    ref = cxx_oracle_layer(case)
    check_oracles_agree(O.select_topk(O.router_logits(case.x64, case.wr64, case.bias64), cfg.k),
                        ref.ids, ref.logits, cfg.k)
    res = case.li.x if cfg.residual else None
    for tiled in (False, True) if tiled_ok(cfg) else (False,):
        buf = buffers(cfg, tiled)
        say(f"[cxx {name} tiled={tiled}] moe_layer")
        buf.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(tiled), residual=res)
        sync()
        stats, same = check_routes(buf.topk_ids.cpu().numpy(),
                                   buf.topk_w.cpu().numpy().astype(np.float64),
                                   ref.logits, ref.ids, ref.w, cfg.k)
        vs = check_values(decode(buf.out, cfg.act)[same], ref.out[same], cfg.act, "out")
        say(f"[cxx {name} tiled={tiled}] routes {stats} out {vs}")


@pytest.mark.parametrize("name,cfg,layer", [("prefill", C3, 0), ("stack_int4", C4, 0),
                                            ("stack_int4", C4, 47)])
def test_full_layer_sampled_against_cxx_oracle(name, cfg, layer):
    """One full-size layer (tiled weights) through moe_layer; 32 sampled
    tokens through the C++ oracle; routes bit-exact except near ties and
    those tokens' outputs within the bf16 tolerance."""
    from tests.gpu_util import cxx_oracle_layer
    case = make_case(cfg, layer=layer)
    sample = np.sort(np.random.default_rng(77 + layer).choice(cfg.T, size=32, replace=False))
    say(f"[cxx full {name} layer {layer}] C++ oracle on 32 tokens")
    ref = cxx_oracle_layer(case, sample)
    check_oracles_agree(O.select_topk(O.router_logits(case.x64[sample], case.wr64, case.bias64),
                                      cfg.k), ref.ids, ref.logits, cfg.k)
    buf = buffers(cfg, tiled_ok(cfg))
    res = case.li.x if cfg.residual else None
    say(f"[cxx full {name} layer {layer}] moe_layer")
    buf.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(tiled_ok(cfg)), residual=res)
    sync()
    stats, same = check_routes(buf.topk_ids.cpu().numpy()[sample],
                               buf.topk_w.cpu().numpy().astype(np.float64)[sample],
                               ref.logits, ref.ids, ref.w, cfg.k)
    vs = check_values(decode(buf.out, cfg.act)[sample][same], ref.out[same], cfg.act, "out")
    say(f"[cxx full {name} layer {layer}] routes {stats} out {vs}")


@pytest.mark.parametrize("tiled", [False, True], ids=["row", "tiled"])
@pytest.mark.parametrize("wfmt", ["int4_g32", "int2_g32"])
def test_lowbit_full_code_range_against_cxx_oracle(wfmt, tiled):
    """Uniformly random packed bytes, so every code occurs, including the
    most negative one (-8, -2) that the quantizer never writes but that must
    decode as q * s; random fp16 scales.  moe_layer against the C++ oracle."""
    from oracle import oracle_c as C
    T, H, E, I, k = 37, 256, 8, 128, 3
    bits = 4 if wfmt == "int4_g32" else 2
    rng = np.random.default_rng(11 + bits)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((0.02 * rng.standard_normal((E, H))).astype(np.float32)).to(torch.bfloat16)
    host = {}
    for n, (rows, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        host[n] = rng.integers(0, 256, (E, rows, K * bits // 8), dtype=np.uint8)
        host[n + "_scale"] = rng.uniform(0.002, 0.02, (E, rows, K // 32)).astype(np.float16)
    dev = {n: torch.from_numpy(a).to(DEV) for n, a in host.items()}
    ex = M.make_experts(dev["gate"], dev["up"], dev["down"], dev["gate_scale"], dev["up_scale"],
                        dev["down_scale"])
    keep = None
    if tiled:
        keep = {n: torch.empty_like(t) for n, t in dev.items()}
        ext = M.make_experts(keep["gate"], keep["up"], keep["down"], keep["gate_scale"],
                             keep["up_scale"], keep["down_scale"])
        M.moe_tile_experts(M.make_shape(T, H, E, I, k, "bf16", wfmt), ex, ext)
        ex = ext
    buf = M.MoELayerBuffers(T, H, E, I, k, "bf16", wfmt, device=DEV, tiled=tiled)
    xd, wrd = x.to(DEV), wr.to(DEV)
    say(f"[full code range {wfmt} tiled={tiled}] moe_layer")
    buf.layer(xd, wrd, None, ex)
    sync()
    st = {n: (a.view(np.uint16) if a.dtype == np.float16 else a) for n, a in host.items()}
    x64, wr64 = x.double().numpy(), wr.double().numpy()
    ref = C.moe_layer_c(x64, wr64, None, st, wfmt, "bf16", k)
    stats, same = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                               ref.logits, ref.ids, ref.w, k)
    vs = check_values(decode(buf.out, "bf16")[same], ref.out[same], "bf16", "out")
    say(f"[full code range {wfmt} tiled={tiled}] routes {stats} out {vs}")
    del keep


def test_full_prefill_routes_against_cxx_oracle():
    """Full-size prefill (4096 tokens, Zipf bias): routes and the permutation
    of the HIP path against the C++ oracle's, bit-exact except near ties
    (moe_permute is fed the oracle's ids, so the permutation is compared
    exactly)."""
    from oracle import oracle_c as C
    cfg = C3
    case = make_case(cfg)
    say("[cxx prefill routes] C++ oracle routes")
    logits, ids, w, perm = C.routes_c(case.x64, case.wr64, case.bias64, cfg.k)
    buf = buffers(cfg)
    say("[cxx prefill routes] moe_route")
    buf.route(case.li.x, case.li.w_router, case.li.bias)
    sync()
    stats, _ = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                            logits, ids, w, cfg.k)
    say(f"[cxx prefill routes] {stats}; moe_permute on the C++ oracle's ids")
    buf.permute(topk_ids=i32(ids))
    sync()
    assert np.array_equal(buf.counts.cpu().numpy(), perm.counts)
    assert np.array_equal(buf.offsets.cpu().numpy(), perm.offsets)
    assert np.array_equal(buf.sorted_pair.cpu().numpy(), perm.sorted_pair)
    assert np.array_equal(buf.pair_row.cpu().numpy(), perm.pair_row)
    assert int(buf.n_active.item()) == perm.n_active


# --------------------------------------------------------------------------
# Full-size workloads (sampled where the oracle cannot do every output)
# --------------------------------------------------------------------------

def _full_layer_check(cfg, layer, n_sample, seed):
    say(f"[full {cfg.name} layer {layer}] generate")
    case = make_case(cfg, layer=layer)
    rng = np.random.default_rng(seed)
    sample = np.sort(rng.choice(cfg.T, size=min(n_sample, cfg.T), replace=False))
    res64 = case.x64 if cfg.residual else None
    say(f"[full {cfg.name} layer {layer}] oracle (routes for all tokens, experts for {len(sample)})")
    ref = O.moe_layer(case.x64, case.wr64, case.bias64, case.ex_oracle, cfg.k, residual=res64,
                      only_tokens=sample)
    buf = buffers(cfg)
    say(f"[full {cfg.name} layer {layer}] moe_route")
    buf.route(case.li.x, case.li.w_router, case.li.bias)
    sync()
    stats, _ = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                            ref.logits, ref.ids, ref.w, cfg.k)
    say(f"[full {cfg.name} layer {layer}] routes {stats}; permute on oracle ids")
    buf.permute(topk_ids=i32(ref.ids))
    sync()
    assert np.array_equal(buf.sorted_pair.cpu().numpy(), ref.perm.sorted_pair)
    assert np.array_equal(buf.pair_row.cpu().numpy(), ref.perm.pair_row)
    assert np.array_equal(buf.counts.cpu().numpy(), ref.perm.counts)
    keep, perm = _oracle_perm_tensors(ref.perm)
    rows = ref.perm.pair_row[(sample[:, None] * cfg.k + np.arange(cfg.k)).reshape(-1)]
    res = case.li.x if cfg.residual else None
    for tiled, fused in ((False, False), (True, False), (True, True)):
        if fused and cfg.T * cfg.k > 16384:
            continue
        b2 = buffers(cfg, tiled, fused)
        say(f"[full {cfg.name} layer {layer} tiled={tiled} fused={fused}] ffn on oracle permutation")
        if fused:
            b2.ffn_fused(case.li.x, case.experts(tiled), perm=perm)
        else:
            b2.grouped_ffn(case.li.x, case.experts(tiled), perm=perm)
        sync()
        yv = check_values(decode(b2.y, cfg.act)[rows], ref.Y[rows], cfg.act, "Y")
        say(f"[full {cfg.name} layer {layer} tiled={tiled} fused={fused}] Y {yv}; moe_layer")
        b2.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(tiled), residual=res)
        sync()
        ids = b2.topk_ids.cpu().numpy()
        same = (ids[sample] == ref.ids[sample]).all(axis=1)
        near = O.near_tie_tokens(ref.logits[sample], cfg.k)
        assert (same | near).all()
        got = decode(b2.out, cfg.act)[sample]
        ov = check_values(got[same], ref.out[sample][same], cfg.act, "out")
    ua = int(ref.perm.n_active)
    say(f"[full {cfg.name} layer {layer}] out {ov}; unique experts {ua}; "
        f"repeat fraction {O.repeat_fraction(ref.ids):.3f}; max load {ref.perm.counts.max()}")
    return ref


def test_full_decode():
    _full_layer_check(C2, 0, 8, 0)


def test_full_prefill():
    ref = _full_layer_check(C3, 0, 12, 1)
    c = ref.perm.counts
    assert c.max() > 10 * c[c > 0].mean()          # Zipf bias skews loads as specified


def test_full_prefill_merged():
    """Eight 4096-token windows in one call (T = 32768), the shape where the
    grouped GEMMs pass the bf16 ridge; routes for all tokens, outputs for a
    sample."""
    ref = _full_layer_check(C3.with_(name="prefill_merged", T=32768), 0, 8, 5)
    assert int(ref.perm.n_active) == C3.E or ref.perm.counts.max() > 100


@pytest.mark.parametrize("layer", [0, 47])
def test_full_stack_int4_layer(layer):
    _full_layer_check(C4, layer, 12, 2 + layer)


@pytest.mark.parametrize("layer", [0, 47])
def test_full_verify_int2_layer(layer):
    ref = _full_layer_check(C5, layer, 16, 3 + layer)
    assert O.repeat_fraction(ref.ids) > 0.5


def test_stack_teacher_forced_int2():
    """Layers 0..2 of the int2 verifier stack: the oracle runs the chain
    x_{l+1} = bf16(x_l + moe_l(x_l)); the GPU layer l is fed the oracle's x_l
    and must reproduce the oracle's x_{l+1}."""
    cfg = C5
    say("[stack int2] generate 3 layers")
    cases = [make_case(cfg, layer=l) for l in range(3)]
    xs = O.moe_stack(cases[0].x64, [(lambda c=c: (c.wr64, c.bias64, c.ex_oracle)) for c in cases],
                     cfg.k, cfg.act)
    buf = buffers(cfg, tiled=True)
    for l, c in enumerate(cases):
        x_l = to_act_tensor(xs[l], cfg.act)
        say(f"[stack int2] layer {l}")
        buf.layer(x_l, c.li.w_router, c.li.bias, c.ex_gpu_tiled, residual=x_l)
        sync()
        ref_r = O.moe_layer(xs[l], c.wr64, c.bias64, c.ex_oracle, cfg.k, residual=xs[l])
        stats, same = check_routes(buf.topk_ids.cpu().numpy(),
                                   buf.topk_w.cpu().numpy().astype(np.float64), ref_r.logits,
                                   ref_r.ids, ref_r.w, cfg.k)
        got = decode(buf.out, cfg.act)
        check_values(got[same], xs[l + 1][same], cfg.act, f"x_{l + 1}")


# --------------------------------------------------------------------------
# Properties and edge cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,layout", [("decode", "row"), ("decode", "tiled"),
                                         ("bf16_tiles128", "tiled"), ("int4_many_rows", "tiled"),
                                         ("int2_small", "tiled")])
def test_determinism_three_runs(name, layout):
    """Bitwise-identical outputs, routes and permutation over three runs
    (each kernel family: small tiles, 64-row low-bit tiles, 128-row tiles)."""
    case, _ = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    outs = []
    for i in range(3):
        buf = buffers(cfg, tiled)
        say(f"[determinism {name} {layout}] run {i}")
        buf.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(tiled))
        sync()
        outs.append((buf.out.view(torch.int16).cpu().numpy(), buf.topk_ids.cpu().numpy(),
                     buf.topk_w.cpu().numpy(), buf.sorted_pair.cpu().numpy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["prefill_chunked", "int4_small", "tiny"])
def test_fused_equals_staged(name):
    case, _ = get(name)
    cfg = case.cfg
    res = case.li.x if cfg.residual else None
    a, b = buffers(cfg), buffers(cfg)
    say(f"[fused==staged {name}]")
    a.layer(case.li.x, case.li.w_router, case.li.bias, case.ex_gpu, residual=res)
    b.route(case.li.x, case.li.w_router, case.li.bias)
    b.permute()
    b.grouped_ffn(case.li.x, case.ex_gpu)
    b.combine(residual=res)
    sync()
    for name_ in ("out", "topk_ids", "topk_w", "sorted_pair", "pair_row", "counts"):
        ta, tb = getattr(a, name_), getattr(b, name_)
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), name_


PERM_NAMES = ("counts", "offsets", "sorted_pair", "pair_row", "active", "n_active")


@pytest.mark.parametrize("name", ["bf16_ragged", "int4_small", "decode"])
def test_check_finite_clean_equals_unchecked(name):
    """MOE_F_CHECK_FINITE on finite inputs: same bits as without the flag."""
    case, _ = get(name)
    cfg = case.cfg
    res = case.li.x if cfg.residual else None
    a, b = buffers(cfg), M.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt,
                                           device=DEV, check_finite=True)
    say(f"[check_finite clean {name}]")
    a.layer(case.li.x, case.li.w_router, case.li.bias, case.ex_gpu, residual=res)
    b.layer(case.li.x, case.li.w_router, case.li.bias, case.ex_gpu, residual=res)
    sync()
    for n in ("out", "topk_ids", "topk_w") + PERM_NAMES:
        ta, tb = getattr(a, n), getattr(b, n)
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), n
    a.route(case.li.x, case.li.w_router, case.li.bias)
    b.route(case.li.x, case.li.w_router, case.li.bias)
    sync()
    for n in ("topk_ids", "topk_w", "logits"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n


@pytest.mark.parametrize("where", ["x_nan", "x_inf", "router_nan", "expert_inf"])
def test_check_finite_rejects_and_publishes_nothing(where):
    """A NaN or infinity anywhere on the path returns MOE_E_NONFINITE and
    leaves every caller output at its sentinel (the fail-closed publication
    rule)."""
    cfg = SMALL["bf16_ragged"]
    case = make_case(cfg)
    x, wr = case.li.x.clone(), case.li.w_router.clone()
    ex = {n: (None if t is None else t.clone()) for n, t in case.li.experts.items()}
    if where == "x_nan":
        x[3, 17] = float("nan")
    elif where == "x_inf":
        x[0, 0] = float("inf")
    elif where == "router_nan":
        wr[5, 100] = float("nan")
    else:
        probe = buffers(cfg)
        probe.route(x, wr, case.li.bias)
        sync()
        e0 = int(probe.topk_ids[0, 0].item())
        ex["gate"][e0, :, :] = float("inf")                  # every row of a selected expert
    exg = M.make_experts(ex["gate"], ex["up"], ex["down"])
    b = M.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt, device=DEV,
                          check_finite=True)
    sentinels = {"out": 7.0, "topk_ids": -5, "topk_w": 3.0, "logits": 9.0}
    for n in PERM_NAMES:
        sentinels[n] = -7
    for n, v in sentinels.items():
        getattr(b, n).fill_(v)
    sync()
    say(f"[check_finite reject {where}] moe_layer")
    with pytest.raises(M.MoEError) as err:
        b.layer(x, wr, case.li.bias, exg)
    assert err.value.status == 11
    if where != "expert_inf":
        say(f"[check_finite reject {where}] moe_route")
        with pytest.raises(M.MoEError) as err:
            b.route(x, wr, case.li.bias)
        assert err.value.status == 11
    sync()
    for n, v in sentinels.items():
        t = getattr(b, n)
        assert bool((t == v).all()), f"{n} was written"


def test_batch_partition_invariance():
    """Routes of 512 tokens in one call equal those of 8 calls of 64 tokens
    (the replay/decode route-parity requirement), bit for bit."""
    cfg = C3.with_(T=512)
    case = make_case(cfg)
    whole = buffers(cfg)
    say("[partition] whole batch")
    whole.route(case.li.x, case.li.w_router, case.li.bias)
    part = buffers(cfg.with_(T=64))
    for i in range(8):
        say(f"[partition] part {i}")
        part.route(case.li.x[64 * i:64 * (i + 1)].contiguous(), case.li.w_router, case.li.bias)
        sync()
        assert torch.equal(part.topk_ids, whole.topk_ids[64 * i:64 * (i + 1)])
        assert torch.equal(part.topk_w, whole.topk_w[64 * i:64 * (i + 1)])
        assert torch.equal(part.logits, whole.logits[64 * i:64 * (i + 1)])


def _small_dense(T=24, H=256, E=16, I=64, k=4):
    return C2.with_(T=T, H=H, E=E, I=I, k=k)


def test_zero_router_exact_ties():
    cfg = _small_dense()
    case = make_case(cfg)
    buf = buffers(cfg)
    say("[ties] zero router")
    buf.route(case.li.x, torch.zeros_like(case.li.w_router), None)
    sync()
    assert (buf.topk_ids.cpu().numpy() == np.arange(cfg.k)).all()
    assert np.allclose(buf.topk_w.cpu().numpy(), 1.0 / cfg.k, atol=1e-7)


def test_duplicate_router_rows_lower_index_first():
    cfg = _small_dense()
    case = make_case(cfg)
    wr = case.li.w_router.clone()
    wr[9] = wr[3]
    bias = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
    bias[3] = bias[9] = 50.0
    buf = buffers(cfg)
    say("[ties] duplicate rows")
    buf.route(case.li.x, wr, bias)
    sync()
    ids = buf.topk_ids.cpu().numpy()
    assert (ids[:, 0] == 3).all() and (ids[:, 1] == 9).all()


def test_forced_routes_by_bias():
    cfg = _small_dense(E=40, k=5)
    case = make_case(cfg)
    order = [17, 2, 33, 8, 25]
    bias = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
    for j, e in enumerate(order):
        bias[e] = 100.0 - 10 * j
    buf = buffers(cfg)
    say("[forced routes]")
    buf.layer(case.li.x, case.li.w_router, bias, case.ex_gpu)
    sync()
    assert (buf.topk_ids.cpu().numpy() == np.array(order)).all()
    assert int(buf.n_active.item()) == 5
    ref = O.moe_layer(case.x64, case.wr64, bias.double().cpu().numpy(), case.ex_oracle, cfg.k)
    check_values(decode(buf.out, cfg.act), ref.out, cfg.act, "out")


def test_k_equals_E():
    cfg = _small_dense(T=9, E=16, k=16)
    case = make_case(cfg)
    ref = O.moe_layer(case.x64, case.wr64, None, case.ex_oracle, cfg.k)
    buf = buffers(cfg)
    say("[k == E]")
    buf.layer(case.li.x, case.li.w_router, None, case.ex_gpu)
    sync()
    check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                 ref.logits, ref.ids, ref.w, cfg.k)
    check_values(decode(buf.out, cfg.act), ref.out, cfg.act, "out")


@pytest.mark.parametrize("T", [1, 2, 31, 33])
def test_small_T(T):
    cfg = C2.with_(T=T, H=512, E=64, I=128, k=6)
    case = make_case(cfg)
    ref = O.moe_layer(case.x64, case.wr64, None, case.ex_oracle, cfg.k)
    buf = buffers(cfg)
    say(f"[small T={T}]")
    buf.layer(case.li.x, case.li.w_router, None, case.ex_gpu)
    sync()
    _, same = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                           ref.logits, ref.ids, ref.w, cfg.k)
    check_values(decode(buf.out, cfg.act)[same], ref.out[same], cfg.act, "out")


def test_hot_experts_many_tiles():
    """Every token picks the same k experts: each has T rows, split into many
    tiles, and every tile must read the right rows."""
    cfg = C2.with_(T=300, H=256, E=32, I=64, k=3)
    case = make_case(cfg)
    bias = torch.zeros(cfg.E, dtype=torch.float32, device=DEV)
    bias[[5, 6, 7]] = torch.tensor([60.0, 50.0, 40.0], device=DEV)
    ref = O.moe_layer(case.x64, case.wr64, bias.double().cpu().numpy(), case.ex_oracle, cfg.k)
    buf = buffers(cfg)
    say("[hot experts]")
    buf.layer(case.li.x, case.li.w_router, bias, case.ex_gpu)
    sync()
    assert (buf.counts.cpu().numpy()[[5, 6, 7]] == 300).all()
    check_values(decode(buf.out, cfg.act), ref.out, cfg.act, "out")


@pytest.mark.parametrize("T", [24, 40])   # 32-token permutation path and the general one
def test_max_experts(T):
    cfg = C2.with_(T=T, H=256, E=1024, I=64, k=32)
    case = make_case(cfg)
    ref = O.moe_layer(case.x64, case.wr64, None, case.ex_oracle, cfg.k)
    buf = buffers(cfg)
    say(f"[E=1024, k=32, T={T}]")
    buf.layer(case.li.x, case.li.w_router, None, case.ex_gpu)
    sync()
    _, same = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                           ref.logits, ref.ids, ref.w, cfg.k)
    check_values(decode(buf.out, cfg.act)[same], ref.out[same], cfg.act, "out")


def test_t_zero_noop():
    cfg = C2.with_(T=0)
    s = M.make_shape(0, cfg.H, cfg.E, cfg.I, cfg.k)
    assert M.moe_layer(s, None, None, None, None, None, None, None, None, None, None, 0) == 0


@pytest.mark.parametrize("wfmt", ["dense", "int4_g32", "int2_g32"])
def test_tile_layout_bit_exact(wfmt):
    """moe_tile_experts against the layout formula of include/moe.h,
    evaluated with numpy reshapes."""
    cfg = C4.with_(T=8, H=512, E=3, I=256, k=2, wfmt=wfmt)
    case = make_case(cfg)
    say(f"[tile layout {wfmt}]")
    sync()
    src, dst = case.li.experts, case.tiled_keep

    def int4_words(v):
        """each 4-byte piece (natural nibble order c0..c7, two's complement)
        -> one word: c_2m at nibble m, c_2m+1 at nibble m+4, offset binary"""
        d = np.ascontiguousarray(v).reshape(-1, 4).copy().view(np.uint32).reshape(-1).astype(np.uint64)
        out = np.zeros_like(d)
        for m in range(4):
            out |= ((d >> (8 * m)) & 0xF) << (4 * m)
            out |= ((d >> (8 * m + 4)) & 0xF) << (4 * (m + 4))
        return (out.astype(np.uint32) ^ np.uint32(0x88888888)).view(np.uint8)

    def int2_words(v):
        """pieces of 2 bytes (c_j at bits 2j, two's complement), 4 per lane
        unit -> 2 words: piece 2w+sub's c_2m at bits 8 sub + 2m and c_2m+1 at
        bits 16 + 8 sub + 2m of word w, offset binary"""
        p = np.ascontiguousarray(v).reshape(-1, 2, 2, 2).copy().view(np.uint16)[..., 0].astype(np.uint64)
        out = np.zeros(p.shape[:2], dtype=np.uint64)               # [units, w]
        for sub in range(2):
            for m in range(4):
                out |= ((p[:, :, sub] >> (4 * m)) & 3) << (8 * sub + 2 * m)
                out |= ((p[:, :, sub] >> (4 * m + 2)) & 3) << (16 + 8 * sub + 2 * m)
        return (out.astype(np.uint32) ^ np.uint32(0xAAAAAAAA)).reshape(-1).view(np.uint8)

    def arrange(a, N, K):
        if wfmt == "dense":                                   # [E*N][K] elements
            v = a.reshape(-1, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4)
            return np.ascontiguousarray(v).reshape(-1)
        B = 4 if wfmt == "int4_g32" else 2                    # bytes per 8 codes
        v = np.ascontiguousarray(a.reshape(-1, 16, K // 128, 4, 4, B).transpose(0, 2, 4, 1, 3, 5))
        return int4_words(v) if wfmt == "int4_g32" else int2_words(v)

    def arrange_scales(a, K):
        v = a.reshape(-1, 16, K // 128, 4).transpose(0, 2, 1, 3)
        return np.ascontiguousarray(v).reshape(-1)

    for name, N, K in (("gate", cfg.I, cfg.H), ("up", cfg.I, cfg.H), ("down", cfg.H, cfg.I)):
        a = np_of(src[name])
        got = np_of(dst[name]).reshape(-1)
        assert np.array_equal(got, arrange(a.reshape(a.shape[0] * a.shape[1], -1), N, K)), name
        if wfmt != "dense":
            sa = np_of(src[name + "_scale"])
            sg = np_of(dst[name + "_scale"]).reshape(-1)
            assert np.array_equal(sg, arrange_scales(sa.reshape(-1, K // 32), K)), name + " scales"


def test_stream_read_probe():
    """The read-bandwidth probe runs and leaves its sink alone on zero data
    (the fold of zeros never equals the magic value)."""
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    assert M.moe_stream_read(buf, buf.numel(), sink) == 0
    sync()
    assert int(sink.item()) == 5


def _locality_check(ids_np, E):
    T, k = ids_np.shape
    buf = M.MoELayerBuffers(T, 256, E, 64, k, "bf16", "dense", device=DEV)
    ov, blocks = buf.route_locality(topk_ids=i32(ids_np))
    sync()
    assert np.array_equal(ov.cpu().numpy(), O.overlap_with_previous(ids_np))
    for B in range(1, 6):
        assert np.array_equal(blocks[B - 1].cpu().numpy(), O.block_unique(ids_np, B)), B


@pytest.mark.parametrize("T,k,E", [(1, 10, 512), (2, 10, 512), (13, 10, 512), (37, 7, 100),
                                   (200, 32, 1024), (64, 1, 3), (300, 10, 16)])
def test_route_locality_random(T, k, E):
    """Seeded random routes with distinct experts per token, bit-exact."""
    rng = np.random.default_rng(1000 + T + k)
    ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], dtype=np.int32)
    say(f"[locality T={T} k={k} E={E}]")
    _locality_check(ids, E)


@pytest.mark.parametrize("name", ["decode", "int2_small", "prefill_chunked"])
def test_route_locality_oracle_routes(name):
    """The oracle's routes of a workload fed to the kernel (teacher forcing)."""
    case, ref = get(name)
    say(f"[locality {name}] oracle routes")
    _locality_check(ref.ids.astype(np.int32), case.cfg.E)


@pytest.mark.parametrize("name,layout", [("decode", "tiled"), ("int4_small", "tiled"),
                                         ("prefill_chunked", "row")])
def test_layer_hip_graph_replay(name, layout):
    """The staged layer (route, permute, gate/up, down, combine) captured in a
    HIP graph: every replay, with eager work and synchronizations between
    replays, equals the eager result bit for bit (no memset nodes)."""
    case, _ = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    res = case.li.x if cfg.residual else None
    ex = case.experts(tiled)
    eager = buffers(cfg, tiled)
    eager.route(case.li.x, case.li.w_router, case.li.bias)
    eager.permute()
    eager.ffn_gate_up(case.li.x, ex)
    eager.ffn_down(ex)
    eager.combine(residual=res)
    sync()
    g_buf = buffers(cfg, tiled)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    say(f"[graph {name} {layout}] capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            g_buf.route(case.li.x, case.li.w_router, case.li.bias, stream=s)
            g_buf.permute(stream=s)
            g_buf.ffn_gate_up(case.li.x, ex, stream=s)
            g_buf.ffn_down(ex, stream=s)
            g_buf.combine(residual=res, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    sync()
    for rep in range(4):
        g_buf.out.fill_(0)
        g_buf.topk_ids.fill_(-1)
        junk = torch.randn(1 << 20, device=DEV).sum()           # eager work between replays
        sync()
        graph.replay()
        sync()
        say(f"[graph {name} {layout}] replay {rep}")
        assert torch.equal(g_buf.out.view(torch.int16) if g_buf.out.dtype == torch.bfloat16
                           else g_buf.out, eager.out.view(torch.int16)
                           if eager.out.dtype == torch.bfloat16 else eager.out)
        assert torch.equal(g_buf.topk_ids, eager.topk_ids)
        assert torch.equal(g_buf.sorted_pair, eager.sorted_pair)
        del junk


STAGE_CASES = [("int4_small", "tiled", "pinned", False), ("int2_small", "tiled", "pinned", True),
               ("bf16_ragged", "row", "pinned", True), ("int4_many_rows", "row", "device", False)]
EXPERT_PIECES = ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")


@pytest.mark.parametrize("name,layout,where,split", STAGE_CASES)
def test_stage_experts(name, layout, where, split):
    """moe_stage_experts copies exactly the active experts' records (from
    pinned host or device memory), leaves every other expert's region as it
    was, and the layer run on the staged records equals the layer run on the
    resident ones bit for bit.  With `split`, gate/up is staged first (down
    regions still untouched) and down on a second stream while gate/up runs."""
    case, _ = get(name)
    cfg = case.cfg
    tiled = layout == "tiled"
    src_t = case.tiled_keep if tiled else case.li.experts
    src_t = {n: (None if src_t.get(n) is None else
                 (src_t[n].cpu().pin_memory() if where == "pinned" else src_t[n].clone()))
             for n in EXPERT_PIECES}
    dst_t = {n: (None if t is None else torch.empty_like(t, device=DEV)) for n, t in src_t.items()}
    for t in dst_t.values():
        if t is not None:
            t.view(torch.uint8).fill_(0x5A)
    src = M.make_experts(*(src_t[n] for n in EXPERT_PIECES))
    dst = M.make_experts(*(dst_t[n] for n in EXPERT_PIECES))
    ex = case.experts(tiled)
    res = case.li.x if cfg.residual else None
    b = buffers(cfg, tiled)
    b.route(case.li.x, case.li.w_router, case.li.bias)
    b.permute()
    say(f"[stage {name} {layout} {where} split={split}] stage")
    if split:
        b.stage_experts(src, dst, parts=M.MOE_STAGE_GATE_UP)
        sync()
        for n in ("down", "down_scale"):
            if dst_t[n] is not None:
                assert bool((dst_t[n].view(torch.uint8) == 0x5A).all()), f"{n} written by gate/up stage"
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        b.stage_experts(src, dst, parts=M.MOE_STAGE_DOWN, stream=side)
    else:
        b.stage_experts(src, dst)
    sync()
    n_act = int(b.n_active.item())
    active = set(b.active[:n_act].cpu().tolist())
    assert active == set(np.nonzero(b.counts.cpu().numpy())[0].tolist())
    for n in EXPERT_PIECES:
        if src_t[n] is None:
            continue
        s8 = src_t[n].view(torch.uint8).reshape(cfg.E, -1).cpu()
        d8 = dst_t[n].view(torch.uint8).reshape(cfg.E, -1).cpu()
        for e in range(cfg.E):
            if e in active:
                assert torch.equal(d8[e], s8[e]), f"{n}: expert {e} not copied"
            else:
                assert bool((d8[e] == 0x5A).all()), f"{n}: inactive expert {e} written"
    say(f"[stage {name} {layout} {where} split={split}] layer on staged records")
    b.ffn_gate_up(case.li.x, dst)
    b.ffn_down(dst)
    b.combine(residual=res)
    staged = b.out.clone()
    b.ffn_gate_up(case.li.x, ex)
    b.ffn_down(ex)
    b.combine(residual=res)
    sync()
    assert torch.equal(staged.view(torch.int16), b.out.view(torch.int16))


def test_stage_experts_none_active_and_pageable():
    """n_active = 0 writes nothing; pageable host memory is rejected with
    MOE_E_MEMORY before any launch."""
    case, _ = get("int4_small")
    cfg = case.cfg
    src_t = {n: case.li.experts.get(n) for n in EXPERT_PIECES}
    dst_t = {n: (None if t is None else torch.empty_like(t)) for n, t in src_t.items()}
    for t in dst_t.values():
        if t is not None:
            t.view(torch.uint8).fill_(0x5A)
    b = buffers(cfg)
    b.route(case.li.x, case.li.w_router, case.li.bias)
    b.permute()
    b.n_active.fill_(0)
    dst = M.make_experts(*(dst_t[n] for n in EXPERT_PIECES))
    b.stage_experts(M.make_experts(*(src_t[n] for n in EXPERT_PIECES)), dst)
    sync()
    assert all(bool((t.view(torch.uint8) == 0x5A).all()) for t in dst_t.values() if t is not None)
    pageable = {n: (None if t is None else t.cpu()) for n, t in src_t.items()}
    st = M.moe_stage_experts(b.shape, M.make_experts(*(pageable[n] for n in EXPERT_PIECES)), dst,
                             b.perm, check=False)
    assert st == 12


# --------------------------------------------------------------------------
# Fused gate/up -> down component waves (moe_ffn_fused, MOE_F_FUSED_FFN)
# --------------------------------------------------------------------------

FUSED_CASES = [n for n in SMALL if tiled_ok(SMALL[n]) and SMALL[n].T * SMALL[n].k <= 16384]


@pytest.mark.parametrize("name", FUSED_CASES)
@pytest.mark.parametrize("wave", [0, 1, 2, 4])
def test_ffn_fused(name, wave):
    """moe_ffn_fused on the oracle permutation against the oracle's expert
    outputs, for waves of 1, 2, 4 and all tiles."""
    case, ref = get(name)
    cfg = case.cfg
    buf = buffers(cfg, tiled=True, fused=True)
    keep, perm = _oracle_perm_tensors(ref.perm)
    say(f"[fused {name} wave={wave}] moe_ffn_fused on oracle permutation")
    buf.ffn_fused(case.li.x, case.experts(True), wave_tiles=wave, perm=perm)
    sync()
    stats = check_values(decode(buf.y, cfg.act), ref.Y, cfg.act, "Y")
    say(f"[fused {name} wave={wave}] Y {stats}")


@pytest.mark.parametrize("name", FUSED_CASES)
def test_layer_fused(name):
    """moe_layer with MOE_F_FUSED_FFN (fused FFN + combine of the partial
    results) against the oracle layer."""
    case, ref = get(name)
    cfg = case.cfg
    buf = buffers(cfg, tiled=True, fused=True)
    res = case.li.x if cfg.residual else None
    say(f"[fused {name}] moe_layer")
    buf.layer(case.li.x, case.li.w_router, case.li.bias, case.experts(True), residual=res)
    sync()
    stats, same = check_routes(buf.topk_ids.cpu().numpy(), buf.topk_w.cpu().numpy().astype(np.float64),
                               ref.logits, ref.ids, ref.w, cfg.k)
    vs = check_values(decode(buf.out, cfg.act)[same], ref.out[same], cfg.act, "out")
    say(f"[fused {name}] layer routes {stats} out {vs}")


@pytest.mark.parametrize("wave", [0, 2])
def test_fused_item_clock(wave):
    """Item clock of moe_ffn_fused: for every item of the plan start <=
    gate/up done <= down done; entries past the last item stay untouched."""
    case, ref = get("int4_small")
    cfg = case.cfg
    buf = buffers(cfg, tiled=True, fused=True)
    keep, perm = _oracle_perm_tensors(ref.perm)
    cap = M.moe_ffn_fused_items(buf.shape)
    clock = torch.full((3 * cap,), -1, dtype=torch.int64, device=DEV)
    buf.ffn_fused(case.li.x, case.experts(True), wave_tiles=wave, item_clock=clock, perm=perm)
    sync()
    rt = 16 * (1 if cfg.T <= 16 or cfg.T * cfg.k <= 12 * cfg.E else (2 if cfg.T <= 1024 else 4))
    counts = ref.perm.counts
    n_tiles = int(sum((c + rt - 1) // rt for c in counts if c > 0))
    n_items = n_tiles * (cfg.I // 64)
    c = clock.view(-1, 3).cpu().numpy()
    assert (c[:n_items] > 0).all()
    assert (c[:n_items, 0] <= c[:n_items, 1]).all() and (c[:n_items, 1] <= c[:n_items, 2]).all()
    assert (c[n_items:] == -1).all()
    assert M.moe_device_clock_khz() > 0
