"""The two combined component calls against the calls they combine, through
the C ABI, bit for bit:

  moe_route_permute    == moe_route + moe_permute      (ids, weights, logits,
                                                        permutation, and the
                                                        tile plan, through the
                                                        FFN that reads it)
  moe_ffn_down_combine == moe_ffn_down + moe_combine   (layer output)

on both sides of the size limits of the single-launch paths (up to 32
tokens, bf16, tiled weights with 16-row tiles), with and without a residual,
for every weight format, and on repeated calls that reuse one workspace (the
tile plan must be rewritten in full each time).  Parity of the layer
against the oracle on these paths is covered by the moe_layer tests, which
run them."""
import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from moe_inputs import CONFIGS, make_x
from tests.gpu_util import DEV, buffers, make_case, say

pytestmark = pytest.mark.gpu

C1, C2, C3, C4, C5 = (CONFIGS[i] for i in range(1, 6))

CASES = {
    "decode": C2,                                                         # fused, full size
    "decode_T1": C2.with_(T=1, H=1024, E=128, I=256),
    "decode_T32": C2.with_(T=32, H=1024, E=128, I=256),                   # fused limit
    "decode_T33": C2.with_(T=33, H=1024, E=128, I=256),                   # two launches
    "verify_int2": C5.with_(H=1024, E=96, I=256, layers=1),               # residual, int2
    "int4_T5": C4.with_(T=5, H=512, E=64, I=128, k=8, layers=1),
    "ragged_E": C2.with_(T=19, H=384, E=100, I=128, k=7),
    "E1024_k32": C2.with_(T=24, H=256, E=1024, I=128, k=32),
    "k80": C2.with_(T=4, H=256, E=96, I=128, k=80),                      # top-k past 64: three launches
    "hot_bf16_T32": C5.with_(T=32, H=1024, E=96, I=256, wfmt="dense", layers=1),  # 2-tile experts
    "pairs_510": C2.with_(T=51, H=512, E=256, I=128),                     # 16-row tiles, many experts
    "prefill_small": C3.with_(T=200, H=256, I=128),                      # two launches
    "tiny_f32": C1,                                                       # float32: two launches
}


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _equal(a, b):
    return torch.equal(_bits(a), _bits(b))


@pytest.mark.parametrize("name", list(CASES))
def test_route_permute_equals_route_then_permute(name):
    cfg = CASES[name]
    case = make_case(cfg)
    tiled = case.ex_gpu_tiled is not None
    a, b = buffers(cfg, tiled), buffers(cfg, tiled)
    say(f"[{name}] moe_route + moe_permute vs moe_route_permute (tiled={tiled})")
    a.route(case.li.x, case.li.w_router, case.li.bias)
    a.permute()
    for rep in range(2):     # the second call reuses the workspace
        for t in (b.topk_ids, b.counts, b.offsets, b.sorted_pair, b.pair_row, b.active, b.n_active):
            t.fill_(-7)
        b.route_permute(case.li.x, case.li.w_router, case.li.bias)
        torch.cuda.synchronize()
        for key in ("topk_ids", "topk_w", "logits", "counts", "offsets", "sorted_pair", "pair_row",
                    "active", "n_active"):
            assert _equal(getattr(a, key), getattr(b, key)), f"{name} call {rep}: {key}"
    # the tile plan each left in its workspace drives the same expert outputs
    ex = case.experts(tiled)
    for buf in (a, b):
        buf.ffn_gate_up(case.li.x, ex)
        buf.ffn_down(ex)
    torch.cuda.synchronize()
    assert _equal(a.h, b.h) and _equal(a.y, b.y)


@pytest.mark.parametrize("name", list(CASES))
def test_down_combine_equals_down_then_combine(name):
    cfg = CASES[name]
    case = make_case(cfg)
    tiled = case.ex_gpu_tiled is not None
    ex = case.experts(tiled)
    buf = buffers(cfg, tiled)
    say(f"[{name}] moe_ffn_down + moe_combine vs moe_ffn_down_combine (tiled={tiled})")
    buf.route(case.li.x, case.li.w_router, case.li.bias)
    buf.permute()
    buf.ffn_gate_up(case.li.x, ex)
    for residual in (None, case.li.x):
        buf.ffn_down(ex)
        ref = torch.empty_like(buf.out)
        buf.combine(residual=residual, out=ref)
        for rep in range(3):     # repeated calls on one workspace
            out = torch.full_like(buf.out, float("nan"))
            buf.ffn_down_combine(ex, residual=residual, out=out)
            torch.cuda.synchronize()
            assert _equal(ref, out), f"{name} residual={residual is not None} call {rep}"
    assert torch.isfinite(ref.float()).all()


def test_layer_sequence_reuses_workspace():
    """A 6-layer chain through moe_layer (single-launch routing and
    down + combine) on one workspace, new weights every layer, against the
    five separate calls on another."""
    cfg = C5.with_(T=16, H=512, E=64, I=128, layers=6)
    tiled_bufs = [buffers(cfg, True), buffers(cfg, True)]
    x = make_x(cfg, DEV)
    xa, xb = x.clone(), x.clone()
    for l in range(cfg.layers):
        case = make_case(cfg, layer=l, x=xa)
        ex = case.experts(True)
        a, b = tiled_bufs
        oa = torch.empty_like(xa)
        a.layer(xa, case.li.w_router, case.li.bias, ex, residual=xa, out=oa)
        ob = torch.empty_like(xb)
        b.route(xb, case.li.w_router, case.li.bias, logits=False)
        b.permute()
        b.ffn_gate_up(xb, ex)
        b.ffn_down(ex)
        b.combine(residual=xb, out=ob)
        torch.cuda.synchronize()
        assert _equal(oa, ob), f"layer {l}"
        assert np.isfinite(oa.float().cpu().numpy()).all()
        xa, xb = oa, ob
