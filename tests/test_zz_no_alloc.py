"""moe_layer_noalloc (the layer entry point that allocates nothing; its
scratch is a fixed device array inside the library) against moe_layer with a
caller workspace, through the C ABI.  Two calls in a row on the same device
array, the second with fewer tokens, so the second call runs on scratch that
still holds the first call's contents.  The two entry points run the same
kernels on the same inputs, so routes, permutation and output must agree bit
for bit (stricter than the oracle tolerance)."""
import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from moe_inputs import CONFIGS, make_layer, make_x
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu

C2, C5 = CONFIGS[2], CONFIGS[5]
# (name, layer shape, token counts of the two calls, tiled weights)
CASES = [
    ("bf16_tiled", C2.with_(name="noalloc_bf16", H=1024, E=128, I=256, k=8), (300, 9), True),
    ("int2_residual", C5.with_(name="noalloc_int2", H=1024, E=96, I=256, layers=1), (40, 3), True),
    ("bf16_row", C2.with_(name="noalloc_row", H=512, E=64, I=128, k=6), (70, 1), False),
    ("decode_full", C2, (8, 5), True),
]


def _experts(cfg, tiled):
    li = make_layer(cfg, device=DEV, with_x=False)
    ex = li.experts
    mk = lambda d: M.make_experts(d["gate"], d["up"], d["down"], d["gate_scale"], d["up_scale"],
                                  d["down_scale"])
    keep = [ex]
    exs = mk(ex)
    if tiled:
        dst = {n: (None if t is None else torch.empty_like(t)) for n, t in ex.items()}
        M.moe_tile_experts(M.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt),
                           exs, mk(dst))
        keep.append(dst)
        exs = mk(dst)
    return li, exs, keep


def _outputs(cfg, T, tiled):
    flags = M.MOE_F_TILED_WEIGHTS if tiled else 0
    shape = M.make_shape(T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt, flags)
    P = T * cfg.k
    i32 = dict(dtype=torch.int32, device=DEV)
    o = {"out": torch.full((T, cfg.H), float("nan"), dtype=torch.bfloat16, device=DEV),
         "ids": torch.full((T, cfg.k), -7, **i32),
         "w": torch.full((T, cfg.k), -1.0, dtype=torch.float32, device=DEV),
         "counts": torch.full((cfg.E,), -7, **i32), "offsets": torch.full((cfg.E + 1,), -7, **i32),
         "sorted_pair": torch.full((P,), -7, **i32), "pair_row": torch.full((P,), -7, **i32),
         "active": torch.full((cfg.E,), -7, **i32), "n_active": torch.full((1,), -7, **i32)}
    perm = M.make_perm(o["counts"], o["offsets"], o["sorted_pair"], o["pair_row"], o["active"],
                       o["n_active"])
    return shape, o, perm


@pytest.mark.parametrize("name,cfg,Ts,tiled", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_moe_layer(name, cfg, Ts, tiled):
    say(f"noalloc {name}: T={Ts} H={cfg.H} E={cfg.E} I={cfg.I} k={cfg.k} {cfg.wfmt} tiled={tiled}")
    li, exs, _keep = _experts(cfg, tiled)
    for call, T in enumerate(Ts):
        x = make_x(cfg, DEV, batch=call, T=T)
        res = x if cfg.residual else None
        shape, ref, perm_ref = _outputs(cfg, T, tiled)
        ws_bytes = M.moe_workspace_size(shape)
        assert 0 < ws_bytes <= M.MOE_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
        M.moe_layer(shape, x, li.w_router, li.bias, exs, res, ref["out"], ref["ids"], ref["w"],
                    perm_ref, ws, ws_bytes)
        _, got, perm_got = _outputs(cfg, T, tiled)
        M.moe_layer_noalloc(shape, x, li.w_router, li.bias, exs, res, got["out"], got["ids"],
                            got["w"], perm_got)
        # the permutation kept in the scratch array itself (perm == NULL)
        _, got2, _ = _outputs(cfg, T, tiled)
        M.moe_layer_noalloc(shape, x, li.w_router, li.bias, exs, res, got2["out"], got2["ids"],
                            got2["w"], None)
        torch.cuda.synchronize()
        for key in ref:
            a, b = ref[key].cpu(), got[key].cpu()
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"{name} call {call} (T={T}): {key} differs"
        for key in ("out", "ids", "w"):
            a, b = ref[key].cpu(), got2[key].cpu()
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"{name} call {call} (T={T}, perm NULL): {key} differs"
        assert np.isfinite(ref["out"].float().cpu().numpy()).all()
        say(f"  call {call} T={T}: identical (n_active {int(got['n_active'].item())})")


def test_noalloc_rejects_oversized_shape():
    """A shape whose workspace exceeds the fixed array is refused before any
    launch; the outputs keep their sentinels."""
    cfg = CONFIGS[3]
    shape = M.make_shape(4096, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt, M.MOE_F_TILED_WEIGHTS)
    assert M.moe_workspace_size(shape) > M.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, cfg.H), dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    exs = M.make_experts(g, g, g)
    _, o, perm = _outputs(cfg.with_(T=4096), 4096, True)
    st = M.moe_layer_noalloc(shape, x, wr, None, exs, None, o["out"], o["ids"], o["w"], perm,
                             check=False)
    assert st == 7, M.moe_status_str(st)      # MOE_E_WORKSPACE
    torch.cuda.synchronize()
    assert (o["ids"] == -7).all() and (o["n_active"] == -7).all()
    assert torch.isnan(o["out"].float()).all()
