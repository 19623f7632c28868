"""Exact top-k with many tied logits, on every top-k path.

The router rows repeat: expert e uses base row (7 e + 3) mod R, so each
logit value is shared by about E / R experts spread over the selection's
slots and lanes.  Activations and base rows are small integers, so every
logit is an exact integer on the GPU (float32) and in the float64 oracle,
and logits tie exactly where the rows repeat.  The selected experts must
equal the oracle's (rank-count definition, lower index first among equal
logits) on every token, and the weights must match within the weight
tolerance.  With R = 24 the top group holds 21-22 experts, so the first
k = 10 ranks all come from one tie group; with R = 100 the top k spans
several groups of about 5 and ties cross the k-th rank.  Both stay within
the 64 candidates the threshold selection ranks directly; R = 1 (every
logit equal) takes the round-by-round selection.

Tie rule: "Agent Field Notes -- full corpus", AFN-017, section "Tie handling
belongs to membership"; rank order: AFN-021, section "The key equivalence
-- and where it breaks".
"""
import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL_W, say, to_act_tensor

pytestmark = pytest.mark.gpu

H, E, K, I = 256, 512, 10, 128


def tied_inputs(T, R, seed):
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(T, H)).astype(np.float64)
    base = rng.integers(-2, 3, size=(R, H)).astype(np.float64)
    wr = base[(7 * np.arange(E) + 3) % R]
    return x, wr


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("T", [8, 40, 100, 1100])
@pytest.mark.parametrize("R", [1, 24, 100])
def test_topk_exact_ties(T, R, act):
    if act == "f32" and T > 100:
        pytest.skip("one float32 case per size class is enough")
    x, wr = tied_inputs(T, R, seed=1000 * R + T)
    logits = O.router_logits(x, wr)
    assert np.array_equal(logits, logits.astype(np.float32)), "logits not exact in float32"
    ids_ref = O.select_topk(logits, K)
    w_ref = O.route_weights(logits, ids_ref)
    buf = M.MoELayerBuffers(T, H, E, I, K, act, "dense", device=DEV)
    xt, wt = to_act_tensor(x, act), to_act_tensor(wr, act)
    calls = [("route", lambda: buf.route(xt, wt, None))]
    if act == "bf16" and T <= 32:
        calls.append(("route_permute", lambda: buf.route_permute(xt, wt, None)))
    for name, call in calls:
        say(f"[ties T={T} R={R} {act}] {name}")
        buf.topk_ids.fill_(-7)
        call()
        torch.cuda.synchronize()
        ids = buf.topk_ids.cpu().numpy()
        bad = np.nonzero((ids != ids_ref).any(axis=1))[0]
        assert bad.size == 0, f"{name}: token {bad[0]} got {ids[bad[0]]}, oracle {ids_ref[bad[0]]}"
        w = buf.topk_w.cpu().numpy().astype(np.float64)
        assert np.abs(w - w_ref).max() <= TOL_W, f"{name}: weights off by {np.abs(w - w_ref).max():.3g}"
        if name == "route_permute":
            counts = np.bincount(ids_ref.ravel(), minlength=E)
            assert np.array_equal(buf.counts.cpu().numpy(), counts)
