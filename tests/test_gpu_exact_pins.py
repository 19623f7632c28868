"""Exact-arithmetic pin of the router on the GPU.

With small-integer activations and router weights that are signed powers of
two (or zero), every product and every partial sum of the router reduction
is a multiple of 2^-6 below 2^15, so it is exact in float32 whatever the
summation order.  The GPU's float32 logits must then equal the float64
oracle's logits exactly (the oracle value is itself checked to be exact in
float32), on every router path: the small-batch kernel (T <= 64), the
LDS kernel whose group sums the top-k kernel finishes (T <= 1024), the LDS
kernel that finishes them itself (larger T), and the float32 path.  The
selected experts must then equal the oracle's bit for bit: integer logits
tie exactly where they tie, and the lower index must win those ties.

The logit definition pinned here is "Agent Field Notes -- full corpus",
AFN-001, section "Phase 1: separate math from acceleration" (router logits,
float32 softmax and normalized top-k); the tie rule is AFN-017, section
"Tie handling belongs to membership".
"""
import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from oracle import moe_oracle as O
from tests.gpu_util import DEV, TOL_W, say, to_act_tensor

pytestmark = pytest.mark.gpu

H, E, K = 2560, 512, 10


def exact_inputs(T, seed):
    """x: integers in [-8, 8]; W_router: 0 or +-2^-m, m in 0..6; bias:
    multiples of 2^-6 in [-1, 1].  All exact in bf16 and float32."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-8, 9, size=(T, H)).astype(np.float64)
    wr = rng.choice([-1.0, 0.0, 1.0], size=(E, H)) * np.ldexp(1.0, -rng.integers(0, 7, size=(E, H)))
    bias = rng.integers(-64, 65, size=E).astype(np.float64) / 64.0
    return x, wr, bias


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("T", [16, 512, 2048])
def test_router_logits_exact(act, T):
    x, wr, bias = exact_inputs(T, seed=7000 + T)
    ref = O.router_logits(x, wr, bias)
    # the inputs make the exact sums representable in float32
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    buf = M.MoELayerBuffers(T, H, E, 640, K, act, "dense", device=DEV)
    say(f"exact router logits: act={act} T={T}")
    buf.route(to_act_tensor(x, act), to_act_tensor(wr, act),
              torch.from_numpy(bias.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    got = buf.logits.cpu().numpy()
    bad = got.astype(np.float64) != ref
    assert not bad.any(), (f"{int(bad.sum())} logits differ; first at {np.argwhere(bad)[0]}: "
                           f"{got[bad][0]!r} vs {ref[bad][0]!r}")
    ids_ref = O.select_topk(ref, K)
    ids = buf.topk_ids.cpu().numpy()
    assert np.array_equal(ids, ids_ref)
    w_ref = O.route_weights(ref, ids_ref)
    werr = float(np.abs(buf.topk_w.cpu().numpy().astype(np.float64) - w_ref).max())
    assert werr <= TOL_W
    # exact ties between a selected and an unselected expert, resolved by index
    srt = np.sort(ref, axis=1)[:, ::-1]
    ties = int((srt[:, K - 1] == srt[:, K]).sum())
    say(f"  logits identical ({T * E}), ids identical, weights {werr:.2g}, "
        f"{ties} tokens with an exact tie at the selection boundary")
