"""The C++ float64 oracle (oracle/moe_oracle_c.cpp) checked on the CPU.

It is pinned against the numpy oracle, whose own pins live in
test_oracle_pins.py, and against the dense brute force (every token through
every expert, gated by the top-k mask), which shares no permutation or
grouping with either: routes and the permutation bit-exact, float values to
float64 summation-order noise.  Special cases that the pages fix are checked
directly: equal logits go to the lower expert index, k = E keeps every
expert, and the thread count does not change a bit of the result.  The
low-bit decoders are pinned by closed forms: the most negative code (-8,
-2) decodes as q * s, and codes sit lowest bits first within a byte.
"""
import numpy as np
import pytest
import torch

from moe_inputs import get_config, make_layer, tensor_to_numpy_storage
from oracle import moe_oracle as O
from oracle import oracle_c as C

RTOL = 1e-11


def _cases():
    tiny = get_config("tiny")
    pre, st4, v2 = get_config("prefill"), get_config("stack_int4"), get_config("verify_int2")
    return {
        "tiny_f32": tiny,
        "tiny_k_eq_E": tiny.with_(T=5, k=16),
        "bf16_zipf": pre.with_(T=24, H=256, E=16, I=64, k=4),
        "bf16_T1": pre.with_(T=1, H=128, E=8, I=64, k=3),
        "int4_residual": st4.with_(T=12, H=128, E=8, I=64, k=3, layers=1),
        "int2_hotset_residual": v2.with_(T=10, H=128, E=8, I=64, k=3, layers=1),
    }


CASES = _cases()


def _inputs(cfg):
    li = make_layer(cfg, device="cpu")
    x64 = O.decode_act(tensor_to_numpy_storage(li.x), cfg.act)
    wr64 = O.decode_act(tensor_to_numpy_storage(li.w_router), cfg.act)
    b64 = None if li.bias is None else li.bias.double().numpy()
    st = C.storage_arrays(li.experts)
    ex = O.ExpertWeights(cfg.wfmt, cfg.act, cfg.H, cfg.I, st["gate"], st["up"], st["down"],
                         st["gate_scale"], st["up_scale"], st["down_scale"])
    res = x64 if cfg.residual else None
    return x64, wr64, b64, st, ex, res


def _close(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, what
    assert np.isfinite(a).all(), what
    scale = max(float(np.abs(b).max()), 1e-300)
    err = float(np.abs(a - b).max())
    assert err <= RTOL * scale, f"{what}: max err {err} vs scale {scale}"


@pytest.mark.parametrize("name", list(CASES))
def test_c_oracle_matches_numpy_oracle(name):
    cfg = CASES[name]
    x64, wr64, b64, st, ex, res = _inputs(cfg)
    got = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k, res)
    ref = O.moe_layer(x64, wr64, b64, ex, cfg.k, residual=res)
    _close(got.logits, ref.logits, "logits")
    np.testing.assert_array_equal(got.ids, ref.ids)
    # the rank-count selection equals a stable sort on (-logit, index)
    order = np.argsort(-got.logits, axis=1, kind="stable")[:, :cfg.k]
    np.testing.assert_array_equal(got.ids, order)
    _close(got.w, ref.w, "weights")
    np.testing.assert_array_equal(got.perm.counts, ref.perm.counts)
    np.testing.assert_array_equal(got.perm.offsets, ref.perm.offsets)
    np.testing.assert_array_equal(got.perm.sorted_pair, ref.perm.sorted_pair)
    np.testing.assert_array_equal(got.perm.pair_row, ref.perm.pair_row)
    np.testing.assert_array_equal(got.perm.active, ref.perm.active)
    _close(got.Y, ref.Y, "expert rows")
    _close(got.out, ref.out, "layer output")


@pytest.mark.parametrize("name", ["tiny_f32", "int4_residual", "int2_hotset_residual"])
def test_c_oracle_matches_dense_brute_force(name):
    cfg = CASES[name]
    x64, wr64, b64, st, ex, res = _inputs(cfg)
    got = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k, res)
    _close(got.out, O.dense_moe_layer(x64, wr64, b64, ex, cfg.k, residual=res), "dense brute force")


def test_c_oracle_equal_logits_pick_lower_index():
    # a zero router gives every expert the same logit: the top-k is 0..k-1 in
    # order and each weight is 1/k
    cfg = CASES["tiny_f32"]
    x64, wr64, _, st, _, _ = _inputs(cfg)
    got = C.moe_layer_c(x64, np.zeros_like(wr64), None, st, cfg.wfmt, cfg.act, cfg.k)
    np.testing.assert_array_equal(got.ids, np.tile(np.arange(cfg.k), (cfg.T, 1)))
    np.testing.assert_allclose(got.w, np.full((cfg.T, cfg.k), 1.0 / cfg.k), rtol=1e-15)


def test_c_oracle_k_equals_E_keeps_all_experts_in_logit_order():
    cfg = CASES["tiny_k_eq_E"]
    x64, wr64, b64, st, _, _ = _inputs(cfg)
    got = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k)
    for t in range(cfg.T):
        # stable descending sort of the logits (lower index first among equals)
        want = np.argsort(-got.logits[t], kind="stable")
        np.testing.assert_array_equal(got.ids[t], want)
    # renormalizing over all experts is the full softmax
    p = torch.softmax(torch.from_numpy(got.logits), dim=1).numpy()
    np.testing.assert_allclose(got.w, np.take_along_axis(p, got.ids, axis=1), rtol=1e-12)
    assert got.perm.n_active == cfg.E
    np.testing.assert_array_equal(got.perm.counts, np.full(cfg.E, cfg.T))


def test_c_oracle_routes_only_equals_layer():
    cfg = CASES["bf16_zipf"]
    x64, wr64, b64, st, _, _ = _inputs(cfg)
    full = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k)
    logits, ids, w, perm = C.routes_c(x64, wr64, b64, cfg.k)
    np.testing.assert_array_equal(logits, full.logits)
    np.testing.assert_array_equal(ids, full.ids)
    np.testing.assert_array_equal(w, full.w)
    for f in ("counts", "offsets", "sorted_pair", "pair_row", "active"):
        np.testing.assert_array_equal(getattr(perm, f), getattr(full.perm, f))


def test_c_oracle_thread_count_is_bit_invariant():
    cfg = CASES["int4_residual"]
    x64, wr64, b64, st, _, res = _inputs(cfg)
    a = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k, res, threads=1)
    b = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k, res, threads=5)
    for f in ("logits", "ids", "w", "Y", "out"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_c_oracle_rejects_non_finite_logits():
    cfg = CASES["tiny_f32"]
    x64, wr64, b64, st, _, _ = _inputs(cfg)
    x64 = x64.copy()
    x64[3, 7] = np.inf
    with pytest.raises(ValueError):
        C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k)


@pytest.mark.parametrize("wfmt,neg_byte,one_byte,qneg", [("int4_g32", 0x88, 0x11, -8),
                                                         ("int2_g32", 0xAA, 0x55, -2)])
def test_c_oracle_most_negative_code_closed_form(wfmt, neg_byte, one_byte, qneg):
    # every gate code is the most negative one (never produced by the
    # quantizer, still decoded as q * s), every up code +1, every down code
    # the most negative one at scale 0.5: g = qneg S, u = S with S = sum(x),
    # y_n = I * (0.5 qneg) * silu(g) * u
    T, H, I, E = 1, 128, 32, 1
    bits = 4 if wfmt == "int4_g32" else 2
    rng = np.random.default_rng(5)
    x = np.round(rng.standard_normal((T, H)) * 8) / 64        # exact in bf16
    wr = np.zeros((E, H))
    one, half = 0x3C00, 0x3800                                 # fp16 1.0, 0.5
    st = {"gate": np.full((E, I, H * bits // 8), neg_byte, np.uint8),
          "up": np.full((E, I, H * bits // 8), one_byte, np.uint8),
          "down": np.full((E, H, I * bits // 8), neg_byte, np.uint8),
          "gate_scale": np.full((E, I, H // 32), one, np.uint16),
          "up_scale": np.full((E, I, H // 32), one, np.uint16),
          "down_scale": np.full((E, H, I // 32), half, np.uint16)}
    got = C.moe_layer_c(x, wr, None, st, wfmt, "bf16", 1)
    S = x.sum()
    g = qneg * S
    a = g / (1.0 + np.exp(-g)) * S
    np.testing.assert_allclose(got.out, np.full((T, H), I * 0.5 * qneg * a), rtol=1e-12)


@pytest.mark.parametrize("wfmt,byte,codes", [("int4_g32", 0x1F, [-1, 1]),
                                             ("int2_g32", 0x1B, [-1, -2, 1, 0])])
def test_c_oracle_code_order_within_a_byte(wfmt, byte, codes):
    # element c of a row sits at byte c*bits/8, bit (c*bits)%8, lowest first:
    # with every byte equal, gate row i is the periodic pattern `codes`
    T, H, I, E = 1, 128, 32, 1
    bits = 4 if wfmt == "int4_g32" else 2
    rng = np.random.default_rng(6)
    x = np.round(rng.standard_normal((T, H)) * 8) / 64
    one = 0x3C00
    st = {"gate": np.full((E, I, H * bits // 8), byte, np.uint8),
          "up": np.full((E, I, H * bits // 8), 0x11 if bits == 4 else 0x55, np.uint8),
          "down": np.full((E, H, I * bits // 8), 0x11 if bits == 4 else 0x55, np.uint8),
          "gate_scale": np.full((E, I, H // 32), one, np.uint16),
          "up_scale": np.full((E, I, H // 32), one, np.uint16),
          "down_scale": np.full((E, H, I // 32), one, np.uint16)}
    got = C.moe_layer_c(x, np.zeros((E, H)), None, st, wfmt, "bf16", 1)
    pattern = np.tile(np.array(codes, dtype=np.float64), H // len(codes))
    g = float(pattern @ x[0])
    S = x.sum()
    a = g / (1.0 + np.exp(-g)) * S
    np.testing.assert_allclose(got.out, np.full((T, H), I * a), rtol=1e-12)


def test_round_bf16_closed_forms_and_numpy():
    """The C++ oracle's bf16 storage rounding: ties to even in the normal
    and subnormal ranges, overflow to infinity, signed zero; and the same bits
    as the numpy oracle over values spanning the whole exponent range."""
    from oracle import moe_oracle as O
    one = 1.0
    cases = {one + 2**-8: 1.0, one + 3 * 2**-8: 1.0 + 2**-6, one + 2**-8 + 2**-30: 1.0 + 2**-7,
             -(one + 3 * 2**-8): -(1.0 + 2**-6), 1.5 * 2.0**-133: 2.0**-132, 2.0**-134: 0.0,
             2.0**-134 + 2.0**-160: 2.0**-133, 3.4e38: float("inf"), -3.4e38: float("-inf")}
    v = np.array(list(cases))
    got = C.decode_act_c(C.round_bf16_c(v), "bf16")
    assert np.array_equal(got, np.array(list(cases.values())))
    assert C.round_bf16_c(np.array([-0.0]))[0] == 0x8000
    rng = np.random.default_rng(5)
    w = rng.standard_normal(50000) * np.exp(rng.uniform(-95, 95, 50000))
    assert np.array_equal(C.round_bf16_c(w), O.bf16_bits_of(O.round_to_bf16(w)))
    bits = rng.integers(0, 1 << 16, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]                  # finite patterns
    assert np.array_equal(C.decode_act_c(bits, "bf16"), O.decode_bf16(bits))
