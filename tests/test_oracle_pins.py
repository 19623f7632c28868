"""Pins for the CPU oracle: it is checked against what the reference pages
print, closed forms, brute force, invariants and library routines that the
special cases reduce to -- never against itself.

Every check looks up oracle functions through the module object ``O`` at
call time, so tests/test_oracle_mutations.py can plant a mistake in the
oracle and require that some pin here fails.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_constants():
    out = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, value = line.split()[:2]
            out[name] = float(value)
    return out


PAGE = _page_constants()


def _dense_experts(wg, wu, wd, act="f32"):
    """Wrap float arrays (exactly representable in float32) as dense f32
    storage for the oracle."""
    E, I, H = wg.shape
    return O.ExpertWeights("dense", act, H, I, wg.astype(np.float32), wu.astype(np.float32),
                           wd.astype(np.float32))


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# Page constants (accounting)
# --------------------------------------------------------------------------


def test_pin_params_per_expert():
    assert O.params_per_expert(2560, 640) == PAGE["params_per_expert"]


def test_pin_param_uses_per_token():
    assert O.param_uses_per_token(48, 10, 2560, 640) == PAGE["param_uses_per_token"]


def test_pin_ideal_payload():
    mib = O.ideal_payload_bytes_per_token(48, 10, 2560, 640, 2) / 2**20
    gib = O.ideal_payload_bytes_per_token(48, 10, 2560, 640, 4) / 2**30
    assert mib == PAGE["payload_2bit_MiB"]
    assert round(gib, 4) == PAGE["payload_4bit_GiB"]


def test_pin_intermediate_and_labels():
    assert O.intermediate_bytes(10, 640) == PAGE["intermediate_bytes_layer"]
    assert O.intermediate_bytes(10, 640, 48) == PAGE["intermediate_bytes_token"]
    assert O.route_label_bytes(10, 48) == PAGE["route_label_bytes_token"]


def test_pin_breakeven():
    assert O.breakeven_unique_experts(10, 4) == PAGE["breakeven_block5_tau4"]
    assert 10 * 5 == PAGE["worstcase_block5"]


def test_record_bytes_closed_form():
    n = 4915200
    assert O.expert_record_bytes(2560, 640, "dense") == 2 * n
    assert O.expert_record_bytes(2560, 640, "int4_g32") == n // 2 + n // 32 * 2
    assert O.expert_record_bytes(2560, 640, "int2_g32") == n // 4 + n // 32 * 2


# --------------------------------------------------------------------------
# Storage decoding
# --------------------------------------------------------------------------


def test_decode_bf16_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x4049], dtype=np.uint16)
    v = O.decode_bf16(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.25 and v[3] == 0.0
    assert v[4] == 3.140625


def test_decode_bf16_matches_torch():
    r = _rng(0).standard_normal(1000).astype(np.float32)
    t = torch.from_numpy(r).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.decode_bf16(bits), t.to(torch.float64).numpy())


def test_decode_fp16_patterns():
    bits = np.array([0x3C00, 0xB800, 0x0001, 0x7BFF], dtype=np.uint16)
    v = O.decode_fp16(bits)
    assert v[0] == 1.0 and v[1] == -0.5 and v[2] == 2.0**-24 and v[3] == 65504.0


def test_unpack_int4_nibble_order_and_sign():
    # byte 0x8F: low nibble 0xF = -1 (element 0), high nibble 0x8 = -8 (element 1)
    # byte 0x71: low 1, high 7
    codes = O.unpack_codes(np.array([[0x8F, 0x71]], dtype=np.uint8), 4, 4)
    assert codes.tolist() == [[-1, -8, 1, 7]]


def test_unpack_int2_order_and_sign():
    # 0xE4 = 0b11_10_01_00: elements (low bits first) 0, 1, -2, -1
    codes = O.unpack_codes(np.array([[0xE4, 0x1B]], dtype=np.uint8), 2, 8)
    assert codes.tolist() == [[0, 1, -2, -1, -1, -2, 1, 0]]


def test_dequantize_group_scale():
    # 64 codes all = +1 (nibble 0x1), scales 1.0 then 0.5 (fp16 0x3C00, 0x3800)
    packed = np.full((1, 32), 0x11, dtype=np.uint8)
    sc = np.array([[0x3C00, 0x3800]], dtype=np.uint16)
    w = O.dequantize(packed, sc, 4, 64)
    np.testing.assert_array_equal(w[0, :32], 1.0)
    np.testing.assert_array_equal(w[0, 32:], 0.5)
    # int2: code -1 everywhere with scale 2.0 (0x4000)
    packed2 = np.full((1, 8), 0xFF, dtype=np.uint8)
    w2 = O.dequantize(packed2, np.array([[0x4000]], dtype=np.uint16), 2, 32)
    np.testing.assert_array_equal(w2, -2.0)


def test_round_to_bf16_ties_to_even():
    one = 1.0
    assert O.round_to_bf16(np.array([one + 2**-8]))[0] == 1.0             # halfway -> even
    assert O.round_to_bf16(np.array([one + 3 * 2**-8]))[0] == 1.0 + 2**-6  # halfway -> even
    assert O.round_to_bf16(np.array([one + 2**-8 + 2**-30]))[0] == 1.0 + 2**-7
    assert O.round_to_bf16(np.array([-(one + 3 * 2**-8)]))[0] == -(1.0 + 2**-6)
    # subnormal bf16 values sit on the grid 2^-133 (smallest normal 2^-126)
    assert O.round_to_bf16(np.array([1.5 * 2.0**-133]))[0] == 2.0**-132      # halfway -> even
    assert O.round_to_bf16(np.array([2.0**-134]))[0] == 0.0                   # halfway -> even (0)
    assert O.round_to_bf16(np.array([2.0**-134 + 2.0**-160]))[0] == 2.0**-133
    assert O.round_to_bf16(np.array([3 * 2.0**-130 + 2.0**-140]))[0] == 3 * 2.0**-130


def test_round_to_bf16_matches_torch_on_float32():
    r = (_rng(1).standard_normal(5000) * 3).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(r.astype(np.float64)), ref)


# --------------------------------------------------------------------------
# Router logits
# --------------------------------------------------------------------------


def test_router_closed_form():
    x = np.array([[1.0, 2.0]])
    W = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-3.0, 0.5]])
    assert O.router_logits(x, W).tolist() == [[1.0, 2.0, 3.0, -2.0]]
    assert O.router_logits(x, W, np.array([0.5, 0, 0, 1])).tolist() == [[1.5, 2.0, 3.0, -1.0]]


def test_router_one_hot_input_reads_column():
    rng = _rng(2)
    W = rng.standard_normal((7, 5))
    for h in range(5):
        x = np.zeros((1, 5))
        x[0, h] = 1.0
        np.testing.assert_array_equal(O.router_logits(x, W)[0], W[:, h])


def test_router_bias_only():
    b = np.array([0.25, -1.0, 3.0])
    np.testing.assert_array_equal(O.router_logits(np.ones((2, 4)), np.zeros((3, 4)), b),
                                  np.tile(b, (2, 1)))


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------


def _topk_by_sort(logits, k):
    E = logits.shape[1]
    out = []
    for row in logits:
        order = sorted(range(E), key=lambda e: (-row[e], e))
        out.append(order[:k])
    return np.array(out)


def test_topk_hand_example():
    l = np.array([[0.1, 0.5, 0.5, -1.0, 0.3]])
    assert O.select_topk(l, 3).tolist() == [[1, 2, 4]]
    assert O.select_topk(l, 1).tolist() == [[1]]


def test_topk_zero_router_ties_lower_index():
    assert O.select_topk(np.zeros((3, 9)), 4).tolist() == [[0, 1, 2, 3]] * 3


def test_topk_tie_at_boundary_membership():
    # experts 5 and 2 tie for the last place: the lower index (2) is a member
    l = np.array([[0.0, 0.0, 1.0, 0.0, 3.0, 1.0, 2.0]])
    assert O.select_topk(l, 3).tolist() == [[4, 6, 2]]


def test_topk_negative_zero_equals_zero():
    assert O.select_topk(np.array([[-0.0, 0.0, -1.0]]), 1).tolist() == [[0]]
    assert O.select_topk(np.array([[0.0, -0.0, -1.0]]), 1).tolist() == [[0]]


def test_topk_matches_sort_with_ties():
    rng = _rng(3)
    l = np.round(rng.standard_normal((64, 40)) * 2) / 2      # many exact ties
    for k in (1, 3, 10, 40):
        np.testing.assert_array_equal(O.select_topk(l, k), _topk_by_sort(l, k))


def test_topk_k_equals_E_is_full_order():
    l = _rng(4).standard_normal((5, 12))
    np.testing.assert_array_equal(O.select_topk(l, 12), np.argsort(-l, axis=1, kind="stable"))


def test_topk_rejects_nonfinite():
    with pytest.raises(ValueError):
        O.select_topk(np.array([[0.0, np.inf]]), 1)


# --------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------


def test_weights_closed_form():
    l = np.log(np.array([[1.0, 2.0, 3.0, 4.0]]))
    ids = O.select_topk(l, 2)
    assert ids.tolist() == [[3, 2]]
    np.testing.assert_allclose(O.route_weights(l, ids), [[4 / 7, 3 / 7]], rtol=0, atol=1e-15)
    ids4 = O.select_topk(l, 4)
    np.testing.assert_allclose(O.route_weights(l, ids4), [[0.4, 0.3, 0.2, 0.1]], atol=1e-15)


def test_weights_k_equals_E_is_scipy_softmax():
    l = _rng(5).standard_normal((6, 9)) * 4
    ids = O.select_topk(l, 9)
    p = scipy.special.softmax(l, axis=1)
    np.testing.assert_allclose(O.route_weights(l, ids), np.take_along_axis(p, ids, 1), rtol=1e-13)


def test_weights_invariants():
    l = _rng(6).standard_normal((50, 32)) * 3
    ids = O.select_topk(l, 6)
    w = O.route_weights(l, ids)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
    assert (np.diff(w, axis=1) <= 1e-15).all()
    np.testing.assert_allclose(O.route_weights(l + 123.0, ids), w, rtol=1e-12)
    np.testing.assert_array_equal(O.route_weights(l, O.select_topk(l, 1)), 1.0)


def test_weights_zero_router():
    w = O.route_weights(np.zeros((2, 10)), O.select_topk(np.zeros((2, 10)), 4))
    np.testing.assert_allclose(w, 0.25, atol=1e-15)


# --------------------------------------------------------------------------
# Permutation
# --------------------------------------------------------------------------


def test_permutation_hand_example():
    p = O.permutation(np.array([[2, 0], [0, 1], [2, 1]]), 4)
    assert p.counts.tolist() == [2, 2, 2, 0]
    assert p.offsets.tolist() == [0, 2, 4, 6, 6]
    assert p.sorted_pair.tolist() == [1, 2, 3, 5, 0, 4]
    assert p.pair_row.tolist() == [4, 0, 1, 2, 5, 3]
    assert p.active.tolist() == [0, 1, 2] and p.n_active == 3


def test_permutation_matches_stable_argsort():
    rng = _rng(7)
    E, T, k = 37, 50, 5
    ids = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    p = O.permutation(ids, E)
    np.testing.assert_array_equal(p.sorted_pair, np.argsort(ids.reshape(-1), kind="stable"))
    np.testing.assert_array_equal(p.pair_row[p.sorted_pair], np.arange(T * k))
    np.testing.assert_array_equal(p.counts, np.bincount(ids.reshape(-1), minlength=E))
    np.testing.assert_array_equal(p.active, np.unique(ids))
    for e in range(E):
        seg = p.sorted_pair[p.offsets[e]:p.offsets[e + 1]]
        assert (ids.reshape(-1)[seg] == e).all()
        assert (np.diff(seg // k) > 0).all()          # ascending tokens


# --------------------------------------------------------------------------
# Expert FFN
# --------------------------------------------------------------------------


def test_swiglu_closed_form():
    a, b = 0.75, -1.25
    Wg = np.array([[1.0, 0.0], [0.0, 1.0]])
    Wu = np.array([[2.0, 0.0], [0.0, 3.0]])
    Wd = np.array([[1.0, 1.0], [0.0, 1.0]])
    sil = lambda z: z * scipy.special.expit(z)
    h0, h1 = sil(a) * 2 * a, sil(b) * 3 * b
    y = O.swiglu_expert(np.array([[a, b]]), Wg, Wu, Wd)
    np.testing.assert_allclose(y, [[h0 + h1, h1]], rtol=1e-15)


def test_swiglu_rectangular_closed_form():
    # H=3, I=1: g = x . wg, u = x . wu, y = wd * silu(g) * u
    x = np.array([[1.0, -2.0, 0.5]])
    wg = np.array([[0.5, 0.25, 1.0]])
    wu = np.array([[1.0, 1.0, 2.0]])
    wd = np.array([[1.0], [-2.0], [4.0]])
    g, u = 0.5 - 0.5 + 0.5, 1.0 - 2.0 + 1.0
    h = g * scipy.special.expit(g) * u
    np.testing.assert_allclose(O.swiglu_expert(x, wg, wu, wd), [[h, -2 * h, 4 * h]], rtol=1e-15)


def test_silu_values():
    np.testing.assert_allclose(O.silu(np.array([0.0, 1.0, -1.0, 30.0, -40.0])),
                               [0.0, scipy.special.expit(1.0), -scipy.special.expit(-1.0),
                                30.0 * scipy.special.expit(30.0), -40.0 * scipy.special.expit(-40.0)],
                               rtol=1e-14, atol=1e-300)


def test_swiglu_matches_torch_mlp():
    rng = _rng(8)
    x = rng.standard_normal((7, 24))
    Wg, Wu, Wd = rng.standard_normal((16, 24)), rng.standard_normal((16, 24)), rng.standard_normal((24, 16))
    tx = torch.from_numpy(x)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(tx, torch.from_numpy(Wg)))
        * torch.nn.functional.linear(tx, torch.from_numpy(Wu)), torch.from_numpy(Wd))
    np.testing.assert_allclose(O.swiglu_expert(x, Wg, Wu, Wd), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_down_scaling_doubles_output():
    rng = _rng(9)
    x, Wg, Wu, Wd = (rng.standard_normal(s) for s in ((3, 8), (4, 8), (4, 8), (8, 4)))
    np.testing.assert_array_equal(O.swiglu_expert(x, Wg, Wu, 2 * Wd), 2 * O.swiglu_expert(x, Wg, Wu, Wd))


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------


def test_combine_one_hot_and_residual():
    Y = np.arange(12, dtype=np.float64).reshape(6, 2)
    pair_row = np.array([5, 0, 1, 3, 2, 4])           # T=3, k=2
    w = np.array([[1.0, 0.0], [0.0, 1.0], [0.25, 0.75]])
    out = O.combine(Y, pair_row, w)
    np.testing.assert_array_equal(out[0], Y[5])
    np.testing.assert_array_equal(out[1], Y[3])
    np.testing.assert_array_equal(out[2], 0.25 * Y[2] + 0.75 * Y[4])
    res = np.full((3, 2), 10.0)
    np.testing.assert_array_equal(O.combine(Y, pair_row, w, res), out + 10.0)


# --------------------------------------------------------------------------
# Whole layer: sparse oracle vs dense brute force (different code paths)
# --------------------------------------------------------------------------


def _tiny_layer(seed, T=6, H=32, E=7, I=16, k=3, scale=0.3):
    rng = _rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    Wr = (rng.standard_normal((E, H)) * scale).astype(np.float32).astype(np.float64)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    wg = (rng.standard_normal((E, I, H)) * scale).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) * scale).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) * scale).astype(np.float32)
    return x, Wr, bias, _dense_experts(wg, wu, wd)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_matches_dense_bruteforce(seed):
    x, Wr, bias, ex = _tiny_layer(seed)
    r = O.moe_layer(x, Wr, bias, ex, 3)
    dense = O.dense_moe_layer(x, Wr, bias, ex, 3)
    np.testing.assert_allclose(r.out, dense, rtol=1e-12, atol=1e-14)
    res = x * 0.5
    np.testing.assert_allclose(O.moe_layer(x, Wr, bias, ex, 3, residual=res).out,
                               O.dense_moe_layer(x, Wr, bias, ex, 3, residual=res), rtol=1e-12, atol=1e-14)


def test_layer_single_expert_is_plain_mlp():
    x, Wr, _, ex = _tiny_layer(4, E=1, k=1)
    wg, wu, wd = ex.expert(0)
    r = O.moe_layer(x, Wr, None, ex, 1)
    tx = torch.from_numpy(x)
    F = torch.nn.functional
    ref = F.linear(F.silu(F.linear(tx, torch.from_numpy(wg))) * F.linear(tx, torch.from_numpy(wu)),
                   torch.from_numpy(wd)).numpy()
    np.testing.assert_allclose(r.out, ref, rtol=1e-12, atol=1e-14)


def test_layer_lowbit_matches_dense_bruteforce():
    rng = _rng(11)
    T, H, E, I, k = 5, 64, 6, 32, 2
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    Wr = rng.standard_normal((E, H)) * 0.2
    pk = lambda r, K: rng.integers(0, 256, (E, r, K // 2), dtype=np.uint8)
    sc = lambda r, K: np.float16(rng.uniform(0.01, 0.05, (E, r, K // 32))).view(np.uint16)
    ex = O.ExpertWeights("int4_g32", "bf16", H, I, pk(I, H), pk(I, H), pk(H, I),
                         sc(I, H), sc(I, H), sc(H, I))
    np.testing.assert_allclose(O.moe_layer(x, Wr, None, ex, k).out,
                               O.dense_moe_layer(x, Wr, None, ex, k), rtol=1e-12, atol=1e-14)


def test_dense_oracle_ceiling_enforced():
    x = np.zeros((1, 2560))
    ex = O.ExpertWeights("dense", "f32", 2560, 640, None, None, None)
    with pytest.raises(ValueError):
        O.dense_moe_layer(x, np.zeros((1024, 2560)), None, ex, 1)


def test_layer_only_tokens_is_exact_subset():
    x, Wr, bias, ex = _tiny_layer(5, T=9)
    full = O.moe_layer(x, Wr, bias, ex, 3)
    part = O.moe_layer(x, Wr, bias, ex, 3, only_tokens=[2, 7])
    np.testing.assert_array_equal(part.out[[2, 7]], full.out[[2, 7]])
    assert np.isnan(part.out[0]).all()


# --------------------------------------------------------------------------
# Stack
# --------------------------------------------------------------------------


def test_stack_zero_down_is_identity():
    x, Wr, bias, ex = _tiny_layer(6)
    zero = O.ExpertWeights("dense", "f32", ex.H, ex.I, ex.gate, ex.up, np.zeros_like(ex.down))
    xs = O.moe_stack(x, [lambda: (Wr, bias, zero)] * 3, 3, "f32")
    for xl in xs:
        np.testing.assert_array_equal(xl, x)


def test_stack_rounds_each_layer_to_storage_and_subset_exact():
    x, Wr, bias, ex = _tiny_layer(7, T=8)
    xs = O.moe_stack(x, [lambda: (Wr, bias, ex)] * 2, 3, "bf16")
    for xl in xs[1:]:
        np.testing.assert_array_equal(O.round_to_bf16(xl), xl)
    sub = O.moe_stack(x, [lambda: (Wr, bias, ex)] * 2, 3, "bf16", only_tokens=[1, 6])
    np.testing.assert_array_equal(sub[-1], xs[-1][[1, 6]])
    # one layer with residual = x equals x + (layer without residual), rounded
    one = O.moe_layer(x, Wr, bias, ex, 3).out
    np.testing.assert_allclose(xs[1], O.round_to_bf16(x + one), rtol=0, atol=0)


# --------------------------------------------------------------------------
# Near ties and block statistics
# --------------------------------------------------------------------------


def test_near_ties():
    l = np.array([[3.0, 2.0, 2.0, 1.0],                # exact tie: not a near tie
                  [3.0, 2.0, 2.0 - 1e-9, 1.0],         # near tie inside top-(k+1)
                  [3.0, 2.0, 1.0, 1.0 - 1e-9]])        # near tie below the cut
    assert O.near_tie_tokens(l, 2).tolist() == [False, True, False]


def test_repeat_fraction_and_unique():
    ids = np.array([[0, 1], [0, 2], [3, 4]])
    assert O.unique_experts(ids) == 5
    assert O.repeat_fraction(ids) == pytest.approx(2 / 6)


def test_grouped_stages_compose_to_ffn():
    x, Wr, bias, ex = _tiny_layer(12, T=7)
    ids = O.select_topk(O.router_logits(x, Wr, bias), 3)
    perm = O.permutation(ids, Wr.shape[0])
    A = O.grouped_intermediate(x, perm, 3, ex)
    np.testing.assert_allclose(O.grouped_down(A, perm, ex), O.grouped_ffn(x, perm, 3, ex),
                               rtol=1e-13, atol=1e-15)
    # intermediate of one row against its closed form
    r = 0
    e = ids.reshape(-1)[perm.sorted_pair[r]]
    t = perm.sorted_pair[r] // 3
    wg, wu, _ = ex.expert(int(e))
    g, u = wg @ x[t], wu @ x[t]
    np.testing.assert_allclose(A[r], g * scipy.special.expit(g) * u, rtol=1e-13)


# ---- route locality (AFN-019 "Hypothesis H7", "Gate B - trace-only locality") ----

def _window_ids(T, k, E, step):
    """token t selects experts (step*t + j) mod E, j < k"""
    return np.array([[(step * t + j) % E for j in range(k)] for t in range(T)])


def test_pin_locality_closed_forms():
    T, k, E = 13, 10, 512
    same = np.tile(np.arange(k), (T, 1))
    assert list(O.overlap_with_previous(same)) == [0] + [k] * (T - 1)
    slide = _window_ids(T, k, E, 1)                 # consecutive tokens share k - 1 experts
    assert list(O.overlap_with_previous(slide)) == [0] + [k - 1] * (T - 1)
    disjoint = _window_ids(T, k, E, k)              # no expert in common
    assert list(O.overlap_with_previous(disjoint)) == [0] * T
    for B in range(1, 6):
        lens = [min(B, T - b) for b in range(0, T, B)]   # last block ragged (13 tokens)
        assert list(O.block_unique(same, B)) == [k] * len(lens)
        assert list(O.block_unique(slide, B)) == [k + n - 1 for n in lens]
        assert list(O.block_unique(disjoint, B)) == [k * n for n in lens]


def test_pin_locality_bitset_bruteforce():
    """Against an independent bitset/popcount formulation on random routes."""
    rng = np.random.default_rng(11)
    for T, k, E in ((7, 3, 9), (17, 5, 23), (1, 4, 4)):
        ids = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)])
        masks = [sum(1 << int(e) for e in row) for row in ids]
        ov = [0] + [bin(masks[t] & masks[t - 1]).count("1") for t in range(1, T)]
        assert list(O.overlap_with_previous(ids)) == ov
        for B in range(1, 6):
            un = []
            for b in range(0, T, B):
                m = 0
                for t in range(b, min(T, b + B)):
                    m |= masks[t]
                un.append(bin(m).count("1"))
            assert list(O.block_unique(ids, B)) == un


def test_pin_breakeven_tau_and_skew():
    # the page's block-of-five example: 40 unique experts break even at tau = 4
    assert O.breakeven_tau(PAGE["breakeven_block5_tau4"], 10) == 4
    assert O.breakeven_tau(PAGE["worstcase_block5"], 10) == 5
    assert O.layer_skew(np.full(16, 5), k=2, T=40) == 1.0
    c = np.zeros(16, dtype=np.int64)
    c[3] = 80
    assert O.layer_skew(c, k=2, T=40) == 16.0
