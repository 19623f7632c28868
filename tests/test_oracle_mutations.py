"""Planted-mistake test for the oracle (CPU only).

Each mutation replaces one oracle function with a plausible wrong variant
(a dropped term, a wrong sign, a wrong index or order, a transposed operand);
the pin suite in test_oracle_pins.py must then fail somewhere.  A mutation
that survives means the oracle's arithmetic in that spot is unpinned.
"""
import inspect

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import test_oracle_pins as PINS

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _pin_functions():
    out = []
    for name, fn in inspect.getmembers(PINS, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "seed" in params:
            out.append((name, lambda fn=fn: fn(seed=0)))
        elif not params:
            out.append((name, fn))
    return out


# --- mutated variants -------------------------------------------------------

def m_decode_bf16_shift(bits):
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def m_unpack_unsigned(packed, bits, K):
    q = _orig["unpack_codes"](packed, bits, K)
    return np.where(q < 0, q + (1 << bits), q)


def m_unpack_high_first(packed, bits, K):
    q = _orig["unpack_codes"](packed, bits, K)
    per = 8 // bits
    return q.reshape(q.shape[:-1] + (K // per, per))[..., ::-1].reshape(q.shape)


def m_dequant_tile(packed, scale_bits, bits, K):
    q = O.unpack_codes(packed, bits, K).astype(np.float64)
    s = O.decode_fp16(scale_bits)
    return q * np.tile(s, (1,) * (s.ndim - 1) + (32,))


def m_router_no_bias(x, w, bias=None):
    return x @ w.T


def m_router_reversed_experts(x, w, bias=None):
    return _orig["router_logits"](x, w[::-1], bias)


def m_router_transposed_bias_sign(x, w, bias=None):
    return _orig["router_logits"](x, w, None if bias is None else -np.asarray(bias))


def m_topk_higher_index_ties(logits, k):
    E = logits.shape[1]
    ids = _orig["select_topk"](logits[:, ::-1], k)
    return E - 1 - ids


def m_topk_smallest(logits, k):
    return _orig["select_topk"](-logits, k)


def m_topk_index_order(logits, k):
    return np.sort(_orig["select_topk"](logits, k), axis=1)


def m_weights_unnormalized(logits, ids):
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids, axis=1)


def m_weights_sign(logits, ids):
    return _orig["route_weights"](-logits, ids)


def m_perm_descending_tokens(ids, E):
    T, k = np.asarray(ids).shape
    p = _orig["permutation"](np.asarray(ids)[::-1], E)
    # map back pair indices of the reversed token order
    sp = p.sorted_pair
    t, j = sp // k, sp % k
    sp2 = (T - 1 - t) * k + j
    pr = np.empty_like(sp2)
    pr[sp2] = np.arange(sp2.size)
    return O.Permutation(p.counts, p.offsets, sp2, pr, p.active, p.n_active)


def m_perm_not_inverse(ids, E):
    p = _orig["permutation"](ids, E)
    return O.Permutation(p.counts, p.offsets, p.sorted_pair, p.sorted_pair.copy(), p.active, p.n_active)


def m_silu_sigmoid(g):
    return 1.0 / (1.0 + np.exp(-g))


def m_silu_sign(g):
    return g / (1.0 + np.exp(g))


def m_swiglu_swap(x, wg, wu, wd):
    return _orig["swiglu_expert"](x, wu, wg, wd)


def m_swiglu_drop_up(x, wg, wu, wd):
    return O.silu(x @ wg.T) @ wd.T


def m_swiglu_down_transposed(x, wg, wu, wd):
    a = O.silu(x @ wg.T) * (x @ wu.T)
    return (wd.T @ a.T).T if wd.shape[0] == wd.shape[1] else a @ wd.reshape(wd.shape[1], wd.shape[0])


def m_combine_reversed(Y, pair_row, w, residual=None):
    return _orig["combine"](Y, pair_row, w[:, ::-1], residual)


def m_combine_no_residual(Y, pair_row, w, residual=None):
    return _orig["combine"](Y, pair_row, w, None)


def m_combine_pair_index(Y, pair_row, w, residual=None):
    return _orig["combine"](Y, np.arange(pair_row.size), w, residual)


def m_params_down_square(H, I):
    return H * I + H * I + I * I


def m_round_truncate(v):
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def m_act_round_identity(v, act):
    return np.asarray(v, dtype=np.float64)


def m_payload_bits_bytes(layers, k, H, I, bits):
    return O.param_uses_per_token(layers, k, H, I) * bits / 10


def m_overlap_two_back(ids):
    ids = np.asarray(ids)
    out = np.zeros(ids.shape[0], dtype=np.int64)
    for t in range(2, ids.shape[0]):
        out[t] = len(set(ids[t].tolist()) & set(ids[t - 2].tolist()))
    return out


def m_block_unique_overlapping(ids, B):
    ids = np.asarray(ids)
    return np.array([len(set(ids[b:b + B + 1].reshape(-1).tolist()))
                     for b in range(0, ids.shape[0], B)], dtype=np.int64)


def m_block_unique_count_pairs(ids, B):
    ids = np.asarray(ids)
    return np.array([ids[b:b + B].size for b in range(0, ids.shape[0], B)], dtype=np.int64)


MUTATIONS = [
    ("overlap_with_previous", m_overlap_two_back),
    ("block_unique", m_block_unique_overlapping),
    ("block_unique", m_block_unique_count_pairs),
    ("decode_bf16", m_decode_bf16_shift),
    ("unpack_codes", m_unpack_unsigned),
    ("unpack_codes", m_unpack_high_first),
    ("dequantize", m_dequant_tile),
    ("router_logits", m_router_no_bias),
    ("router_logits", m_router_reversed_experts),
    ("router_logits", m_router_transposed_bias_sign),
    ("select_topk", m_topk_higher_index_ties),
    ("select_topk", m_topk_smallest),
    ("select_topk", m_topk_index_order),
    ("route_weights", m_weights_unnormalized),
    ("route_weights", m_weights_sign),
    ("permutation", m_perm_descending_tokens),
    ("permutation", m_perm_not_inverse),
    ("silu", m_silu_sigmoid),
    ("silu", m_silu_sign),
    ("swiglu_expert", m_swiglu_swap),
    ("swiglu_expert", m_swiglu_drop_up),
    ("swiglu_expert", m_swiglu_down_transposed),
    ("combine", m_combine_reversed),
    ("combine", m_combine_no_residual),
    ("combine", m_combine_pair_index),
    ("params_per_expert", m_params_down_square),
    ("round_to_bf16", m_round_truncate),
    ("act_round", m_act_round_identity),
    ("ideal_payload_bytes_per_token", m_payload_bits_bytes),
]


@pytest.mark.parametrize("target,mutant", MUTATIONS, ids=[m.__name__ for _, m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(O, target, mutant)
    caught = []
    for name, fn in _pin_functions():
        try:
            fn()
        except Exception:      # assertion or a crash in the mutated oracle
            caught.append(name)
    assert caught, f"mutation {mutant.__name__} of {target} survived every pin"
