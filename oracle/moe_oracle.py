"""Plain CPU oracle for the routed sparse-MoE layer (TEST INFRASTRUCTURE ONLY).

This module is the executable specification the HIP path is checked against.
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline legs of
``bench.py`` may import it; the product library never does, and it shares no
code, table or helper with the HIP path.  Everything is computed in float64
from the exact stored input values (bf16, fp16, fp32 and small integers all
convert exactly to float64).

Sources.  The reference is a set of web pages; citations name the page title,
the note and the section:

* [P-019] "Agent Field Notes — full corpus", note AFN-019 "Hide SSD misses
  before the router knows they exist" (the same text is the page "Hide SSD
  misses before the router knows they exist"):
  - section "Why overlap alone cannot defeat the byte roofline": the layer
    geometry (48 layers, 512 routed experts, top-10, hidden 2,560, routed
    intermediate 640), the gate+up+down parameter count per expert, the
    parameter uses per token, the ideal low-bit payload per token, and the
    byte-saving mechanisms (low-bit storage, dedupe of repeated routes across
    a verifier block, grouping token rows by expert);
  - section "Hypothesis H4: ExpertMajor should stream as a wavefront, not a
    barrier": gate and up are consumed together, down only after the SwiGLU
    intermediate exists; experts write separate result slots and the final
    weighted sum runs in a fixed route-rank order;
  - section "Hypothesis H5: prefill and decode need different streaming
    modes": a verifier block reads the deduplicated union of its routes;
  - section "Hypothesis H6: another request is the only general filler for a
    hard miss": later-layer routes depend on earlier-layer results, so layers
    run strictly in sequence;
  - section "Hypothesis H7: DFlash block size must follow I/O cost": the
    routed-byte break-even U_B < 10 tau(B) and its block-of-five example.
* [P-001] same page, note AFN-001 "Porting Qwen3.8-Flash-Next to Hebrus:
  evidence before execution", section "Phase 1: separate math from
  acceleration": the router is a float32 softmax followed by a normalized
  top-10 selection; the tie policy is a contract case.
* [P-021] same page, note AFN-021 "Replay decode as prefill: a training
  flywheel for predictive MoE I/O":
  - section "The key equivalence — and where it breaks": expert IDs and
    their rank order must match exactly, weights within a declared tolerance;
  - section "Do not store every large activation": the [10,640] float32
    intermediate (25,600 B per layer and token) and the 3,840 B of top-10
    labels per token.
* [P-017] same page, note AFN-017 "Top-k chooses the set; time chooses the
  order", sections "Tie handling belongs to membership" (equal scores pick the
  smaller position, decided while choosing membership) and "The dense-parity
  property" (a sparse result must equal the dense one when nothing is cut).
* [P-011] same page, note AFN-011 "A reference algorithm needs an expiry
  condition", section "Decision": a simple dense reference is only valid
  inside a machine-enforced size ceiling.

Readings taken where the pages leave a step open (each is listed in the
design notes of the repository):

R1 selection is made on the logits (softmax is strictly increasing, so the
   set and its order are the same as on probabilities);
R2 ties are broken by the lower expert index during membership selection and
   the selected experts are emitted in rank order;
R3 "normalized top-k": full softmax over all experts, then each selected
   probability is divided by the sum of the selected ones;
R4 an optional float32 router bias is added to the logits before selection
   and softmax;
R5 low-bit weights are signed symmetric integer codes times an fp16 scale per
   group of 32 along the reduction dimension; packing is little-endian, code
   k of a row sits in byte k//2 (low nibble first) for int4 and in byte k//4
   at bit 2*(k%4) for int2; codes are two's complement;
R6 inside an expert segment of the permutation, rows are in ascending pair
   order (hence ascending token order);
R7 a stacked layer feeds ``x_{l+1} = act_round(x_l + moe_l(x_l))`` where the
   activation storage type rounds once per layer;
R8 route locality is measured on the token sequence t = 0..T-1 of one call:
   overlap with the previous token, and unions over consecutive blocks of B
   tokens (the last block may be shorter).

Parity unpinned: last-bit behaviour of exp/silu is not pinned by the pages
(only by closed forms and library special cases at tolerance level).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# Storage decoding.  These define what the stored bytes mean; they are exact.
# ----------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half
    of an IEEE binary32)."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.ascontiguousarray(bits).view(np.uint16).view(np.float16).astype(np.float64)


def decode_act(arr: np.ndarray, act: str) -> np.ndarray:
    """Activation / dense-weight storage -> float64.  ``act`` is 'f32' or
    'bf16' (bf16 arrays hold the raw uint16 bit patterns)."""
    if act == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if act == "bf16":
        return decode_bf16(arr)
    raise ValueError(f"unknown activation storage {act!r}")


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even) and return
    them as float64.  Used only at a stacked layer boundary (reading R7).
    Works on the significand directly so that there is exactly one rounding."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits in the binade 2**(e-1) .. 2**e; below
    # 2**-126 its values are subnormal, on the fixed grid 2**-133
    e = np.maximum(e, -125)
    q = np.rint(np.ldexp(v, 8 - e))
    return np.ldexp(q, e - 8)


def act_round(v: np.ndarray, act: str) -> np.ndarray:
    """Round float64 values to the activation storage type (as float64)."""
    if act == "f32":
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    if act == "bf16":
        return round_to_bf16(v)
    raise ValueError(act)


def bf16_bits_of(v: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are already exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


WFMT_BITS = {"int4_g32": 4, "int2_g32": 2}
GROUP = 32


def unpack_codes(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Unpack little-endian two's-complement codes along the last axis
    (reading R5): element k sits in byte k*bits//8 at bit (k*bits) % 8."""
    packed = np.asarray(packed, dtype=np.uint8)
    per_byte = 8 // bits
    assert packed.shape[-1] * per_byte == K, (packed.shape, bits, K)
    out = np.empty(packed.shape[:-1] + (K,), dtype=np.int64)
    mask = (1 << bits) - 1
    for slot in range(per_byte):
        raw = (packed.astype(np.int64) >> (slot * bits)) & mask
        signed = np.where(raw >= (1 << (bits - 1)), raw - (1 << bits), raw)
        out[..., slot::per_byte] = signed
    return out


def dequantize(packed: np.ndarray, scale_bits: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Group dequantization w = q * s, one fp16 scale per 32 consecutive
    elements along the reduction axis (reading R5; low-bit storage is the
    first byte owner named in [P-019] "Why overlap alone cannot defeat the
    byte roofline")."""
    q = unpack_codes(packed, bits, K).astype(np.float64)
    s = decode_fp16(scale_bits)
    assert s.shape[-1] * GROUP == K
    return q * np.repeat(s, GROUP, axis=-1)


# ----------------------------------------------------------------------------
# Layer steps
# ----------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h] (+ bias[e]).

    The native router scores every expert from the token's representation
    ([P-019] "Hypothesis H2", [P-001] "Phase 1"); the optional bias is reading
    R4.  Inputs are float64 arrays x[T, H], Wr[E, H]."""
    logits = x @ w_router.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Exact top-k expert IDs in rank order, by the rank-count definition.

    rank(t, e) = #{e' : l[t,e'] > l[t,e]} + #{e' < e : l[t,e'] == l[t,e]};
    e is selected iff rank < k and then ids[t, rank] = e.  The index term is
    the equal-score rule of [P-017] "Tie handling belongs to membership"
    applied during membership (reading R2); rank order is required by
    [P-021] "The key equivalence — and where it breaks".  -0.0 == +0.0 by
    IEEE comparison; non-finite logits are rejected."""
    logits = np.asarray(logits, dtype=np.float64)
    if not np.all(np.isfinite(logits)):
        raise ValueError("non-finite router logits")
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.full((T, k), -1, dtype=np.int64)
    idx = np.arange(E)
    lower = idx[None, :] < idx[:, None]          # [e, e'] : e' < e
    chunk = max(1, (1 << 22) // (E * E))
    for t0 in range(0, T, chunk):
        l = logits[t0:t0 + chunk]                # [c, E]
        li = l[:, :, None]                       # candidate e
        lj = l[:, None, :]                       # competitor e'
        rank = (lj > li).sum(axis=2) + ((lj == li) & lower[None]).sum(axis=2)
        for c in range(l.shape[0]):
            sel = np.nonzero(rank[c] < k)[0]
            ids[t0 + c, rank[c, sel]] = sel
    assert (ids >= 0).all()
    return ids


def route_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """float32-router semantics of [P-001] "Phase 1" in float64: a softmax
    over all experts, then the selected probabilities renormalized to sum to
    one (reading R3).  Returns w[T, k] aligned with ``ids``."""
    logits = np.asarray(logits, dtype=np.float64)
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


@dataclass
class Permutation:
    counts: np.ndarray       # [E]    rows per expert
    offsets: np.ndarray      # [E+1]  exclusive scan of counts
    sorted_pair: np.ndarray  # [T*k]  row -> pair index p = t*k + j
    pair_row: np.ndarray     # [T*k]  pair index -> row
    active: np.ndarray       # [n_active] experts with count > 0, ascending
    n_active: int


def permutation(ids: np.ndarray, E: int) -> Permutation:
    """Group token rows by expert ([P-019] "Why overlap alone cannot defeat
    the byte roofline": grouping rows by expert; "Hypothesis H5": the block
    union deduplicated across rows).  A stable counting sort: pairs are
    visited in ascending p and appended to their expert's segment (reading
    R6), so each selected expert appears once in ``active``."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = np.zeros(E, dtype=np.int64)
    sorted_pair = np.full(P, -1, dtype=np.int64)
    pair_row = np.full(P, -1, dtype=np.int64)
    for p in range(P):
        e = flat[p]
        row = offsets[e] + fill[e]
        fill[e] += 1
        sorted_pair[row] = p
        pair_row[p] = row
    active = np.array([e for e in range(E) if counts[e] > 0], dtype=np.int64)
    return Permutation(counts, offsets, sorted_pair, pair_row, active, int(active.size))


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_intermediate(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """The SwiGLU intermediate silu(W_gate x) * (W_up x): gate and up read the
    same input and are combined before down can run ([P-019] "Hypothesis
    H4").  x_rows[m, H], W_gate/W_up[I, H] -> a[m, I]."""
    g = x_rows @ w_gate.T
    u = x_rows @ w_up.T
    return silu(g) * u


def down_projection(a_rows: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """y = W_down a for each row: a_rows[m, I], W_down[H, I] -> y[m, H]."""
    return a_rows @ w_down.T


def swiglu_expert(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                  w_down: np.ndarray) -> np.ndarray:
    """One routed expert: y = W_down (silu(W_gate x) * (W_up x)).  Shapes:
    x_rows[m, H], W_gate/W_up[I, H], W_down[H, I] (the layout whose parameter
    count [P-019] "Why overlap alone cannot defeat the byte roofline" prints);
    returns y[m, H]."""
    return down_projection(swiglu_intermediate(x_rows, w_gate, w_up), w_down)


class ExpertWeights:
    """Decoded view of per-expert weights in storage format.

    ``gate``/``up`` index as [E][I, H...] and ``down`` as [E][H, I...] in the
    storage layout: dense arrays hold f32 values or bf16 bit patterns; packed
    arrays hold uint8 codes with fp16 scale bit patterns alongside.  Any
    object supporting ``obj[e]`` -> numpy array works (the test harness uses
    lazy device views)."""

    def __init__(self, wfmt: str, act: str, H: int, I: int,
                 gate, up, down, gate_scale=None, up_scale=None, down_scale=None):
        self.wfmt, self.act, self.H, self.I = wfmt, act, H, I
        self.gate, self.up, self.down = gate, up, down
        self.gate_scale, self.up_scale, self.down_scale = gate_scale, up_scale, down_scale

    def _dense(self, arr, scale, K):
        if self.wfmt == "dense":
            return decode_act(np.asarray(arr), self.act)
        return dequantize(np.asarray(arr), np.asarray(scale), WFMT_BITS[self.wfmt], K)

    def expert(self, e: int):
        """float64 (W_gate[I,H], W_up[I,H], W_down[H,I]) of expert e."""
        H, I = self.H, self.I
        sc = (lambda s: None) if self.wfmt == "dense" else (lambda s: s[e])
        wg = self._dense(self.gate[e], sc(self.gate_scale), H)
        wu = self._dense(self.up[e], sc(self.up_scale), H)
        wd = self._dense(self.down[e], sc(self.down_scale), I)
        assert wg.shape == (I, H) and wu.shape == (I, H) and wd.shape == (H, I)
        return wg, wu, wd


def grouped_intermediate(x: np.ndarray, perm: Permutation, k: int, experts: ExpertWeights,
                         rows_of: Optional[np.ndarray] = None) -> np.ndarray:
    """SwiGLU intermediates in permuted row order: A[row] = silu(W_gate x_t) *
    (W_up x_t) for the expert and token of the row."""
    P = perm.sorted_pair.size
    A = np.full((P, experts.I), np.nan)
    for e in perm.active:
        rows = np.arange(int(perm.offsets[e]), int(perm.offsets[e + 1]))
        wg, wu, _ = experts.expert(int(e))
        A[rows] = swiglu_intermediate(x[perm.sorted_pair[rows] // k], wg, wu)
    return A


def grouped_down(A: np.ndarray, perm: Permutation, experts: ExpertWeights) -> np.ndarray:
    """Y[row] = W_down[e(row)] A[row] in permuted row order."""
    Y = np.full((A.shape[0], experts.H), np.nan)
    for e in perm.active:
        rows = np.arange(int(perm.offsets[e]), int(perm.offsets[e + 1]))
        _, _, wd = experts.expert(int(e))
        Y[rows] = down_projection(A[rows], wd)
    return Y


def grouped_ffn(x: np.ndarray, perm: Permutation, k: int, experts: ExpertWeights,
                only_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-pair expert outputs written to separate result slots in permuted
    row order: Y[row] = expert_{e(row)}(x[token(row)]) ([P-019] "Hypothesis
    H4": separate result slots).  Each active expert's weights are read once
    for all of its rows.  ``only_rows`` (sorted row indices) restricts the
    evaluation for sampled checks; the other rows are NaN."""
    P = perm.sorted_pair.size
    H = x.shape[1]
    Y = np.full((P, H), np.nan)
    want = None if only_rows is None else set(int(r) for r in only_rows)
    for e in perm.active:
        r0, r1 = int(perm.offsets[e]), int(perm.offsets[e + 1])
        rows = np.arange(r0, r1)
        if want is not None:
            rows = np.array([r for r in rows if r in want], dtype=np.int64)
            if rows.size == 0:
                continue
        tokens = perm.sorted_pair[rows] // k
        wg, wu, wd = experts.expert(int(e))
        Y[rows] = swiglu_expert(x[tokens], wg, wu, wd)
    return Y


def combine(Y: np.ndarray, pair_row: np.ndarray, w: np.ndarray,
            residual: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = residual[t] + sum_{j=0}^{k-1} w[t, j] * Y[pair_row[t*k + j]],
    accumulated in ascending route rank j ([P-019] "Hypothesis H4": the final
    weighted sum follows a deterministic route-rank order)."""
    T, k = w.shape
    H = Y.shape[1]
    out = np.zeros((T, H)) if residual is None else np.array(residual, dtype=np.float64)
    for j in range(k):
        out = out + w[:, j:j + 1] * Y[pair_row.reshape(T, k)[:, j]]
    return out


@dataclass
class LayerResult:
    logits: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    perm: Permutation
    Y: np.ndarray
    out: np.ndarray          # float64, before any storage rounding


def moe_layer(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
              experts: ExpertWeights, k: int, residual: Optional[np.ndarray] = None,
              only_tokens: Optional[Sequence[int]] = None) -> LayerResult:
    """The routed layer end to end, all in float64 on decoded inputs:
    router logits -> exact top-k -> renormalized weights -> permutation by
    expert -> grouped SwiGLU experts -> rank-order combine (+ residual).

    ``only_tokens`` limits the expert evaluation (not the routing) to a
    sample of tokens; rows and outputs of the other tokens are NaN."""
    E = w_router.shape[0]
    logits = router_logits(x, w_router, bias)
    ids = select_topk(logits, k)
    w = route_weights(logits, ids)
    perm = permutation(ids, E)
    only_rows = None
    if only_tokens is not None:
        tok = np.asarray(only_tokens, dtype=np.int64)
        pairs = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
        only_rows = np.sort(perm.pair_row[pairs])
    Y = grouped_ffn(x, perm, k, experts, only_rows)
    out = combine(Y, perm.pair_row, w, residual)
    return LayerResult(logits, ids, w, perm, Y, out)


# ----------------------------------------------------------------------------
# Bounded dense brute force ([P-017] "The dense-parity property" with the
# machine-enforced ceiling of [P-011] "Decision").
# ----------------------------------------------------------------------------

DENSE_ORACLE_CEILING = 1 << 30   # T * E * H * I multiply-adds per projection


def dense_moe_layer(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray],
                    experts: ExpertWeights, k: int,
                    residual: Optional[np.ndarray] = None) -> np.ndarray:
    """Evaluate EVERY expert on EVERY token and mix with a dense gate matrix
    G[t, e] (the renormalized weight for selected experts, 0 elsewhere).
    It does not use the permutation at all, so it cross-checks the sparse
    path.  Refuses sizes above the ceiling before doing any work."""
    T, H = x.shape
    E = w_router.shape[0]
    if T * E * H * experts.I > DENSE_ORACLE_CEILING:
        raise ValueError("dense oracle ceiling exceeded")
    logits = router_logits(x, w_router, bias)
    # membership by sorting on (-logit, index): a different algorithm than the
    # rank count used by select_topk
    order = np.lexsort((np.broadcast_to(np.arange(E), logits.shape), -logits), axis=1)
    ids = order[:, :k]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    p = p / p.sum(axis=1, keepdims=True)
    G = np.zeros((T, E))
    for t in range(T):
        denom = sum(p[t, e] for e in ids[t])
        for e in ids[t]:
            G[t, e] = p[t, e] / denom
    out = np.zeros((T, H)) if residual is None else np.array(residual, dtype=np.float64)
    for e in range(E):
        wg, wu, wd = experts.expert(e)
        ye = swiglu_expert(x, wg, wu, wd)
        out = out + G[:, e:e + 1] * ye
    return out


# ----------------------------------------------------------------------------
# Stacked layers (reading R7; sequential per [P-019] "Hypothesis H6")
# ----------------------------------------------------------------------------


def moe_stack(x0: np.ndarray, layers: Sequence[Callable[[], tuple]], k: int,
              act: str, only_tokens: Optional[Sequence[int]] = None):
    """x_{l+1} = act_round(x_l + moe_l(x_l)).  ``layers[l]()`` returns
    (w_router float64, bias or None, ExpertWeights) for layer l.  Tokens do
    not interact inside the layer, so ``only_tokens`` runs the stack on a
    subset of rows exactly.  Returns the list of layer inputs x_0..x_L
    (float64 values on the activation grid)."""
    x = np.asarray(x0, dtype=np.float64)
    if only_tokens is not None:
        x = x[np.asarray(only_tokens, dtype=np.int64)]
    xs = [x]
    for get in layers:
        wr, bias, experts = get()
        r = moe_layer(x, wr, bias, experts, k, residual=x)
        x = act_round(r.out, act)
        xs.append(x)
    return xs


# ----------------------------------------------------------------------------
# Near ties (how route mismatches are classified)
# ----------------------------------------------------------------------------


def near_tie_tokens(logits: np.ndarray, k: int, rel: float = 1e-6) -> np.ndarray:
    """Boolean mask of tokens whose top-(k+1) logits contain an adjacent gap
    0 < l_(r) - l_(r+1) < rel * max(|l_(r)|, |l_(r+1)|) for some r < k.
    Exact ties (gap 0) are not near ties: the index rule decides them."""
    T, E = logits.shape
    kk = min(k + 1, E)
    s = -np.sort(-logits, axis=1)[:, :kk]
    a, b = s[:, :-1], s[:, 1:]
    gap = a - b
    thr = rel * np.maximum(np.abs(a), np.abs(b))
    return ((gap > 0) & (gap < thr)).any(axis=1)


# ----------------------------------------------------------------------------
# Accounting ([P-019] "Why overlap alone cannot defeat the byte roofline",
# [P-021] "Do not store every large activation", [P-019] "Hypothesis H7")
# ----------------------------------------------------------------------------


def params_per_expert(H: int, I: int) -> int:
    """gate [I x H] + up [I x H] + down [H x I]."""
    return H * I + H * I + I * H


def param_uses_per_token(layers: int, k: int, H: int, I: int) -> int:
    return layers * k * params_per_expert(H, I)


def ideal_payload_bytes_per_token(layers: int, k: int, H: int, I: int, bits: int) -> float:
    """Payload only: no scales, metadata or alignment."""
    return param_uses_per_token(layers, k, H, I) * bits / 8


def expert_record_bytes(H: int, I: int, wfmt: str, act_bytes: int = 2) -> int:
    """Bytes of one expert (gate+up+down) as stored here: dense at
    ``act_bytes`` per weight, or packed codes plus one fp16 scale per 32."""
    n = params_per_expert(H, I)
    if wfmt == "dense":
        return n * act_bytes
    bits = WFMT_BITS[wfmt]
    return n * bits // 8 + (n // GROUP) * 2


def intermediate_bytes(k: int, I: int, layers: int = 1) -> int:
    """float32 SwiGLU intermediate [k, I] per token."""
    return k * I * 4 * layers


def route_label_bytes(k: int, layers: int) -> int:
    """int32 ID + float32 weight per selected expert."""
    return k * (4 + 4) * layers


def breakeven_unique_experts(k: int, tau: float) -> float:
    """Average unique experts per layer below which a verifier block reads
    fewer routed bytes per accepted token than top-k decoding."""
    return k * tau


def unique_experts(ids: np.ndarray) -> int:
    return int(np.unique(np.asarray(ids)).size)


def repeat_fraction(ids: np.ndarray) -> float:
    """Fraction of the T*k (token, slot) pairs whose expert is also chosen by
    at least one other token of the block."""
    flat = np.asarray(ids).reshape(-1)
    vals, cnt = np.unique(flat, return_counts=True)
    rep = set(vals[cnt >= 2].tolist())
    return float(np.mean([e in rep for e in flat]))


# ----------------------------------------------------------------------------
# Route locality of a token sequence ([P-019] "Hypothesis H7: DFlash block
# size must follow I/O cost" and the routing measurements of its "Gate B -
# trace-only locality": overlap with the previous token, block unions for
# block sizes 2-5, unique experts per block, per-layer skew, and the routed-
# byte break-even U_B < 10 tau(B)).  Reading R8: tokens are in sequence
# order t = 0..T-1; S_t is the set of experts token t selects; a block of
# size B is tokens bB .. min(T, bB+B)-1 (the last block may be shorter).
# ----------------------------------------------------------------------------


def overlap_with_previous(ids: np.ndarray) -> np.ndarray:
    """|S_t intersect S_{t-1}| for t >= 1; 0 for t = 0."""
    ids = np.asarray(ids)
    out = np.zeros(ids.shape[0], dtype=np.int64)
    for t in range(1, ids.shape[0]):
        out[t] = len(set(ids[t].tolist()) & set(ids[t - 1].tolist()))
    return out


def block_unique(ids: np.ndarray, B: int) -> np.ndarray:
    """|S_bB union ... union S_min(T,bB+B)-1| for every block b."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    return np.array([len(set(ids[b:b + B].reshape(-1).tolist())) for b in range(0, T, B)],
                    dtype=np.int64)


def layer_skew(counts: np.ndarray, k: int, T: int) -> float:
    """Largest expert load over the mean load per expert (T*k / E)."""
    counts = np.asarray(counts)
    return float(counts.max() / (T * k / counts.size))


def breakeven_tau(mean_unique: float, k: int) -> float:
    """Accepted tokens per block at which a block with mean_unique unique
    experts per layer reads as many routed bytes per accepted token as top-k
    decoding (the equality case of U_B < k tau(B))."""
    return mean_unique / k
