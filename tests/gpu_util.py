"""Helpers shared by the GPU parity tests (not a test module).

Direction of data: the seeded generator makes the inputs on the device; the
oracle reads those input bytes back and computes expected values; HIP stages
may be fed oracle outputs (teacher forcing).  No HIP output is ever an oracle
input."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import sparse_moe_routed_amd as M
from moe_inputs import MoEConfig, expert_view_to_numpy, make_layer, tensor_to_numpy_storage
from oracle import moe_oracle as O

DEV = torch.device("cuda")

# output tolerances (bf16: max-abs and relative L2; float32: max-abs)
TOL_BF16_ABS, TOL_BF16_RL2 = 2e-2, 1e-2
TOL_F32_ABS = 1e-5
TOL_W = 1e-5


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def np_of(t):
    return tensor_to_numpy_storage(t)


def decode(t, act):
    return O.decode_act(np_of(t), act)


def act_torch(act):
    return torch.float32 if act == "f32" else torch.bfloat16


def to_act_tensor(v64: np.ndarray, act: str) -> torch.Tensor:
    """float64 values already on the activation grid -> device tensor."""
    if act == "f32":
        return torch.from_numpy(v64.astype(np.float32)).to(DEV)
    bits = O.bf16_bits_of(v64)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@dataclass
class Case:
    cfg: MoEConfig
    li: object              # LayerInputs on the device
    x64: np.ndarray
    wr64: np.ndarray
    bias64: np.ndarray | None
    ex_oracle: O.ExpertWeights
    ex_gpu: object
    tiled_keep: dict | None = None
    ex_gpu_tiled: object = None

    def experts(self, tiled: bool):
        return self.ex_gpu_tiled if tiled else self.ex_gpu


def tiled_ok(cfg: MoEConfig) -> bool:
    return cfg.act == "bf16" and cfg.I % 128 == 0


def make_tiled(case: Case) -> None:
    """Convert the case's row-major expert weights with moe_tile_experts."""
    cfg, ex = case.cfg, case.li.experts
    dst = {n: (None if t is None else torch.empty_like(t)) for n, t in ex.items()}
    exd = M.make_experts(dst["gate"], dst["up"], dst["down"], dst["gate_scale"], dst["up_scale"],
                         dst["down_scale"])
    M.moe_tile_experts(M.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt),
                       case.ex_gpu, exd)
    case.tiled_keep, case.ex_gpu_tiled = dst, exd


def make_case(cfg: MoEConfig, layer: int = 0, x: torch.Tensor | None = None) -> Case:
    li = make_layer(cfg, layer=layer, device=DEV, with_x=x is None)
    if x is not None:
        li.x = x
    ex = li.experts
    V = expert_view_to_numpy
    ex_oracle = O.ExpertWeights(cfg.wfmt, cfg.act, cfg.H, cfg.I, V(ex["gate"]), V(ex["up"]),
                                V(ex["down"]), V(ex["gate_scale"]) if ex["gate_scale"] is not None else None,
                                V(ex["up_scale"]) if ex["up_scale"] is not None else None,
                                V(ex["down_scale"]) if ex["down_scale"] is not None else None)
    ex_gpu = M.make_experts(ex["gate"], ex["up"], ex["down"], ex["gate_scale"], ex["up_scale"],
                            ex["down_scale"])
    bias64 = None if li.bias is None else li.bias.double().cpu().numpy()
    case = Case(cfg, li, decode(li.x, cfg.act), decode(li.w_router, cfg.act), bias64, ex_oracle, ex_gpu)
    if tiled_ok(cfg):
        make_tiled(case)
    return case


def buffers(cfg: MoEConfig, tiled: bool = False, fused: bool = False) -> M.MoELayerBuffers:
    return M.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt, device=DEV,
                             tiled=tiled, fused=fused)


def check_routes(ids_gpu, w_gpu, logits64, ids_ref, w_ref, k):
    """Bit-exact IDs except on near-tie tokens; weights within TOL_W."""
    near = O.near_tie_tokens(logits64, k)
    mism = (ids_gpu != ids_ref).any(axis=1)
    bad = mism & ~near
    assert not bad.any(), f"route mismatch on tokens without near ties: {np.nonzero(bad)[0][:8]}"
    ok = ~mism
    werr = float(np.abs(w_gpu[ok] - w_ref[ok]).max()) if ok.any() else 0.0
    assert werr <= TOL_W, f"weight error {werr}"
    return dict(mismatch=int(mism.sum()), near_ties=int(near.sum()), max_w_err=werr), ~mism


def check_values(got64, ref64, act, what, scaled=False):
    """max-abs and rel-L2 of GPU values against float64 oracle values.

    scaled=True (rows whose scale grows beyond 1, as in the 48-layer residual
    stacks, where the activations and with them the expert outputs grow layer
    by layer): the bf16 max-abs bound holds at unit scale and is applied row
    by row to max_n |got - ref| / max(1, rms(ref row)).  Rounding the bf16
    intermediate and outputs gives errors proportional to the size of the
    values (a bf16 value v alone is off by up to |v| * 2^-9, more than 2e-2
    once |v| > 10.24), so a fixed absolute bound stops being attainable for
    rows of a few units; for rows of rms <= 1 the scaled bound is the
    absolute one."""
    got64 = np.asarray(got64, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    assert got64.shape == ref64.shape
    assert np.isfinite(got64).all(), f"{what}: non-finite GPU values"
    err = np.abs(got64 - ref64)
    mx = float(err.max()) if err.size else 0.0
    rl2 = float(np.linalg.norm(got64 - ref64) / max(np.linalg.norm(ref64), 1e-300)) if err.size else 0.0
    out = dict(max_abs=mx, rel_l2=rl2)
    if act == "f32":
        assert mx <= TOL_F32_ABS, f"{what}: max-abs {mx} (rel-L2 {rl2})"
    elif scaled:
        r2 = ref64.reshape(-1, ref64.shape[-1]) if ref64.ndim else ref64.reshape(1, 1)
        e2 = err.reshape(r2.shape)
        row_rms = np.sqrt(np.mean(r2 ** 2, axis=1)) if r2.size else np.zeros(0)
        ms = float((e2.max(axis=1) / np.maximum(1.0, row_rms)).max()) if r2.size else 0.0
        rms = float(np.sqrt(np.mean(ref64 ** 2))) if err.size else 0.0
        out["max_scaled"], out["rms_ref"] = ms, rms
        assert ms <= TOL_BF16_ABS and rl2 <= TOL_BF16_RL2, \
            f"{what}: max over rows of max-abs / max(1, row rms) = {ms} (max-abs {mx}, rms {rms}), rel-L2 {rl2}"
    else:
        assert mx <= TOL_BF16_ABS and rl2 <= TOL_BF16_RL2, f"{what}: max-abs {mx} rel-L2 {rl2}"
    return out


def cxx_oracle_layer(case: Case, tokens=None):
    """The layer through the C++ float64 oracle on the case's input bytes,
    for all tokens or for the rows `tokens` (every step is per token except
    the row order of the permutation, so a subset gives those tokens' exact
    outputs).  The C++ oracle decodes the activation and router bytes itself
    and its own router picks the experts whose weights are copied to the host
    (the other experts' pages stay zero and are never read)."""
    from oracle import oracle_c as C
    cfg = case.cfg
    xs = np_of(case.li.x)
    if tokens is not None:
        xs = xs[np.asarray(tokens)]
    x64 = C.decode_act_c(xs, cfg.act)
    wr64 = C.decode_act_c(np_of(case.li.w_router), cfg.act)
    need = np.unique(C.routes_c(x64, wr64, case.bias64, cfg.k)[1])
    host = host_experts(case.li.experts, need)
    res = x64 if cfg.residual else None
    return C.moe_layer_c(x64, wr64, case.bias64, host, cfg.wfmt, cfg.act, cfg.k, res)


def host_experts(ex: dict, need) -> dict:
    """Host storage arrays of the expert tensors (row-major) with the experts
    in `need` copied from the device and every other expert zero (untouched
    pages cost no memory)."""
    host = {}
    for n, t in ex.items():
        if t is None:
            host[n] = None
            continue
        st = tensor_to_numpy_storage(t[:1])
        a = np.zeros((t.shape[0],) + st.shape[1:], dtype=st.dtype)
        for e in need:
            a[int(e)] = tensor_to_numpy_storage(t[int(e)])
        host[n] = a
    return host


def check_oracles_agree(ids_numpy, ids_cxx, logits64, k):
    """The two oracles' routes: identical outside near-tie tokens."""
    near = O.near_tie_tokens(logits64, k)
    bad = (np.asarray(ids_numpy) != np.asarray(ids_cxx)).any(axis=1) & ~near
    assert not bad.any(), f"numpy and C++ oracle routes differ on tokens {np.nonzero(bad)[0][:8]}"
