"""Seeded synthetic input generation (torch is used as a random source and for
storage only).

Recipe (identical on every device; values drawn on different devices differ
because torch's CPU and GPU generators differ, so a check always reads the
bytes that were actually generated):

* every tensor has its own generator, keyed by (config seed, tensor name,
  layer, batch) through CRC32, so tensors never share a stream;
* normals are drawn in float32, scaled by the stated standard deviation and
  rounded once (round-to-nearest-even) to the storage type; the rounded values
  are the inputs;
* expert weights are drawn in blocks of up to 32 experts, in expert order,
  from the (tensor, layer) stream;
* low-bit experts: signed symmetric codes, qmax = 2**(b-1) - 1 (int4 -> +-7,
  int2 -> +-1), one fp16 scale per 32 consecutive elements of the reduction
  axis, s = fp16(max|w| / qmax), q = clamp(round_half_even(w / s), +-qmax)
  (q = 0 where s = 0); codes are packed little-endian in two's complement:
  code k of a row at byte k*b//8, bit (k*b) % 8.  The (code, scale) pairs are
  the weights; the normals they came from are discarded;
* router bias: none; 'zipf' -> bias[e] = zipf_scale * ln(r^-s / sum_r' r'^-s)
  with r = e + 1; 'hotset' -> hot_count experts drawn per layer get hot_bias,
  all others 0.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import MoEConfig

_ACT_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
_BITS = {"int4_g32": 4, "int2_g32": 2}
GROUP = 32
EXPERT_BLOCK = 32


def _generator(cfg: MoEConfig, tensor: str, layer: int, batch: int, device) -> torch.Generator:
    key = zlib.crc32(f"{cfg.seed}/{tensor}/{layer}/{batch}".encode()) + (cfg.seed << 32)
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(key)
    return g


def _normal(shape, std, g, device) -> torch.Tensor:
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def make_x(cfg: MoEConfig, device="cpu", batch: int = 0, T: Optional[int] = None) -> torch.Tensor:
    """Activations x[T, H] in the activation storage type."""
    T = cfg.T if T is None else T
    g = _generator(cfg, "x", 0, batch, device)
    return _normal((T, cfg.H), cfg.x_std, g, device).to(_ACT_DTYPE[cfg.act])


def make_router(cfg: MoEConfig, layer: int = 0, device="cpu"):
    """(W_router[E, H] in the activation type, bias float32 [E] or None)."""
    g = _generator(cfg, "router", layer, 0, device)
    wr = _normal((cfg.E, cfg.H), cfg.router_std, g, device).to(_ACT_DTYPE[cfg.act])
    bias = None
    if cfg.bias == "zipf":
        r = np.arange(1, cfg.E + 1, dtype=np.float64)
        w = r ** (-cfg.zipf_s)
        w = w / w.sum()
        bias = torch.tensor(cfg.zipf_scale * np.log(w), dtype=torch.float32, device=device)
    elif cfg.bias == "hotset":
        gh = _generator(cfg, "hotset", layer, 0, "cpu")
        hot = torch.randperm(cfg.E, generator=gh)[: cfg.hot_count]
        b = torch.zeros(cfg.E, dtype=torch.float32)
        b[hot] = cfg.hot_bias
        bias = b.to(device)
    elif cfg.bias != "none":
        raise ValueError(cfg.bias)
    return wr, bias


def quantize_pack(w: torch.Tensor, bits: int):
    """Symmetric group-32 quantization of float32 w[..., K] along the last
    axis.  Returns (packed uint8 [..., K*bits/8], fp16 scales [..., K/32])."""
    K = w.shape[-1]
    assert K % GROUP == 0
    qmax = (1 << (bits - 1)) - 1
    grp = w.reshape(*w.shape[:-1], K // GROUP, GROUP)
    s16 = (grp.abs().amax(dim=-1) / qmax).to(torch.float16)
    s = s16.to(torch.float32).unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.where(s > 0, torch.round(grp / safe), torch.zeros_like(grp))
    q = q.clamp(-qmax, qmax).to(torch.int32).reshape(w.shape)
    per = 8 // bits
    u = (q & ((1 << bits) - 1)).reshape(*w.shape[:-1], K // per, per)
    packed = torch.zeros(u.shape[:-1], dtype=torch.int32, device=w.device)
    for i in range(per):
        packed = packed | (u[..., i] << (bits * i))
    return packed.to(torch.uint8), s16


def make_experts(cfg: MoEConfig, layer: int = 0, device="cpu", n_experts: Optional[int] = None):
    """Expert weights in storage format.  Dense: gate/up [E, I, H], down
    [E, H, I] in the activation type.  Low-bit: packed uint8 gate/up
    [E, I, H*b/8], down [E, H, I*b/8] plus fp16 scales [E, I, H/32],
    [E, H, I/32].  Returns dict with keys gate, up, down, gate_scale,
    up_scale, down_scale (scales None when dense)."""
    E = cfg.E if n_experts is None else n_experts
    out = {}
    for name, (rows, K) in (("gate", (cfg.I, cfg.H)), ("up", (cfg.I, cfg.H)),
                            ("down", (cfg.H, cfg.I))):
        g = _generator(cfg, name, layer, 0, device)
        blocks = [(e0, min(E, e0 + EXPERT_BLOCK)) for e0 in range(0, E, EXPERT_BLOCK)]
        if cfg.wfmt == "dense":
            t = torch.empty((E, rows, K), dtype=_ACT_DTYPE[cfg.act], device=device)
            for e0, e1 in blocks:
                t[e0:e1] = _normal((e1 - e0, rows, K), cfg.expert_std, g, device).to(t.dtype)
            out[name], out[name + "_scale"] = t, None
        else:
            bits = _BITS[cfg.wfmt]
            pk = torch.empty((E, rows, K * bits // 8), dtype=torch.uint8, device=device)
            sc = torch.empty((E, rows, K // GROUP), dtype=torch.float16, device=device)
            for e0, e1 in blocks:
                pk[e0:e1], sc[e0:e1] = quantize_pack(
                    _normal((e1 - e0, rows, K), cfg.expert_std, g, device), bits)
            out[name], out[name + "_scale"] = pk, sc
    return out


@dataclass
class LayerInputs:
    x: Optional[torch.Tensor]
    w_router: torch.Tensor
    bias: Optional[torch.Tensor]
    experts: dict


def make_layer(cfg: MoEConfig, layer: int = 0, device="cpu", with_x: bool = True,
               batch: int = 0) -> LayerInputs:
    x = make_x(cfg, device, batch) if with_x else None
    wr, bias = make_router(cfg, layer, device)
    return LayerInputs(x, wr, bias, make_experts(cfg, layer, device))


# ----------------------------------------------------------------------------
# Host views of storage bytes (for the checker side)
# ----------------------------------------------------------------------------


def tensor_to_numpy_storage(t: Optional[torch.Tensor]):
    """Storage bytes of a tensor as numpy: bf16/fp16 -> uint16 bit patterns,
    float32 -> float32, uint8 -> uint8."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class expert_view_to_numpy:
    """Lazy ``view[e]`` -> numpy storage of one expert (copies from device on
    demand, so only the experts a check needs cross PCIe)."""

    def __init__(self, t: Optional[torch.Tensor]):
        self.t = t

    def __getitem__(self, e):
        return tensor_to_numpy_storage(self.t[int(e)])
