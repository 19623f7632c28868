"""The five workloads of the routed-MoE layer.

Geometry of the full-size layer (hidden 2,560, 512 routed experts, top-10,
SwiGLU intermediate 640, 48 layers) is the one stated in "Agent Field Notes —
full corpus", AFN-019, section "Why overlap alone cannot defeat the byte
roofline".  The workloads are:

1. ``tiny``      T=16, H=256, E=16, k=2, I=64, fp32, seed 0, no bias.
2. ``decode``    T=8 decode batch, bf16, near-uniform routing, seed 1.
3. ``prefill``   T=4096 prefill/replay, bf16, Zipf(1.1) router bias, seed 2.
4. ``stack_int4`` 48 layers, T=512, int4 group-32 experts, residual, seed 3.
5. ``verify_int2`` 48 layers, T=16 verifier block, int2 group-32 experts,
   hot-set router bias so that most of each token's experts repeat across the
   block, residual, seed 4.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    I: int
    k: int
    act: str          # 'f32' | 'bf16'  (x, router weights, dense expert weights)
    wfmt: str         # 'dense' | 'int4_g32' | 'int2_g32'
    layers: int
    seed: int
    bias: str         # 'none' | 'zipf' | 'hotset'
    residual: bool
    x_std: float = 1.0
    router_std: float = 0.02
    expert_std: float = 0.02
    zipf_s: float = 1.1
    zipf_scale: float = 0.5
    hot_count: int = 6
    hot_bias: float = 4.0

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


CONFIGS = {
    1: MoEConfig("tiny", T=16, H=256, E=16, I=64, k=2, act="f32", wfmt="dense",
                 layers=1, seed=0, bias="none", residual=False),
    2: MoEConfig("decode", T=8, H=2560, E=512, I=640, k=10, act="bf16", wfmt="dense",
                 layers=1, seed=1, bias="none", residual=False),
    3: MoEConfig("prefill", T=4096, H=2560, E=512, I=640, k=10, act="bf16", wfmt="dense",
                 layers=1, seed=2, bias="zipf", residual=False),
    # The stacked workloads state no expert weight distribution.  Their layers
    # feed x + moe(x) forward with no normalization, and with N(0, 0.02^2)
    # experts the MoE term grows with the square of the activations: on the
    # GPU the 48-layer int2 verifier block overflowed bf16 near layer 23 and
    # was NaN from layer ~29 on (its routes then collapsed to 10 experts),
    # while N(0, 0.01^2) keeps the residual stream at rms 1.00-1.01 through
    # all 48 layers of both stacks.
    4: MoEConfig("stack_int4", T=512, H=2560, E=512, I=640, k=10, act="bf16",
                 wfmt="int4_g32", layers=48, seed=3, bias="none", residual=True,
                 expert_std=0.01),
    5: MoEConfig("verify_int2", T=16, H=2560, E=512, I=640, k=10, act="bf16",
                 wfmt="int2_g32", layers=48, seed=4, bias="hotset", residual=True,
                 expert_std=0.01),
}


def get_config(n_or_name) -> MoEConfig:
    if isinstance(n_or_name, int):
        return CONFIGS[n_or_name]
    for c in CONFIGS.values():
        if c.name == n_or_name:
            return c
    raise KeyError(n_or_name)
