"""Device buffers for one layer shape (torch supplies the memory; every step
of the layer runs in libmoe.so)."""
from __future__ import annotations

import torch

from . import _abi


class MoELayerBuffers:
    """Outputs, permutation arrays and workspace for a shape, on one device."""

    def __init__(self, T, H, E, I, top_k, act="bf16", wfmt="dense", device="cuda", tiled=False,
                 check_finite=False, fused=False):
        flags = ((_abi.MOE_F_TILED_WEIGHTS if tiled else 0) | (_abi.MOE_F_CHECK_FINITE if check_finite else 0)
                 | (_abi.MOE_F_FUSED_FFN if fused else 0))
        self.shape = _abi.make_shape(T, H, E, I, top_k, act, wfmt, flags)
        self.T, self.H, self.E, self.I, self.k = T, H, E, I, top_k
        self.act = act
        dt = torch.float32 if act == "f32" else torch.bfloat16
        P = T * top_k
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_ids = torch.empty((T, top_k), **i32)
        self.topk_w = torch.empty((T, top_k), dtype=torch.float32, device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_pair = torch.empty(P, **i32)
        self.pair_row = torch.empty(P, **i32)
        self.active = torch.empty(E, **i32)
        self.n_active = torch.empty(1, **i32)
        self.y = torch.empty((P, H), dtype=dt, device=device)
        self.h = torch.empty((P, I), dtype=dt, device=device)
        self.out = torch.empty((T, H), dtype=dt, device=device)
        self.ws_bytes = _abi.moe_workspace_size(self.shape)
        self.workspace = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)
        self.perm = _abi.make_perm(self.counts, self.offsets, self.sorted_pair, self.pair_row,
                                   self.active, self.n_active)

    def route(self, x, w_router, bias=None, logits=True, stream=None):
        return _abi.moe_route(self.shape, x, w_router, bias, self.topk_ids, self.topk_w,
                              self.logits if logits else None, self.workspace, self.ws_bytes,
                              stream)

    def route_permute(self, x, w_router, bias=None, logits=True, stream=None):
        """moe_route_permute: routes into topk_ids / topk_w (and logits), the
        permutation into this buffer's perm, the tile plan into the workspace."""
        return _abi.moe_route_permute(self.shape, x, w_router, bias, self.topk_ids, self.topk_w,
                                      self.logits if logits else None, self.perm, self.workspace,
                                      self.ws_bytes, stream)

    def ffn_down_combine(self, experts, residual=None, out=None, h=None, stream=None):
        """moe_ffn_down_combine from this buffer's h into out (default self.out)."""
        return _abi.moe_ffn_down_combine(self.shape, self.h if h is None else h, experts, self.perm,
                                         self.topk_w, residual, self.out if out is None else out,
                                         self.workspace, self.ws_bytes, stream)

    def permute(self, topk_ids=None, stream=None):
        return _abi.moe_permute(self.shape, self.topk_ids if topk_ids is None else topk_ids,
                                self.perm, self.workspace, self.ws_bytes, stream)

    def ffn_fused(self, x, experts, wave_tiles=0, item_clock=None, perm=None, stream=None):
        """moe_ffn_fused into self.y (needs fused=True and tiled=True)."""
        return _abi.moe_ffn_fused(self.shape, x, experts, self.perm if perm is None else perm, self.y,
                                  wave_tiles, item_clock, self.workspace, self.ws_bytes, stream)

    def stage_experts(self, src, dst, parts=None, stream=None):
        """Copy the records of this call's active experts (the permutation
        already built by permute()) from `src` to `dst` (moe_experts structs;
        src may be pinned host memory); `parts` selects gate/up and/or down."""
        return _abi.moe_stage_experts(self.shape, src, dst, self.perm, parts, stream)

    def route_locality(self, topk_ids=None, stream=None):
        """(overlap_prev [T], [block_unique for B = 1..5]) as device tensors."""
        if not hasattr(self, "overlap_prev"):
            dev = self.topk_ids.device
            self.overlap_prev = torch.empty(self.T, dtype=torch.int32, device=dev)
            self.block_unique = torch.empty(max(_abi.moe_route_locality_blocks(self.T), 1),
                                            dtype=torch.int32, device=dev)
        _abi.moe_route_locality(self.shape, self.topk_ids if topk_ids is None else topk_ids,
                                self.overlap_prev, self.block_unique, stream)
        parts, o = [], 0
        for B in range(1, 6):
            nb = (self.T + B - 1) // B
            parts.append(self.block_unique[o:o + nb])
            o += nb
        return self.overlap_prev, parts

    def grouped_ffn(self, x, experts, perm=None, stream=None):
        return _abi.moe_grouped_ffn(self.shape, x, experts, self.perm if perm is None else perm,
                                    self.y, self.workspace, self.ws_bytes, stream)

    def ffn_gate_up(self, x, experts, perm=None, h=None, stream=None):
        return _abi.moe_ffn_gate_up(self.shape, x, experts, self.perm if perm is None else perm,
                                    self.h if h is None else h, self.workspace, self.ws_bytes,
                                    stream)

    def ffn_down(self, experts, h=None, y=None, stream=None):
        return _abi.moe_ffn_down(self.shape, self.h if h is None else h, experts,
                                 self.y if y is None else y, self.workspace, self.ws_bytes, stream)

    def combine(self, residual=None, y=None, pair_row=None, topk_w=None, out=None, stream=None):
        return _abi.moe_combine(self.shape, self.y if y is None else y,
                                self.pair_row if pair_row is None else pair_row,
                                self.topk_w if topk_w is None else topk_w, residual,
                                self.out if out is None else out, stream)

    def layer(self, x, w_router, bias, experts, residual=None, out=None, use_perm=True,
              stream=None):
        return _abi.moe_layer(self.shape, x, w_router, bias, experts, residual,
                              self.out if out is None else out, self.topk_ids, self.topk_w,
                              self.perm if use_perm else None, self.workspace, self.ws_bytes,
                              stream)
