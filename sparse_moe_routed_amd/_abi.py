"""ctypes binding of libmoe.so: argument marshalling only.

Every function has the name of the C entry point it calls.  Tensor
arguments may be torch tensors (their ``data_ptr()`` is passed), plain
integer addresses or None.  ``stream`` is a ``torch.cuda.Stream``, a raw
``hipStream_t`` integer, or None for torch's current stream.  A non-zero
status raises :class:`MoEError` unless ``check=False``.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_WF_DENSE, MOE_WF_INT4_G32, MOE_WF_INT2_G32 = 0, 1, 2
ACT = {"f32": MOE_DT_F32, "bf16": MOE_DT_BF16}
WFMT = {"dense": MOE_WF_DENSE, "int4_g32": MOE_WF_INT4_G32, "int2_g32": MOE_WF_INT2_G32}

STATUS = {
    0: "MOE_OK", 1: "MOE_E_NULL", 2: "MOE_E_SHAPE", 3: "MOE_E_DTYPE", 4: "MOE_E_FORMAT",
    5: "MOE_E_ALIGN", 6: "MOE_E_ALIAS", 7: "MOE_E_WORKSPACE", 8: "MOE_E_LIMIT",
    9: "MOE_E_DEVICE", 10: "MOE_E_FLAGS", 11: "MOE_E_NONFINITE", 12: "MOE_E_MEMORY",
}
EXPORTS = ("moe_workspace_size", "moe_status_str", "moe_tile_experts", "moe_route", "moe_permute",
           "moe_grouped_ffn", "moe_ffn_gate_up", "moe_ffn_down", "moe_ffn_fused",
           "moe_ffn_fused_items", "moe_device_clock_khz", "moe_combine", "moe_layer",
           "moe_stage_experts", "moe_route_locality_blocks", "moe_route_locality",
           "moe_stream_read", "moe_layer_noalloc", "moe_route_permute",
           "moe_ffn_down_combine")
MOE_F_TILED_WEIGHTS = 0x1
MOE_F_CHECK_FINITE = 0x2
MOE_F_FUSED_FFN = 0x4
MOE_STAGE_GATE_UP = 0x1
MOE_STAGE_DOWN = 0x2


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("top_k", ctypes.c_int32), ("act", ctypes.c_int32),
                ("wfmt", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class moe_experts(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("up_scale", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p)]


class moe_perm(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sorted_pair", ctypes.c_void_p), ("pair_row", ctypes.c_void_p),
                ("active", ctypes.c_void_p), ("n_active", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (fails loudly when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_moe_routed_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER
    lib.moe_workspace_size.argtypes = [P(moe_shape)]
    lib.moe_workspace_size.restype = sz
    lib.moe_status_str.argtypes = [i32]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_tile_experts.argtypes = [P(moe_shape), P(moe_experts), P(moe_experts), vp]
    lib.moe_route.argtypes = [P(moe_shape), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.argtypes = [P(moe_shape), vp, P(moe_perm), vp, sz, vp]
    lib.moe_grouped_ffn.argtypes = [P(moe_shape), vp, P(moe_experts), P(moe_perm), vp, vp, sz, vp]
    lib.moe_ffn_gate_up.argtypes = [P(moe_shape), vp, P(moe_experts), P(moe_perm), vp, vp, sz, vp]
    lib.moe_ffn_down.argtypes = [P(moe_shape), vp, P(moe_experts), vp, vp, sz, vp]
    lib.moe_combine.argtypes = [P(moe_shape), vp, vp, vp, vp, vp, vp]
    lib.moe_ffn_fused.argtypes = [P(moe_shape), vp, P(moe_experts), P(moe_perm), vp, i32, vp, vp,
                                  sz, vp]
    lib.moe_ffn_fused_items.argtypes = [P(moe_shape)]
    lib.moe_ffn_fused_items.restype = sz
    lib.moe_device_clock_khz.argtypes = [P(ctypes.c_int32)]
    lib.moe_stream_read.argtypes = [vp, sz, vp, vp]
    lib.moe_route_locality_blocks.argtypes = [i32]
    lib.moe_route_locality_blocks.restype = sz
    lib.moe_route_locality.argtypes = [P(moe_shape), vp, vp, vp, vp]
    lib.moe_stage_experts.argtypes = [P(moe_shape), P(moe_experts), P(moe_experts), P(moe_perm),
                                      ctypes.c_uint32, vp]
    lib.moe_layer.argtypes = [P(moe_shape), vp, vp, vp, P(moe_experts), vp, vp, vp, vp,
                              P(moe_perm), vp, sz, vp]
    lib.moe_layer_noalloc.argtypes = [P(moe_shape), vp, vp, vp, P(moe_experts), vp, vp, vp, vp,
                                      P(moe_perm), vp]
    lib.moe_route_permute.argtypes = [P(moe_shape), vp, vp, vp, vp, vp, vp, P(moe_perm), vp, sz, vp]
    lib.moe_ffn_down_combine.argtypes = [P(moe_shape), vp, P(moe_experts), P(moe_perm), vp, vp, vp,
                                         vp, sz, vp]
    for name in ("moe_tile_experts", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_ffn_gate_up",
                 "moe_ffn_down", "moe_ffn_fused", "moe_device_clock_khz", "moe_combine", "moe_layer",
                 "moe_route_locality", "moe_stage_experts", "moe_stream_read", "moe_layer_noalloc", "moe_route_permute",
                 "moe_ffn_down_combine"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(T, H, E, I, top_k, act="bf16", wfmt="dense", flags=0) -> moe_shape:
    return moe_shape(T, H, E, I, top_k, ACT.get(act, act), WFMT.get(wfmt, wfmt), flags)


def make_experts(gate, up, down, gate_scale=None, up_scale=None, down_scale=None) -> moe_experts:
    return moe_experts(ptr(gate), ptr(up), ptr(down), ptr(gate_scale), ptr(up_scale), ptr(down_scale))


def make_perm(counts, offsets, sorted_pair, pair_row, active, n_active) -> moe_perm:
    return moe_perm(ptr(counts), ptr(offsets), ptr(sorted_pair), ptr(pair_row), ptr(active),
                    ptr(n_active))


def _ret(status: int, where: str, check: bool) -> int:
    if check and status != 0:
        raise MoEError(status, where)
    return status


def moe_workspace_size(shape: moe_shape) -> int:
    return load().moe_workspace_size(ctypes.byref(shape))


def moe_status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def moe_tile_experts(shape, src, dst, stream=None, check=True) -> int:
    st = load().moe_tile_experts(ctypes.byref(shape), None if src is None else ctypes.byref(src),
                                 None if dst is None else ctypes.byref(dst), stream_handle(stream))
    return _ret(st, "moe_tile_experts", check)


def moe_route(shape, x, w_router, router_bias, topk_ids, topk_w, logits, workspace,
              workspace_bytes, stream=None, check=True) -> int:
    st = load().moe_route(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(router_bias),
                          ptr(topk_ids), ptr(topk_w), ptr(logits), ptr(workspace),
                          workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_route", check)


def moe_permute(shape, topk_ids, perm, workspace=None, workspace_bytes=0, stream=None,
                check=True) -> int:
    st = load().moe_permute(ctypes.byref(shape), ptr(topk_ids),
                            None if perm is None else ctypes.byref(perm), ptr(workspace),
                            workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_permute", check)


def moe_route_permute(shape, x, w_router, router_bias, topk_ids, topk_w, logits, perm, workspace,
                      workspace_bytes, stream=None, check=True) -> int:
    st = load().moe_route_permute(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(router_bias),
                                  ptr(topk_ids), ptr(topk_w), ptr(logits),
                                  None if perm is None else ctypes.byref(perm), ptr(workspace),
                                  workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_route_permute", check)


def moe_ffn_down_combine(shape, h, experts, perm, topk_w, residual, out, workspace, workspace_bytes,
                         stream=None, check=True) -> int:
    st = load().moe_ffn_down_combine(ctypes.byref(shape), ptr(h),
                                     None if experts is None else ctypes.byref(experts),
                                     None if perm is None else ctypes.byref(perm), ptr(topk_w),
                                     ptr(residual), ptr(out), ptr(workspace), workspace_bytes,
                                     stream_handle(stream))
    return _ret(st, "moe_ffn_down_combine", check)


def moe_grouped_ffn(shape, x, experts, perm, y, workspace, workspace_bytes, stream=None,
                    check=True) -> int:
    st = load().moe_grouped_ffn(ctypes.byref(shape), ptr(x),
                                None if experts is None else ctypes.byref(experts),
                                None if perm is None else ctypes.byref(perm), ptr(y),
                                ptr(workspace), workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_grouped_ffn", check)


def moe_ffn_gate_up(shape, x, experts, perm, h, workspace, workspace_bytes, stream=None,
                    check=True) -> int:
    st = load().moe_ffn_gate_up(ctypes.byref(shape), ptr(x),
                                None if experts is None else ctypes.byref(experts),
                                None if perm is None else ctypes.byref(perm), ptr(h),
                                ptr(workspace), workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_ffn_gate_up", check)


def moe_ffn_down(shape, h, experts, y, workspace, workspace_bytes, stream=None, check=True) -> int:
    st = load().moe_ffn_down(ctypes.byref(shape), ptr(h),
                             None if experts is None else ctypes.byref(experts), ptr(y),
                             ptr(workspace), workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_ffn_down", check)


def moe_ffn_fused(shape, x, experts, perm, y, wave_tiles, item_clock, workspace, workspace_bytes,
                  stream=None, check=True) -> int:
    st = load().moe_ffn_fused(ctypes.byref(shape), ptr(x),
                              None if experts is None else ctypes.byref(experts),
                              None if perm is None else ctypes.byref(perm), ptr(y), wave_tiles,
                              ptr(item_clock), ptr(workspace), workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_ffn_fused", check)


def moe_ffn_fused_items(shape) -> int:
    return int(load().moe_ffn_fused_items(ctypes.byref(shape)))


def moe_device_clock_khz(check=True) -> int:
    khz = ctypes.c_int32(0)
    st = load().moe_device_clock_khz(ctypes.byref(khz))
    _ret(st, "moe_device_clock_khz", check)
    return int(khz.value)


def moe_combine(shape, y, pair_row, topk_w, residual, out, stream=None, check=True) -> int:
    st = load().moe_combine(ctypes.byref(shape), ptr(y), ptr(pair_row), ptr(topk_w),
                            ptr(residual), ptr(out), stream_handle(stream))
    return _ret(st, "moe_combine", check)


def moe_layer(shape, x, w_router, router_bias, experts, residual, out, topk_ids, topk_w, perm,
              workspace, workspace_bytes, stream=None, check=True) -> int:
    st = load().moe_layer(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(router_bias),
                          None if experts is None else ctypes.byref(experts), ptr(residual),
                          ptr(out), ptr(topk_ids), ptr(topk_w),
                          None if perm is None else ctypes.byref(perm), ptr(workspace),
                          workspace_bytes, stream_handle(stream))
    return _ret(st, "moe_layer", check)


def moe_layer_noalloc(shape, x, w_router, router_bias, experts, residual, out, topk_ids, topk_w,
                      perm, stream=None, check=True) -> int:
    st = load().moe_layer_noalloc(ctypes.byref(shape), ptr(x), ptr(w_router), ptr(router_bias),
                                  None if experts is None else ctypes.byref(experts), ptr(residual),
                                  ptr(out), ptr(topk_ids), ptr(topk_w),
                                  None if perm is None else ctypes.byref(perm), stream_handle(stream))
    return _ret(st, "moe_layer_noalloc", check)


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_stream_read(buf, nbytes, sink, stream=None, check=True) -> int:
    """Read-bandwidth probe: stream nbytes of buf once (measurement helper)."""
    st = load().moe_stream_read(ptr(buf), nbytes, ptr(sink), stream_handle(stream))
    return _ret(st, "moe_stream_read", check)


def moe_route_locality_blocks(T: int) -> int:
    return int(load().moe_route_locality_blocks(T))


def moe_route_locality(shape, topk_ids, overlap_prev, block_unique, stream=None, check=True) -> int:
    st = load().moe_route_locality(ctypes.byref(shape), ptr(topk_ids), ptr(overlap_prev),
                                   ptr(block_unique), stream_handle(stream))
    return _ret(st, "moe_route_locality", check)


def moe_stage_experts(shape, src, dst, perm, parts=None, stream=None, check=True) -> int:
    parts = MOE_STAGE_GATE_UP | MOE_STAGE_DOWN if parts is None else parts
    st = load().moe_stage_experts(ctypes.byref(shape), None if src is None else ctypes.byref(src),
                                  None if dst is None else ctypes.byref(dst),
                                  None if perm is None else ctypes.byref(perm), parts,
                                  stream_handle(stream))
    return _ret(st, "moe_stage_experts", check)
