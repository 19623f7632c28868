"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/moe.h declares, and rejects invalid calls before
enqueuing anything.  Rejected calls are given host sentinel buffers as their
outputs; the library must not touch them (it never dereferences device
pointers on the host, and a rejected call launches nothing)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import sparse_moe_routed_amd as M
from sparse_moe_routed_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_abi.LIB_PATH),
                                reason="libmoe.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", text, flags=re.M)))


def test_exports_match_header():
    decl = declared_functions()
    assert set(decl) == set(_abi.EXPORTS), decl
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in decl:
        assert name in syms, name
    lib = M.load()
    for name in decl:
        assert hasattr(lib, name)


def test_status_strings():
    for code, name in _abi.STATUS.items():
        assert M.moe_status_str(code).startswith(name)
    assert M.moe_status_str(999) == "unknown moe status"


GOOD = dict(T=8, H=2560, E=512, I=640, top_k=10, act="bf16", wfmt="dense")


def shape(**kw):
    d = dict(GOOD)
    d.update(kw)
    return M.make_shape(**d)


def test_workspace_size():
    s = shape()
    ws = M.moe_workspace_size(s)
    P = 8 * 10
    assert ws >= P * 2560 * 2 + P * 640 * 2          # y and h regions at least
    assert M.moe_workspace_size(shape(T=0)) == 0
    assert M.moe_workspace_size(shape(H=100)) == 0
    big = M.moe_workspace_size(shape(T=4096))
    assert big > ws


class HostBuf:
    """A host numpy buffer standing in for a device pointer with a sentinel."""

    def __init__(self, nbytes, fill=0xA5, offset=0):
        self.a = np.full(nbytes + 64, fill, dtype=np.uint8)
        base = self.a.ctypes.data
        self.addr = (base + 15) // 16 * 16 + offset

    def untouched(self, fill=0xA5):
        return bool((self.a == fill).all())


def bufs():
    return {n: HostBuf(1 << 16) for n in ("x", "wr", "ids", "w", "logits", "ws", "out", "res",
                                          "y", "g", "u", "d", "gs", "us", "ds")}


def _route(s, b, **over):
    args = dict(x=b["x"].addr, w_router=b["wr"].addr, router_bias=None, topk_ids=b["ids"].addr,
                topk_w=b["w"].addr, logits=b["logits"].addr, workspace=b["ws"].addr,
                workspace_bytes=1 << 40)
    args.update(over)
    return M.moe_route(s, stream=0, check=False, **args)


@pytest.mark.parametrize("field,value,code", [
    ("H", 100, 2), ("H", 0, 2), ("I", 48, 2), ("E", 2000, 2), ("top_k", 0, 2),
    ("top_k", 600, 2), ("T", -1, 2), ("T", 131073, 2), ("act", 7, 3), ("wfmt", 9, 4),
    ("flags", 4, 10), ("flags", 0x80000000, 10),
])
def test_route_rejects_bad_shape(field, value, code):
    b = bufs()
    assert _route(shape(**{field: value}), b) == code
    for v in b.values():
        assert v.untouched()


def test_f32_lowbit_combination_rejected():
    b = bufs()
    assert _route(shape(act="f32", wfmt="int4_g32"), b) == 4


def test_null_shape_and_pointers():
    b = bufs()
    lib = M.load()
    assert lib.moe_route(None, None, None, None, None, None, None, None, 0, None) == 1
    assert _route(shape(), b, x=None) == 1
    assert _route(shape(), b, topk_w=None) == 1
    assert all(v.untouched() for v in b.values())


def test_misaligned_rejected():
    b = bufs()
    assert _route(shape(), b, x=b["x"].addr + 2) == 5
    assert _route(shape(), b, logits=b["logits"].addr + 4) == 5
    assert all(v.untouched() for v in b.values())


def test_workspace_too_small():
    b = bufs()
    need = M.moe_workspace_size(shape())
    assert _route(shape(), b, workspace_bytes=need - 1) == 7
    assert _route(shape(), b, workspace=None) == 7
    assert all(v.untouched() for v in b.values())


def test_alias_rejected():
    b = bufs()
    assert _route(shape(), b, topk_w=b["ids"].addr + 16) == 6          # ids and w overlap
    assert _route(shape(), b, logits=b["x"].addr) == 6                   # output over input
    s = shape()
    st = M.moe_combine(s, b["y"].addr, b["ids"].addr, b["w"].addr, b["res"].addr,
                       b["res"].addr + 32, stream=0, check=False)
    assert st == 6
    assert all(v.untouched() for v in b.values())


def test_t_zero_is_noop():
    s = shape(T=0)
    assert M.moe_route(s, None, None, None, None, None, None, None, 0, stream=0, check=False) == 0
    assert M.moe_layer(s, None, None, None, None, None, None, None, None, None, None, 0,
                       stream=0, check=False) == 0


def test_expert_format_checks():
    b = bufs()
    dense = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr, b["gs"].addr, None, None)
    s = shape()
    perm = M.make_perm(*(HostBuf(1 << 12).addr for _ in range(6)))
    st = M.moe_grouped_ffn(s, b["x"].addr, dense, perm, b["y"].addr, b["ws"].addr, 1 << 40,
                           stream=0, check=False)
    assert st == 4                                      # scales given for dense weights
    q = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr, None, None, None)
    st = M.moe_grouped_ffn(shape(wfmt="int4_g32"), b["x"].addr, q, perm, b["y"].addr,
                           b["ws"].addr, 1 << 40, stream=0, check=False)
    assert st == 1                                      # low-bit without scales
    assert all(v.untouched() for v in b.values())


def test_layer_rejects_out_over_x():
    b = bufs()
    ex = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr)
    st = M.moe_layer(shape(), b["x"].addr, b["wr"].addr, None, ex, None, b["x"].addr + 64,
                     b["ids"].addr, b["w"].addr, None, b["ws"].addr, 1 << 40, stream=0,
                     check=False)
    assert st == 6
    assert all(v.untouched() for v in b.values())


def test_tiled_flag_domain():
    b = bufs()
    assert _route(shape(flags=1, act="f32", wfmt="dense", H=256, I=128), b) == 4   # tiled needs bf16
    assert _route(shape(flags=1, I=96), b) == 2                                      # tiled needs I % 128
    assert all(v.untouched() for v in b.values())


def test_tile_experts_validation():
    b = bufs()
    src = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr)
    dst = M.make_experts(b["gs"].addr, b["us"].addr, b["ds"].addr)
    assert M.moe_tile_experts(shape(flags=1), src, dst, stream=0, check=False) == 10   # source is row-major
    assert M.moe_tile_experts(shape(), src, src, stream=0, check=False) == 6           # in place
    assert M.moe_tile_experts(shape(I=96), src, dst, stream=0, check=False) == 2
    assert M.moe_tile_experts(shape(), src, None, stream=0, check=False) == 1
    assert all(v.untouched() for v in b.values())


def test_check_finite_flag_workspace():
    """MOE_F_CHECK_FINITE is a known flag; its private result buffers make
    the workspace larger."""
    plain = M.moe_workspace_size(shape())
    checked = M.moe_workspace_size(shape(flags=M.MOE_F_CHECK_FINITE))
    P = 8 * 10
    assert checked >= plain + 2 * P * 4 + 8 * 2560 * 2 + 4
    b = bufs()
    st = _route(shape(flags=M.MOE_F_CHECK_FINITE), b, workspace_bytes=checked - 1)
    assert st == 7
    assert all(v.untouched() for v in b.values())


def test_stream_read_validation():
    b = HostBuf(1 << 12)
    sink = HostBuf(64)
    assert M.moe_stream_read(None, 16, sink.addr, stream=0, check=False) == 1
    assert M.moe_stream_read(b.addr, 0, sink.addr, stream=0, check=False) == 2
    assert M.moe_stream_read(b.addr, 24, sink.addr, stream=0, check=False) == 2
    assert M.moe_stream_read(b.addr + 8, 16, sink.addr, stream=0, check=False) == 5
    assert M.moe_stream_read(b.addr, 1024, b.addr + 512, stream=0, check=False) == 6
    assert b.untouched() and sink.untouched()


def test_route_locality_blocks_and_validation():
    assert M.moe_route_locality_blocks(13) == 13 + 7 + 5 + 4 + 3
    assert M.moe_route_locality_blocks(1) == 5
    assert M.moe_route_locality_blocks(0) == 0
    b = bufs()
    s = shape()
    assert M.moe_route_locality(s, None, b["ids"].addr, b["w"].addr, stream=0, check=False) == 1
    assert M.moe_route_locality(s, b["ids"].addr, b["ids"].addr, b["w"].addr, stream=0,
                                check=False) == 6
    assert M.moe_route_locality(shape(T=0), None, None, None, stream=0, check=False) == 0
    assert all(v.untouched() for v in b.values())


def test_stage_experts_validation():
    b = bufs()
    src = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr)
    dst = M.make_experts(b["gs"].addr, b["us"].addr, b["ds"].addr)
    pm = M.make_perm(*(b[n].addr for n in ("ids", "w", "logits", "res", "y", "x")))
    s = shape(E=4, top_k=2, H=128, I=32)       # records fit the 64 KiB buffers
    assert M.moe_stage_experts(s, None, dst, pm, stream=0, check=False) == 1
    assert M.moe_stage_experts(s, src, dst, None, stream=0, check=False) == 1
    assert M.moe_stage_experts(s, src, src, pm, stream=0, check=False) == 6            # in place
    assert M.moe_stage_experts(shape(flags=4), src, dst, pm, stream=0, check=False) == 10
    assert M.moe_stage_experts(s, src, dst, pm, parts=0, stream=0, check=False) == 10
    assert M.moe_stage_experts(s, src, dst, pm, parts=4, stream=0, check=False) == 10
    odd = M.make_experts(b["g"].addr + 8, b["u"].addr, b["d"].addr)
    assert M.moe_stage_experts(s, odd, dst, pm, stream=0, check=False) == 5
    # pageable host memory is not device-readable: rejected before any launch
    assert M.moe_stage_experts(s, src, dst, pm, stream=0, check=False) == 12
    assert all(v.untouched() for v in b.values())


def test_fused_flag_domain_and_workspace():
    assert M.moe_workspace_size(shape(flags=4)) == 0                # needs the tiled layout
    base = M.moe_workspace_size(shape(flags=1))
    fused = M.moe_workspace_size(shape(flags=5))
    P = 8 * 10
    assert fused - base >= (640 // 64) * P * 2560 * 4              # float32 partials per slice
    assert M.moe_workspace_size(shape(flags=5, T=1638)) > 0         # T*k = 16380
    assert M.moe_workspace_size(shape(flags=5, T=1639)) == 0        # beyond the partial buffer limit
    assert M.moe_ffn_fused_items(shape(flags=1)) == 0
    assert M.moe_ffn_fused_items(shape(flags=5)) == (P // 16 + P) * (640 // 64)


def test_ffn_fused_validation():
    b = bufs()
    s = shape(E=4, top_k=2, H=128, I=128, T=8, flags=5)
    ex = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr)
    pm = M.make_perm(*(b[n].addr for n in ("ids", "w", "logits", "res", "y", "x")))
    args = dict(x=b["x"].addr, experts=ex, perm=pm, y=b["out"].addr, wave_tiles=0, item_clock=None,
                workspace=b["ws"].addr, workspace_bytes=1 << 40, stream=0, check=False)

    def call(sh=s, **over):
        a = dict(args)
        a.update(over)
        return M.moe_ffn_fused(sh, **a)

    assert call(sh=shape(E=4, top_k=2, H=128, I=128, T=8, flags=1)) == 10   # flag missing
    assert call(wave_tiles=-1) == 2
    assert call(x=None) == 1
    assert call(item_clock=b["gs"].addr + 8) == 5
    assert call(item_clock=b["out"].addr) == 6                               # clock over y
    assert call(workspace_bytes=16) == 7
    assert all(v.untouched() for v in b.values())


def test_layer_noalloc_validation():
    """moe_layer_noalloc validates like moe_layer and refuses a shape whose
    workspace exceeds its fixed device array, all before any HIP call."""
    b = bufs()
    ex = M.make_experts(b["g"].addr, b["u"].addr, b["d"].addr)

    def call(sh, **over):
        a = dict(x=b["x"].addr, w_router=b["wr"].addr, router_bias=None, experts=ex, residual=None,
                 out=b["out"].addr, topk_ids=b["ids"].addr, topk_w=b["w"].addr, perm=None)
        a.update(over)
        return M.moe_layer_noalloc(sh, stream=0, check=False, **a)

    big = shape(T=4096)
    assert M.moe_workspace_size(big) > M.MOE_NOALLOC_SCRATCH_BYTES
    assert call(big) == 7                                    # MOE_E_WORKSPACE
    assert call(shape(T=0)) == 0                             # no-op
    assert call(shape(H=100)) == 2
    assert call(shape(), x=None) == 1
    assert call(shape(), out=b["out"].addr + 8) == 5
    assert all(v.untouched() for v in b.values())
    lib = M.load()
    assert lib.moe_layer_noalloc(None, None, None, None, None, None, None, None, None, None,
                                 None) == 1
