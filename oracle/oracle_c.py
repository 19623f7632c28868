"""ctypes binding of the C++ oracle ``moe_oracle_c.cpp`` (TEST INFRASTRUCTURE
ONLY: loaded by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
legs of ``bench.py``; nothing in the product path).

The C++ oracle is a second, independently written plain CPU implementation
of the routed layer in float64; ``tests/test_oracle_c.py`` checks it against
the pinned numpy oracle (``moe_oracle.py``) and the GPU tests compare the HIP
path with both.  ``build()`` compiles it with g++ into ``oracle/_build``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle_c.cpp")
LIB = os.path.join(HERE, "_build", "liboracle_c.so")
WFMT = {"dense": 0, "int4_g32": 1, "int2_g32": 2}
ACT = {"f32": 0, "bf16": 1}

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C++ oracle (always recompiles)."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def load_from(path: str):
    """A library built from this source (or a copy of it) at `path`, with
    its argument types declared."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.oc_router_logits.argtypes = [i, i, i, P, P, P, i, P]
    lib.oc_select_topk.argtypes = [i, i, i, P, i, P]
    lib.oc_select_topk.restype = i
    lib.oc_route_weights.argtypes = [i, i, i, P, P, P]
    lib.oc_permutation.argtypes = [i, i, P, P, P, P, P, P]
    lib.oc_permutation.restype = i
    lib.oc_grouped_ffn.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P, P, i, i, P]
    lib.oc_combine.argtypes = [i, i, i, P, P, P, P, P]
    lib.oc_decode_act.argtypes = [i, ctypes.c_int64, P, P]
    lib.oc_round_bf16.argtypes = [ctypes.c_int64, P, P]
    return lib


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = load_from(LIB)
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class PermC:
    counts: np.ndarray
    offsets: np.ndarray
    sorted_pair: np.ndarray
    pair_row: np.ndarray
    active: np.ndarray
    n_active: int


@dataclass
class LayerC:
    logits: np.ndarray
    ids: np.ndarray
    w: np.ndarray
    perm: PermC
    Y: np.ndarray
    out: np.ndarray


def storage_arrays(experts: dict) -> dict:
    """Contiguous numpy storage arrays (bf16 / fp16 as uint16 bit patterns,
    packed codes as uint8) from the input generator's expert tensors."""
    import torch
    out = {}
    for n, t in experts.items():
        if t is None:
            out[n] = None
            continue
        t = t.detach().cpu().contiguous()
        if t.dtype in (torch.bfloat16, torch.float16):
            out[n] = t.view(torch.int16).numpy().view(np.uint16)
        else:
            out[n] = t.numpy()
    return out


def decode_act_c(storage: np.ndarray, act: str) -> np.ndarray:
    """Activation storage (float32 values, or bf16 bit patterns as uint16)
    decoded to float64 by the C++ oracle's own decoder."""
    src = np.ascontiguousarray(storage, dtype=np.float32 if act == "f32" else np.uint16)
    out = np.empty(src.shape, dtype=np.float64)
    load().oc_decode_act(ACT[act], src.size, _p(src), _p(out))
    return out


def round_bf16_c(v64: np.ndarray) -> np.ndarray:
    """float64 values rounded once to bf16 by the C++ oracle: bit patterns (uint16)."""
    src = np.ascontiguousarray(v64, dtype=np.float64)
    out = np.empty(src.shape, dtype=np.uint16)
    load().oc_round_bf16(src.size, _p(src), _p(out))
    return out


def routes_c(x64: np.ndarray, wr64: np.ndarray, bias64: Optional[np.ndarray], k: int,
             threads: Optional[int] = None):
    """Router logits, top-k ids, weights and the permutation through the C++
    oracle (no expert FFN): (logits, ids, w, PermC)."""
    lib = load()
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    wr64 = np.ascontiguousarray(wr64, dtype=np.float64)
    b64 = None if bias64 is None else np.ascontiguousarray(bias64, dtype=np.float64)
    T, H = x64.shape
    E = wr64.shape[0]
    th = threads or min(16, os.cpu_count() or 1)
    logits = np.empty((T, E))
    lib.oc_router_logits(T, H, E, _p(x64), _p(wr64), _p(b64), th, _p(logits))
    ids = np.empty((T, k), dtype=np.int32)
    if lib.oc_select_topk(T, E, k, _p(logits), th, _p(ids)) != 0:
        raise ValueError("non-finite router logits")
    w = np.empty((T, k))
    lib.oc_route_weights(T, E, k, _p(logits), _p(ids), _p(w))
    P = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(P, dtype=np.int32)
    pr = np.empty(P, dtype=np.int32)
    active = np.empty(E, dtype=np.int32)
    n_act = lib.oc_permutation(P, E, _p(ids), _p(counts), _p(offsets), _p(sp), _p(pr),
                               _p(active))
    if n_act < 0:
        raise ValueError("expert id outside [0, E)")
    perm = PermC(counts.astype(np.int64), offsets.astype(np.int64), sp.astype(np.int64),
                 pr.astype(np.int64), active[:n_act].astype(np.int64), int(n_act))
    return logits, ids.astype(np.int64), w, perm


def moe_layer_c(x64: np.ndarray, wr64: np.ndarray, bias64: Optional[np.ndarray], experts: dict,
                wfmt: str, act: str, k: int, residual64: Optional[np.ndarray] = None,
                threads: Optional[int] = None, lib=None) -> LayerC:
    """The routed layer through the C++ oracle.  ``experts`` holds storage
    arrays (``storage_arrays``): gate/up [E][I][H...], down [E][H][I...].
    ``lib``: another build of the source (load_from), else the default."""
    lib = lib or load()
    x64 = np.ascontiguousarray(x64, dtype=np.float64)
    wr64 = np.ascontiguousarray(wr64, dtype=np.float64)
    b64 = None if bias64 is None else np.ascontiguousarray(bias64, dtype=np.float64)
    r64 = None if residual64 is None else np.ascontiguousarray(residual64, dtype=np.float64)
    T, H = x64.shape
    E = wr64.shape[0]
    I = experts["gate"].shape[1]
    th = threads or min(16, os.cpu_count() or 1)
    logits = np.empty((T, E))
    lib.oc_router_logits(T, H, E, _p(x64), _p(wr64), _p(b64), th, _p(logits))
    ids = np.empty((T, k), dtype=np.int32)
    if lib.oc_select_topk(T, E, k, _p(logits), th, _p(ids)) != 0:
        raise ValueError("non-finite router logits")
    w = np.empty((T, k))
    lib.oc_route_weights(T, E, k, _p(logits), _p(ids), _p(w))
    P = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(P, dtype=np.int32)
    pr = np.empty(P, dtype=np.int32)
    active = np.empty(E, dtype=np.int32)
    n_act = lib.oc_permutation(P, E, _p(ids), _p(counts), _p(offsets), _p(sp), _p(pr),
                               _p(active))
    if n_act < 0:
        raise ValueError("expert id outside [0, E)")
    g, u, d = (np.ascontiguousarray(experts[n]) for n in ("gate", "up", "down"))
    gs, us, ds = (None if experts[n] is None else np.ascontiguousarray(experts[n])
                  for n in ("gate_scale", "up_scale", "down_scale"))
    Y = np.empty((P, H))
    lib.oc_grouped_ffn(T, H, E, I, k, WFMT[wfmt], ACT[act], _p(x64), _p(g), _p(u), _p(d),
                       _p(gs), _p(us), _p(ds), _p(offsets), _p(sp), _p(active), n_act, th,
                       _p(Y))
    out = np.empty((T, H))
    lib.oc_combine(T, H, k, _p(Y), _p(pr), _p(w), _p(r64), _p(out))
    return LayerC(logits, ids.astype(np.int64), w,
                  PermC(counts.astype(np.int64), offsets.astype(np.int64), sp.astype(np.int64),
                        pr.astype(np.int64), active[:n_act].astype(np.int64), int(n_act)),
                  Y, out)
