#!/usr/bin/env python3
"""Routed-MoE layer throughput on one MI355X.

A step is one pass of the whole routed layer (router -> top-k -> permutation
-> grouped gate/up + SwiGLU -> grouped down -> rank-order combine; for the
stacked workloads all 48 layers, x_{l+1} = x_l + moe_l(x_l)) over one batch of
synthetic tokens already resident in HBM.  Steps cycle over --batches
distinct token batches, so the set of active experts changes from step to step
as it does between decode batches.

Prints one JSON line: tokens/s of the workload, the roofline of the dominant
kernel (the grouped gate/up + SwiGLU kernel, timed with HIP events around
each of its launches on the stream it runs on), the CPU oracles timed on
bounded samples of the same workload (`cpu_baseline`: the plain C++ float64
oracle; `cpu_baseline_numpy`: the numpy float64 oracle) and the GPU routes of
layer 0 checked against the C++ oracle (`oracle_route_check`: mismatches,
near ties, largest logit difference).  With no --workload the headline line
is the decode workload and the other four workloads follow under
`workloads`, each measured the same way in the same process.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

WORKLOADS = {"tiny": 1, "decode": 2, "prefill": 3, "stack_int4": 4, "verify_int2": 5,
             # eight 4096-token prefill windows merged into one call: T*k/U passes the
             # bf16 ridge, so the grouped GEMMs leave the HBM-bound regime
             "prefill_merged": 3}
WORKLOAD_TOKENS = {"prefill_merged": 32768}
WBYTES = {"dense": None, "int4_g32": 0.5, "int2_g32": 0.25}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for one layer, 10 for 48-layer stacks)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=None, choices=list(WORKLOADS),
                    help="one workload only (default: decode as the headline line, the other "
                         "workloads measured after it under `workloads`)")
    ap.add_argument("--only-headline", action="store_true",
                    help="with no --workload: measure decode only")
    ap.add_argument("--batches", type=int, default=16, help="distinct token batches cycled")
    ap.add_argument("--layers", type=int, default=None, help="override the stack depth")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override T (e.g. several prefill windows merged into one call)")
    ap.add_argument("--layout", default="tiled", choices=["tiled", "row"],
                    help="expert weight layout (tiled: converted once at load time)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle sample budget of the headline workload (per oracle)")
    ap.add_argument("--cpu-seconds-other", type=float, default=6.0,
                    help="C++ oracle sample budget of each other workload in the default run")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="read this many MiB of scratch between timed steps (evicts L2/MALL with "
                         "clean lines); each step is then timed on its own and value = tokens / sum "
                         "of step times")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay measurement (extra field `graph`)")
    ap.add_argument("--probe-mib", type=int, default=4096,
                    help="buffer size of the read-bandwidth probe (0: skip)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the host-resident expert measurement (extra field `offload`)")
    ap.add_argument("--offload-steps", type=int, default=20)
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused gate/up -> down measurement (extra field `fused_waves`)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (PMC calibration)")
    return ap.parse_args()


class TimingEvent:
    """A HIP event used only for timing: created with hipEventDisableSystemFence,
    so recording it does not write back and invalidate the caches (a default
    timing event costs the step about 3 us of GPU time per record on the
    MI355X).  Recorded on torch's current stream unless a stream is given."""

    FLAGS = 0x20000000          # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def hip(cls):
        if cls._hip is None:
            import ctypes
            h = ctypes.CDLL("libamdhip64.so")
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None):
        import torch
        st = (stream or torch.cuda.current_stream()).cuda_stream
        if self.hip().hipEventRecord(self.ev, st) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def weight_bytes_per_param(cfg):
    if cfg.wfmt == "dense":
        return 4.0 if cfg.act == "f32" else 2.0
    return WBYTES[cfg.wfmt] + 2.0 / 32            # codes + one fp16 scale per 32


def gateup_traffic(cfg, U):
    """Algorithmic bytes and flops of one grouped gate/up launch: the gate and
    up weights of the U active experts read once and the T token rows read.
    The P x I SwiGLU intermediate it writes is scratch of the implementation
    (the next kernel reads it back) and is not counted."""
    act = 4 if cfg.act == "f32" else 2
    P = cfg.T * cfg.k
    w = U * 2 * cfg.I * cfg.H * weight_bytes_per_param(cfg)
    b = w + cfg.T * cfg.H * act
    f = 2.0 * P * 2 * cfg.I * cfg.H
    return b, f


# tokens of layer 0 (over the cycled batches) whose GPU routes the CPU leg
# checks against the C++ oracle
ROUTE_CHECK_MAX_TOKENS = 16384


def layer_bytes(cfg, U):
    """Algorithmic bytes of one layer: active expert records once, the router
    weight, x in and out."""
    act = 4 if cfg.act == "f32" else 2
    rec = 3 * cfg.I * cfg.H * weight_bytes_per_param(cfg)
    return U * rec + cfg.E * cfg.H * act + 2 * cfg.T * cfg.H * act


# the files that define the grouped FFN kernels and how they are compiled
DIGEST_FILES = ("sparse_moe_routed_amd/csrc/k_ffn.hip", "sparse_moe_routed_amd/csrc/ffn_tiled.h",
                "sparse_moe_routed_amd/csrc/moe_device.h",
                "sparse_moe_routed_amd/csrc/moe_internal.h", "sparse_moe_routed_amd/build.py")


def _code_only(name, text):
    """Source text without comments and with whitespace collapsed, so that
    the digest changes with the code, not with its comments."""
    if name.endswith(".py"):
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_source_digest():
    """Digest of the FFN kernel sources (code only): the committed PMC
    summaries count for the dominant kernel only while it matches."""
    h = hashlib.sha256()
    for f in DIGEST_FILES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode() + _code_only(f, fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, digest):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 PMC summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_moe_routed_amd as M

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return

    M.load()
    headline = args.workload or "decode"
    line = run_workload(args, M, torch, dev, headline, headline=True)
    if args.workload is None and not args.only_headline:
        # the default run also measures the other workloads, each with its own
        # weights, in this process after the headline one (its memory freed)
        line["workloads"] = {}
        for wl in OTHER_WORKLOADS:
            line["workloads"][wl] = summarize(run_workload(args, M, torch, dev, wl, headline=False))
        line["workloads_note"] = (
            "each workload as its own run of the same steps/warmup in this process: tokens/s, "
            "step time, whole-layer HBM fraction, the dominant kernel's roofline, HIP-graph "
            "replay, the C++ float64 oracle timed on the host cores and the oracle route check")
    print(json.dumps(line))


OTHER_WORKLOADS = ("tiny", "prefill", "stack_int4", "verify_int2")


def summarize(r):
    """The fields of one workload's line kept under `workloads` in the default run."""
    keep = ("value", "unit", "steps", "warmup", "ms_per_step", "dtype", "config", "timing",
            "layer_hbm", "graph", "cpu_baseline", "oracle_route_check")
    out = {k: r[k] for k in keep if k in r}
    rf = r["roofline"]
    out["roofline"] = {k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                          "kernel", "avg_launch_us", "hbm_frac", "mfma_frac",
                                          "attainable_frac")}
    return out


def run_workload(args, M, torch, dev, name, headline):
    """One workload end to end: inputs resident in HBM, untimed routing
    statistics, warmup, the timed steps, the dominant-kernel roofline, graph
    replay, and the CPU-oracle leg.  Returns the JSON line as a dict."""
    from moe_inputs import CONFIGS, make_experts, make_router, make_x

    cfg = CONFIGS[WORKLOADS[name]]
    if name in WORKLOAD_TOKENS:
        cfg = cfg.with_(name=name, T=WORKLOAD_TOKENS[name])
    if args.tokens is not None and headline:
        cfg = cfg.with_(T=args.tokens)
    L = cfg.layers if (args.layers is None or not headline) else args.layers
    steps = args.steps if args.steps is not None else (200 if L == 1 else 10)
    warmup = args.warmup if args.warmup is not None else (20 if L == 1 else 3)
    T, k = cfg.T, cfg.k

    # ---- inputs resident in HBM --------------------------------------------
    tiled = args.layout == "tiled" and cfg.act == "bf16" and cfg.I % 128 == 0
    row_shape = M.make_shape(T, cfg.H, cfg.E, cfg.I, k, cfg.act, cfg.wfmt)

    def mk(ex):
        return M.make_experts(ex["gate"], ex["up"], ex["down"], ex["gate_scale"], ex["up_scale"],
                              ex["down_scale"])

    layers = []
    for l in range(L):
        wr, bias = make_router(cfg, l, dev)
        ex = make_experts(cfg, l, dev)
        if tiled:   # one-time layout conversion at load time; the row-major copy is dropped
            tex = {n: (None if t is None else torch.empty_like(t)) for n, t in ex.items()}
            M.moe_tile_experts(row_shape, mk(ex), mk(tex))
            torch.cuda.synchronize()
            ex = tex
        layers.append((wr, bias, ex, mk(ex)))
    xs = [make_x(cfg, dev, batch=b) for b in range(args.batches)]
    buf = M.MoELayerBuffers(T, cfg.H, cfg.E, cfg.I, k, cfg.act, cfg.wfmt, device=dev, tiled=tiled)
    acts = [torch.empty_like(xs[0]) for _ in range(2)]
    torch.cuda.synchronize()

    ev_a = [TimingEvent() for _ in range(steps * L)]
    ev_b = [TimingEvent() for _ in range(steps * L)]

    # one layer = moe_route_permute -> moe_ffn_gate_up -> moe_ffn_down_combine
    # (the same kernels as moe_layer; the gate/up call is separate so that the
    # dominant kernel can be timed on its own)
    def step(i, timed_idx=None):
        x = xs[i % len(xs)]
        for l, (wr, bias, _, exg) in enumerate(layers):
            out = acts[l % 2] if L > 1 else buf.out
            buf.route_permute(x, wr, bias, logits=False)
            if timed_idx is not None:
                ev_a[timed_idx * L + l].record()
            buf.ffn_gate_up(x, exg)
            if timed_idx is not None:
                ev_b[timed_idx * L + l].record()
            buf.ffn_down_combine(exg, residual=x if cfg.residual else None, out=out)
            x = out

    # ---- routing statistics per (batch, layer), untimed ---------------------
    # (layer 0 also keeps the GPU routes and float32 logits of every batch for
    # the oracle route check of the CPU leg; its inputs come from the generator)
    U = np.zeros((len(xs), L), dtype=np.int64)
    loc = {"overlap": [], "blocks": {B: [] for B in range(1, 6)}, "skew": []}
    gpu_routes = []
    check_tokens = 0
    for b in range(len(xs)):
        x = xs[b]
        for l, (wr, bias, _, exg) in enumerate(layers):
            out = acts[l % 2] if L > 1 else buf.out
            keep = l == 0 and check_tokens + T <= ROUTE_CHECK_MAX_TOKENS
            buf.route_permute(x, wr, bias, logits=keep)
            if keep:
                gpu_routes.append((b, buf.topk_ids.cpu().numpy(), buf.logits.cpu().numpy()))
                check_tokens += T
            U[b, l] = int(buf.n_active.item())
            ov, blocks = buf.route_locality()
            loc["overlap"].append(ov[1:].float().mean().item() if T > 1 else 0.0)
            for B in range(1, 6):
                full = blocks[B - 1][: T // B]          # full blocks only
                if full.numel():
                    loc["blocks"][B].append(full.float().mean().item())
            loc["skew"].append(int(buf.counts.max().item()) / (T * k / cfg.E))
            buf.ffn_gate_up(x, exg)
            buf.ffn_down_combine(exg, residual=x if cfg.residual else None, out=out)
            x = out
    torch.cuda.synchronize()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Back to back: one event before the first and after the last step, and the
    # per-step times between the gate/up start events of consecutive steps (a
    # timing event costs about 1 us of GPU time even without the system fence,
    # so the steps carry only the two around the dominant kernel).  Flushing:
    # one event before and one after each step, so that the flush between
    # steps is outside the step times.
    flush = args.flush_mib if headline else 0
    ev_beg = [TimingEvent() for _ in range(steps + 1 if flush else 2)]
    ev_end = [TimingEvent() for _ in range(steps)] if flush else None
    scratch = sink = None
    if flush:
        scratch = torch.zeros(flush << 20, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        M.moe_stream_read(scratch, scratch.numel(), sink)
        torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if scratch is None:
        ev_beg[0].record()
    for i in range(steps):
        if scratch is not None:
            ev_beg[i].record()
        step(i, timed_idx=i)
        if scratch is not None:
            ev_end[i].record()
            M.moe_stream_read(scratch, scratch.numel(), sink)
    ev_beg[-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if scratch is None:
        elapsed_ms = ev_beg[0].elapsed_time(ev_beg[-1])
        step_ms = np.array([ev_a[i * L].elapsed_time(ev_a[(i + 1) * L]) for i in range(steps - 1)]
                           if steps > 1 else [elapsed_ms])
    else:
        step_ms = np.array([ev_beg[i].elapsed_time(ev_end[i]) for i in range(steps)])
        elapsed_ms = float(step_ms.sum())
    ms_per_step = elapsed_ms / steps
    tokens_per_s = T * steps / (elapsed_ms / 1e3)
    del scratch, sink

    # ---- dominant kernel roofline --------------------------------------------
    gu_ms = np.array([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)])
    gu_bytes = np.zeros(steps * L)
    gu_flops = np.zeros(steps * L)
    for i in range(steps):
        for l in range(L):
            gu_bytes[i * L + l], gu_flops[i * L + l] = gateup_traffic(cfg, U[i % len(xs), l])
    avg_ms = float(gu_ms.mean())
    avg_bytes = float(gu_bytes.mean())
    avg_flops = float(gu_flops.mean())
    intensity = avg_flops / avg_bytes
    if cfg.act == "f32":
        bound, peak, unit = "alu", FP32_PEAK_TFLOPS, "TFLOP/s"
        achieved = avg_flops / (avg_ms / 1e3) / 1e12
    elif intensity > RIDGE:
        bound, peak, unit = "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"
        achieved = avg_flops / (avg_ms / 1e3) / 1e12
    else:
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        achieved = avg_bytes / (avg_ms / 1e3) / 1e9
    digest = kernel_source_digest()
    traffic = traffic_from_profiles(name, digest)

    step_bytes = np.mean([sum(layer_bytes(cfg, U[b, l]) for l in range(L)) for b in range(len(xs))])
    graph = None if args.no_graph else graph_replay(torch, buf, layers, xs, acts, cfg, L, steps)
    # route-locality kernel time (on the last routes)
    la, lb = TimingEvent(), TimingEvent()
    buf.route_locality()
    la.record()
    for _ in range(20):
        buf.route_locality()
    lb.record()
    torch.cuda.synchronize()
    ub = {B: (round(float(np.mean(v)), 3) if v else None) for B, v in loc["blocks"].items()}
    route_locality = {
        "over": f"{len(xs)} batches x {L} layers",
        "mean_overlap_with_previous_token": round(float(np.mean(loc["overlap"])), 3),
        "unique_experts_per_block": {str(B): v for B, v in ub.items()},
        "breakeven_tau": {str(B): (round(v / k, 3) if v is not None else None) for B, v in ub.items()},
        "mean_skew_max_over_mean_load": round(float(np.mean(loc["skew"])), 2),
        "kernel_us": round(la.elapsed_time(lb) / 20 * 1e3, 2),
    }
    probe = read_probe(M, dev, args.probe_mib) if (args.probe_mib and headline) else None
    off = None if (args.no_offload or not headline) else offload(M, torch, dev, cfg, layers, xs, buf,
                                                                 args.offload_steps)
    fw = (None if (args.no_fused or not tiled or T * k > 16384 or not headline)
          else fused_waves(M, torch, dev, cfg, layers, xs))

    # ---- CPU leg: the oracles on bounded samples, and the route check --------
    cpu = cpu_np = check = None
    del buf, acts
    if not args.no_cpu_baseline:
        budget = args.cpu_seconds if headline else args.cpu_seconds_other
        check = oracle_route_check(cfg, layers, xs, gpu_routes)
        cpu = cpu_baseline_cxx(cfg, L, layers, xs, budget, dev)
        if headline:
            cpu_np = cpu_baseline(cfg, L, layers, xs, budget, dev)
    n_batches = len(xs)
    del layers, xs
    torch.cuda.empty_cache()

    return {
        "metric": "routed-MoE layer tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "E": cfg.E, "I": cfg.I, "top_k": k,
                   "layers": L, "weights": cfg.wfmt if cfg.wfmt != "dense" else cfg.act,
                   "weight_layout": "tiled" if tiled else "row-major",
                   "batches_cycled": n_batches, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "k_gateup (grouped gate/up + SwiGLU)",
                     "avg_launch_us": round(avg_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": round(avg_bytes),
                     "flops_per_launch": round(avg_flops), "kernel_source_digest": digest,
                     "measured_read_GBps": probe,
                     "frac_of_measured": (round(achieved / probe, 4)
                                          if probe and bound == "hbm" else None),
                     # both roofs for the same launches, and the attainable-roofline
                     # fraction max(F / F_peak, B / B_peak) / t
                     "hbm_frac": round(avg_bytes / (avg_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_frac": round(avg_flops / (avg_ms / 1e3) / 1e12 /
                                        (FP32_PEAK_TFLOPS if cfg.act == "f32" else BF16_PEAK_TFLOPS), 4),
                     "attainable_frac": round(
                         max(avg_flops / ((FP32_PEAK_TFLOPS if cfg.act == "f32" else BF16_PEAK_TFLOPS) * 1e12),
                             avg_bytes / (HBM_PEAK_GBS * 1e9)) / (avg_ms / 1e3), 4)},
        "timing": {"mode": ("steps back to back (per-step times between consecutive steps' "
                             "first gate/up start events)" if not flush else
                            f"{flush} MiB scratch read between steps, excluded"),
                   "step_ms_median": round(float(np.median(step_ms)), 5),
                   "step_ms_p10": round(float(np.percentile(step_ms, 10)), 5),
                   "step_ms_p90": round(float(np.percentile(step_ms, 90)), 5)},
        "layer_hbm": {"bytes_per_step": round(step_bytes),
                      "achieved_GBps": round(step_bytes / (ms_per_step / 1e3) / 1e9, 1),
                      "frac": round(step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                      "mean_unique_experts_per_layer": round(float(U.mean()), 2)},
        "route_locality": route_locality,
        "graph": graph,
        "offload": off,
        "fused_waves": fw,
        "cpu_baseline": cpu,
        "cpu_baseline_numpy": cpu_np,
        "oracle_route_check": check,
        "host_wall_s": round(wall, 3),
    }


def graph_replay(torch, buf, layers, xs, acts, cfg, L, steps):
    """The same steps captured once per token batch as HIP graphs (every
    call of every layer a kernel node) and replayed back to back; reported
    next to the eager timing, which stays the official value because the
    dominant kernel is timed with events around its launches."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graphs = []
        with torch.cuda.stream(s):
            for b in range(len(xs)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    x = xs[b]
                    for l, (wr, bias, _, exg) in enumerate(layers):
                        out = acts[l % 2] if L > 1 else buf.out
                        buf.route_permute(x, wr, bias, logits=False, stream=s)
                        buf.ffn_gate_up(x, exg, stream=s)
                        buf.ffn_down_combine(exg, residual=x if cfg.residual else None, out=out,
                                             stream=s)
                        x = out
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(3):
            graphs[i % len(graphs)].replay()
        a, b = TimingEvent(), TimingEvent()
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        del graphs
        return {"ms_per_step": round(ms, 5), "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
                "graphs": len(xs)}
    except Exception as e:   # capture is optional; the eager numbers stand
        return {"error": f"{type(e).__name__}: {e}"}


def offload(M, torch, dev, cfg, layers, xs, buf, steps):
    """Host-resident expert records: layer 0's records in pinned host memory,
    a device array of the same layout as the staging target.  One step is one
    layer: route -> permute -> stage the exact active union over PCIe (the GPU
    reads the pinned records itself; the active set never reaches the host)
    -> gate/up -> down -> combine.  `split`: gate/up records staged first and
    down on a second stream while gate/up computes; `serial`: one staging
    launch before the FFN.  `full_extent` copies every expert's records (the
    sequential layer-extent mode for prefill) with the staging kernel and
    with a plain host-to-device copy; the crossover is the unique-expert count
    at which the exact union costs as much as the full extent."""
    try:
        wr, bias, ex, _ = layers[0]
        names = ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")
        host = {n: (None if ex[n] is None else
                    torch.empty(ex[n].shape, dtype=ex[n].dtype, pin_memory=True)) for n in names}
        for n in names:
            if ex[n] is not None:
                host[n].copy_(ex[n])
        dst = {n: (None if ex[n] is None else torch.empty_like(ex[n])) for n in names}
        src_s = M.make_experts(*(host[n] for n in names))
        dst_s = M.make_experts(*(dst[n] for n in names))
        rec = sum(t.numel() * t.element_size() for t in ex.values() if t is not None) / cfg.E
        cur, side = torch.cuda.current_stream(), torch.cuda.Stream()
        res_of = (lambda x: x) if cfg.residual else (lambda x: None)

        def one(x, split):
            buf.route(x, wr, bias, logits=False)
            buf.permute()
            if split:
                buf.stage_experts(src_s, dst_s, parts=M.MOE_STAGE_GATE_UP)
                side.wait_stream(cur)
                buf.stage_experts(src_s, dst_s, parts=M.MOE_STAGE_DOWN, stream=side)
                buf.ffn_gate_up(x, dst_s)
                cur.wait_stream(side)
            else:
                buf.stage_experts(src_s, dst_s)
                buf.ffn_gate_up(x, dst_s)
            buf.ffn_down(dst_s)
            buf.combine(residual=res_of(x))

        def timed(split):
            for i in range(2):
                one(xs[i % len(xs)], split)
            torch.cuda.synchronize()
            a, b = TimingEvent(), TimingEvent()
            a.record()
            for i in range(steps):
                one(xs[i % len(xs)], split)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps

        U = []
        for i in range(min(steps, len(xs))):
            buf.route(xs[i], wr, bias, logits=False)
            buf.permute()
            U.append(int(buf.n_active.item()))
        u_mean = float(np.mean([U[i % len(U)] for i in range(steps)]))
        ms_split, ms_serial = timed(True), timed(False)
        staged = u_mean * rec

        # full layer extent: every expert active
        all_active = torch.arange(cfg.E, dtype=torch.int32, device=dev)
        n_all = torch.full((1,), cfg.E, dtype=torch.int32, device=dev)
        allp = M.make_perm(buf.counts, buf.offsets, buf.sorted_pair, buf.pair_row, all_active, n_all)
        a, b = TimingEvent(), TimingEvent()
        M.moe_stage_experts(buf.shape, src_s, dst_s, allp)
        torch.cuda.synchronize()
        a.record()
        M.moe_stage_experts(buf.shape, src_s, dst_s, allp)
        b.record()
        torch.cuda.synchronize()
        full_kernel = cfg.E * rec / (a.elapsed_time(b) / 1e3) / 1e9
        a.record()
        for n in names:
            if ex[n] is not None:
                dst[n].copy_(host[n], non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        full_copy = cfg.E * rec / (a.elapsed_time(b) / 1e3) / 1e9
        sel = staged / (ms_split / 1e3) / 1e9
        del host, dst
        return {"records": "layer 0 expert records in pinned host memory; one step = one layer",
                "record_bytes_per_expert": round(rec), "mean_unique_experts": round(u_mean, 2),
                "staged_bytes_per_step": round(staged),
                "split": {"ms_per_step": round(ms_split, 4),
                          "tokens_per_s": round(cfg.T / (ms_split / 1e3), 1),
                          "staged_GBps": round(sel, 2)},
                "serial": {"ms_per_step": round(ms_serial, 4),
                           "tokens_per_s": round(cfg.T / (ms_serial / 1e3), 1),
                           "staged_GBps": round(staged / (ms_serial / 1e3) / 1e9, 2)},
                "full_extent": {"bytes": round(cfg.E * rec),
                                "stage_kernel_GBps": round(full_kernel, 2),
                                "host_to_device_copy_GBps": round(full_copy, 2)},
                "crossover_unique_experts": round(cfg.E * sel / max(full_kernel, full_copy), 1)}
    except Exception as e:   # optional measurement; the resident numbers stand
        return {"error": f"{type(e).__name__}: {e}"}


def fused_waves(M, torch, dev, cfg, layers, xs, reps=50):
    """The fused gate/up -> down kernel (moe_ffn_fused) next to the two-kernel
    FFN on layer 0 of the workload: FFN time per wave width (1, 2, 4 tiles and
    all), the whole layer with MOE_F_FUSED_FFN against the default layer, and
    the wave completion profile read from the kernel's per-item clock (for
    each wave, the last item's gate/up and down completion, from the first
    item's start)."""
    try:
        wr, bias, _, exg = layers[0]
        mk = lambda fused: M.MoELayerBuffers(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt,
                                             device=dev, tiled=True, fused=fused)
        b0, b1 = mk(False), mk(True)
        res = (lambda x: x) if cfg.residual else (lambda x: None)

        def timeit(fn):
            for i in range(5):
                fn(i)
            torch.cuda.synchronize()
            a, b = TimingEvent(), TimingEvent()
            a.record()
            for i in range(reps):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps * 1e3

        lay0 = timeit(lambda i: b0.layer(xs[i % len(xs)], wr, bias, exg, residual=res(xs[i % len(xs)])))
        lay1 = timeit(lambda i: b1.layer(xs[i % len(xs)], wr, bias, exg, residual=res(xs[i % len(xs)])))
        x = xs[0]
        for b in (b0, b1):
            b.route(x, wr, bias, logits=False)
            b.permute()
        two = timeit(lambda i: (b0.ffn_gate_up(x, exg), b0.ffn_down(exg)))
        widths = {"1": 1, "2": 2, "4": 4, "all": 0}
        fused = {n: round(timeit(lambda i: b1.ffn_fused(x, exg, wave_tiles=w)), 2) for n, w in widths.items()}
        khz = M.moe_device_clock_khz()
        S = cfg.I // 64
        cap = M.moe_ffn_fused_items(b1.shape)
        clock = torch.zeros(3 * cap, dtype=torch.int64, device=dev)
        prof = {}
        for n, w in widths.items():
            clock.zero_()
            b1.ffn_fused(x, exg, wave_tiles=w, item_clock=clock)
            torch.cuda.synchronize()
            c = clock.view(-1, 3).cpu().numpy()
            c = c[c[:, 0] > 0]
            per = (w if w else len(c) // S) * S
            wave = np.arange(len(c)) // per
            t0 = c[:, 0].min()
            gu = np.array([c[wave == v, 1].max() for v in np.unique(wave)]) - t0
            dn = np.array([c[wave == v, 2].max() for v in np.unique(wave)]) - t0
            us = 1e3 / khz
            prof[n] = {"waves": int(wave.max() + 1), "items": int(len(c)),
                       "gate_up_done_us_first_median_last": [round(float(v * us), 2) for v in
                                                             (gu.min(), np.median(gu), gu.max())],
                       "down_done_us_first_median_last": [round(float(v * us), 2) for v in
                                                          (dn.min(), np.median(dn), dn.max())]}
        del b0, b1, clock
        return {"layer_us": {"two_kernel": round(lay0, 2), "fused": round(lay1, 2)},
                "ffn_us": {"two_kernel": round(two, 2), "fused_by_wave_tiles": fused},
                "wave_completion": prof, "clock_khz": khz}
    except Exception as e:   # optional measurement
        return {"error": f"{type(e).__name__}: {e}"}


def read_probe(M, dev, mib):
    """Read bandwidth of the plain streaming probe kernel (moe_stream_read) over
    a buffer of `mib` MiB: median of 5 timed passes after 2 untimed ones."""
    import torch
    n = mib << 20
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        M.moe_stream_read(buf, n, sink)
    ms = []
    for _ in range(5):
        a, b = TimingEvent(), TimingEvent()
        a.record()
        M.moe_stream_read(buf, n, sink)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    del buf
    return round(n / (float(np.median(ms)) / 1e3) / 1e9, 1)


def cpu_baseline(cfg, L, layers, xs, budget_s, dev):
    """The CPU oracle, untuned, on a bounded sample of the same workload: whole
    batches of the first layer(s), until the budget is spent.  Stacked
    workloads are extrapolated from the layers sampled (tokens/s = T /
    (mean seconds per layer * layers)).  The oracle reads row-major weights,
    regenerated from the same seeds (the device may hold the tiled copy).
    Batches above 4096 tokens are sampled as their first 4096 tokens (one
    window; the oracle's cost per token does not depend on T)."""
    import threadpoolctl
    import torch

    from moe_inputs import make_experts
    from moe_inputs import tensor_to_numpy_storage as npy
    from oracle import moe_oracle as O

    threads = os.cpu_count() or 1
    layer_s, tokens = [], 0
    t_budget = time.perf_counter()
    with threadpoolctl.threadpool_limits(threads):
        for b in range(len(xs)):
            tcpu = min(cfg.T, 4096)
            x64 = O.decode_act(npy(xs[b][:tcpu]), cfg.act)
            for l in range(L):
                wr, bias, _, _ = layers[l]
                ex = make_experts(cfg, l, dev)
                wr64 = O.decode_act(npy(wr), cfg.act)
                b64 = None if bias is None else bias.double().cpu().numpy()
                # host copies of the experts this batch selects (copies are not timed)
                ids = O.select_topk(O.router_logits(x64, wr64, b64), cfg.k)
                need = np.unique(ids)
                host = {n: {int(e): npy(ex[n][int(e)]) for e in need} if ex[n] is not None else None
                        for n in ("gate", "up", "down", "gate_scale", "up_scale", "down_scale")}
                oex = O.ExpertWeights(cfg.wfmt, cfg.act, cfg.H, cfg.I, host["gate"], host["up"],
                                      host["down"], host["gate_scale"], host["up_scale"],
                                      host["down_scale"])
                del ex
                torch.cuda.empty_cache()
                c0, t0 = time.process_time(), time.perf_counter()
                r = O.moe_layer(x64, wr64, b64, oex, cfg.k, residual=x64 if cfg.residual else None)
                x64 = O.act_round(r.out, cfg.act)
                layer_s.append((time.perf_counter() - t0, time.process_time() - c0))
                if time.perf_counter() - t_budget > budget_s:
                    break
            tokens += tcpu
            if time.perf_counter() - t_budget > budget_s:
                break
    wall = sum(w for w, _ in layer_s)
    cpu_t = sum(c for _, c in layer_s)
    per_layer = wall / len(layer_s)
    tcpu = min(cfg.T, 4096)
    return {"value": round(tcpu / (per_layer * L), 3), "unit": "tokens/s",
            "cores": threads, "avg_busy_threads": round(cpu_t / wall, 2), "kind": "oracle (numpy)",
            "sample": f"{len(layer_s)} layer passes of {tcpu}"
                      f"{'' if tcpu == cfg.T else ' of the ' + str(cfg.T)} tokens (float64 numpy oracle, "
                      f"{'extrapolated to ' + str(L) + ' layers' if L > 1 else 'whole layer'}); "
                      f"host copies of the selected experts excluded"}


def oracle_route_check(cfg, layers, xs, gpu_routes):
    """GPU routes of layer 0 against the C++ float64 oracle, on the generator's
    bytes of every recorded batch (x, router weight, bias): expert IDs must
    match exactly except on near-tie tokens (the oracle's k+1 best logits have
    an adjacent gap below 1e-6 relative), which are counted separately; the
    GPU's float32 logits are compared with the oracle's float64 logits."""
    from moe_inputs import tensor_to_numpy_storage as npy
    from oracle import moe_oracle as O
    from oracle import oracle_c as C

    if not gpu_routes:
        return None
    wr, bias, _, _ = layers[0]
    wr64 = C.decode_act_c(npy(wr), cfg.act)
    b64 = None if bias is None else bias.double().cpu().numpy()
    n = mism = bad = near = 0
    dmax = rmax = 0.0
    t0 = time.perf_counter()
    for b, ids_gpu, lg_gpu in gpu_routes:
        x64 = C.decode_act_c(npy(xs[b]), cfg.act)
        lg, ids, _, _ = C.routes_c(x64, wr64, b64, cfg.k)
        nt = O.near_tie_tokens(lg, cfg.k)
        mm = (ids_gpu != ids).any(axis=1)
        n += len(ids)
        mism += int(mm.sum())
        bad += int((mm & ~nt).sum())
        near += int(nt.sum())
        d = np.abs(lg_gpu.astype(np.float64) - lg)
        dmax = max(dmax, float(d.max()))
        rmax = max(rmax, float((d / np.maximum(np.abs(lg), 1e-30)).max()))
    return {"tokens": n, "layer": 0, "batches": len(gpu_routes), "mismatched_tokens": mism,
            "mismatches_outside_near_ties": bad, "near_tie_tokens": near,
            "max_abs_dlogit": dmax, "max_rel_dlogit": rmax,
            "oracle": "C++ float64 (routes_c) on the generator's bytes",
            "seconds": round(time.perf_counter() - t0, 2)}


def cpu_baseline_cxx(cfg, L, layers, xs, budget_s, dev):
    """The plain C++ float64 oracle (oracle/moe_oracle_c.cpp), untuned, on a
    bounded sample: the first min(T, 64) tokens of each batch through the
    first layer(s) until the budget is spent, extrapolated per layer (tokens/s
    = tokens / (mean seconds per layer * layers)).  Its inputs are host copies
    of the batch (decoded by the C++ oracle) and of the experts its own router
    selects for the sample (the others stay zero pages); copies are not
    timed.  One thread per output row, all host cores."""
    import torch

    from moe_inputs import make_experts
    from moe_inputs import tensor_to_numpy_storage as npy
    from oracle import oracle_c as C

    threads = os.cpu_count() or 1
    tcpu = min(cfg.T, 64)
    layer_s = []
    t_budget = time.perf_counter()
    for b in range(len(xs)):
        x64 = C.decode_act_c(npy(xs[b][:tcpu]), cfg.act)
        for l in range(L):
            wr, bias, _, _ = layers[l]
            ex = make_experts(cfg, l, dev)
            wr64 = C.decode_act_c(npy(wr), cfg.act)
            b64 = None if bias is None else bias.double().cpu().numpy()
            need = np.unique(C.routes_c(x64, wr64, b64, cfg.k, threads=threads)[1])
            host = {}
            for n, t in ex.items():
                if t is None:
                    host[n] = None
                    continue
                one = npy(t[:1])
                a = np.zeros((t.shape[0],) + one.shape[1:], dtype=one.dtype)
                for e in need:
                    a[int(e)] = npy(t[int(e)])
                host[n] = a
            del ex
            torch.cuda.empty_cache()
            t0 = time.perf_counter()
            r = C.moe_layer_c(x64, wr64, b64, host, cfg.wfmt, cfg.act, cfg.k,
                              x64 if cfg.residual else None, threads=threads)
            layer_s.append(time.perf_counter() - t0)
            x64 = (C.decode_act_c(C.round_bf16_c(r.out), "bf16") if cfg.act == "bf16"
                   else r.out.astype(np.float32).astype(np.float64))
            if time.perf_counter() - t_budget > budget_s:
                break
        if time.perf_counter() - t_budget > budget_s:
            break
    per_layer = sum(layer_s) / len(layer_s)
    return {"value": round(tcpu / (per_layer * L), 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(layer_s)} layer passes of {tcpu}"
                      f"{'' if tcpu == cfg.T else ' of the ' + str(cfg.T)} tokens (float64 C++ oracle, "
                      f"{'extrapolated to ' + str(L) + ' layers' if L > 1 else 'whole layer'}); "
                      f"host copies excluded"}


if __name__ == "__main__":
    main()
