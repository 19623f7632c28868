"""The two 48-layer stacks at full size, every layer checked against the C++
float64 oracle, in the launch configuration bench.py times (tiled weights,
the staged calls route -> permute -> gate/up -> down -> combine).

Layers run strictly in sequence, each fed the previous layer's output plus
its residual ("Agent Field Notes -- full corpus", AFN-019, section
"Hypothesis H6": later-layer routes depend on earlier-layer results); expert
IDs must match exactly and in rank order (AFN-021, section "The key
equivalence -- and where it breaks").

Direction of data (oracle -> GPU only): the oracle runs its own 48-layer
chain from the generator's x_0 on a set S of tokens (all 16 tokens of the
verifier block; 8 seeded tokens of the 512-token window), rounding to bf16 at
every layer boundary like the storage type.  Before each GPU layer the rows S
of the GPU input are overwritten with the oracle's x_l (exact in bf16), so
every layer is checked on the oracle's own input (teacher forcing); the other
rows carry the GPU's own chain.  Every step of the layer is per token, so the
oracle on S alone gives those tokens' exact results.

Per layer: routes of S bit-exact except near-tie tokens (counted), expert
outputs y of every (token, slot) pair of S (the MoE term without the
residual, which would otherwise dominate the comparison) and the layer
output of S within the bf16 tolerance, its max-abs bound taken at unit scale
row by row (max-abs of a row / max(1, rms of the oracle row)) because the
residual stream, and with it the expert outputs, grows layer by layer and the
bf16 rounding errors grow with it.  Reported,
not graded: unique experts per layer (whole batch), the repeat fraction of
the verifier block, near ties, the largest logit difference, and the
free-running drift of a second GPU chain that is never forced (its x_l on S
against the oracle's).
"""
import json
import os

import numpy as np
import pytest
import torch

import sparse_moe_routed_amd as M
from moe_inputs import CONFIGS, make_experts, make_router, make_x
from oracle import moe_oracle as O
from oracle import oracle_c as C
from tests.gpu_util import (DEV, TOL_BF16_ABS, TOL_BF16_RL2, check_routes, check_values, host_experts,
                            np_of, say, to_act_tensor)

pytestmark = pytest.mark.gpu

CASES = [("verify_int2", CONFIGS[5], None), ("stack_int4", CONFIGS[4], 8)]


def _report_dir():
    d = os.environ.get("MOE_REPORT_DIR", "gpurun_out")
    return d if os.path.isdir(d) else None


def _tiled(cfg, ex):
    mk = lambda d: M.make_experts(d["gate"], d["up"], d["down"], d["gate_scale"], d["up_scale"],
                                  d["down_scale"])
    dst = {n: (None if t is None else torch.empty_like(t)) for n, t in ex.items()}
    M.moe_tile_experts(M.make_shape(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k, cfg.act, cfg.wfmt), mk(ex),
                       mk(dst))
    return dst, mk(dst)


def _gpu_layer(buf, x, wr, bias, exg, out, logits):
    buf.route(x, wr, bias, logits=logits)
    buf.permute()
    buf.ffn_gate_up(x, exg)
    buf.ffn_down(exg)
    buf.combine(residual=x, out=out)


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("name,cfg,n_sample", CASES, ids=[c[0] for c in CASES])
def test_stack_48_layers(name, cfg, n_sample):
    T, k, L = cfg.T, cfg.k, cfg.layers
    assert L == 48
    S = (np.arange(T) if n_sample is None else
         np.sort(np.random.default_rng(4800 + cfg.seed).choice(T, size=n_sample, replace=False)))
    St = torch.from_numpy(S).to(DEV)
    x0 = make_x(cfg, DEV, batch=0)
    xo = C.decode_act_c(np_of(x0)[S], cfg.act)                # oracle chain on S
    xg = x0.clone()                                           # GPU chain, S forced
    xf = x0.clone()                                           # GPU chain, free
    outg, outf = torch.empty_like(x0), torch.empty_like(x0)
    buf = M.MoELayerBuffers(T, cfg.H, cfg.E, cfg.I, k, cfg.act, cfg.wfmt, device=DEV, tiled=True)
    rows, worst = [], {"y_abs": 0.0, "y_scaled": 0.0, "y_rl2": 0.0, "out_abs": 0.0, "out_scaled": 0.0,
                       "out_rl2": 0.0}
    say(f"[stack48 {name}] T={T} sample={len(S)} tokens, {cfg.wfmt}, 48 layers")
    for l in range(L):
        wr, bias = make_router(cfg, l, DEV)
        ex = make_experts(cfg, l, DEV)
        _keep, exg = _tiled(cfg, ex)
        # ---- oracle layer l on S (its own input, its own routes pick the experts)
        wr64 = C.decode_act_c(np_of(wr), cfg.act)
        b64 = None if bias is None else bias.double().cpu().numpy()
        need = np.unique(C.routes_c(xo, wr64, b64, k)[1])
        ref = C.moe_layer_c(xo, wr64, b64, host_experts(ex, need), cfg.wfmt, cfg.act, k, xo)
        # ---- GPU layer l, rows S forced to the oracle's x_l
        xg[St] = to_act_tensor(xo, cfg.act)
        _gpu_layer(buf, xg, wr, bias, exg, outg, logits=True)
        torch.cuda.synchronize()
        ids = buf.topk_ids.cpu().numpy()[S]
        stats, same = check_routes(ids, buf.topk_w.cpu().numpy()[S].astype(np.float64),
                                   ref.logits, ref.ids, ref.w, k)
        dlogit = float(np.abs(buf.logits.cpu().numpy()[S].astype(np.float64) - ref.logits).max())
        # expert outputs per pair of S (GPU rows through the GPU permutation,
        # oracle rows through the oracle's)
        pr = buf.pair_row.cpu().numpy()
        ys = np_of(buf.y)
        p_gpu = (S[:, None] * k + np.arange(k)[None, :])[same].ravel()
        p_ref = (np.arange(len(S))[:, None] * k + np.arange(k)[None, :])[same].ravel()
        yv = check_values(O.decode_act(ys[pr[p_gpu]], cfg.act), ref.Y[ref.perm.pair_row[p_ref]],
                          cfg.act, f"{name} layer {l} y", scaled=True)
        ov = check_values(O.decode_act(np_of(outg)[S], cfg.act)[same], ref.out[same], cfg.act,
                          f"{name} layer {l} out", scaled=True)
        n_active = int(buf.n_active.item())
        # ---- free-running GPU chain (never forced), reported only
        _gpu_layer(buf, xf, wr, bias, exg, outf, logits=False)
        # ---- next layer's inputs
        xo = C.decode_act_c(C.round_bf16_c(ref.out), "bf16")
        xg, outg = outg, xg
        xf, outf = outf, xf
        torch.cuda.synchronize()
        drift = _rel_l2(O.decode_act(np_of(xf)[S], cfg.act), xo)
        row = {"layer": l, "unique_experts": n_active, "near_ties": stats["near_ties"],
               "mismatches": stats["mismatch"], "max_abs_dlogit": dlogit,
               "y_max_abs": yv["max_abs"], "y_max_scaled": yv["max_scaled"], "y_rel_l2": yv["rel_l2"],
               "out_max_abs": ov["max_abs"], "out_max_scaled": ov["max_scaled"],
               "out_rel_l2": ov["rel_l2"], "y_rms": yv["rms_ref"], "out_rms": ov["rms_ref"],
               "free_drift_rel_l2": drift,
               "max_abs_x": float(np.abs(xo).max())}
        if n_sample is None:
            row["repeat_fraction"] = O.repeat_fraction(ref.ids)
            row["unique_experts_oracle"] = int(ref.perm.n_active)
        rows.append(row)
        worst["y_abs"] = max(worst["y_abs"], yv["max_abs"])
        worst["y_scaled"] = max(worst["y_scaled"], yv["max_scaled"])
        worst["out_scaled"] = max(worst["out_scaled"], ov["max_scaled"])
        worst["y_rl2"] = max(worst["y_rl2"], yv["rel_l2"])
        worst["out_abs"] = max(worst["out_abs"], ov["max_abs"])
        worst["out_rl2"] = max(worst["out_rl2"], ov["rel_l2"])
        if l % 8 == 7 or l == 0:
            say(f"  layer {l}: U={n_active} routes {stats} |dlogit|={dlogit:.2g} "
                f"y {yv['max_abs']:.3g}/{yv['rel_l2']:.3g} (rms {yv['rms_ref']:.3g}) "
                f"out {ov['max_abs']:.3g}/{ov['rel_l2']:.3g} (rms {ov['rms_ref']:.3g})"
                f" free drift {drift:.3g}"
                + (f" repeat {row['repeat_fraction']:.2f}" if n_sample is None else ""))
        del ex, _keep, exg
    summary = {
        "workload": name, "tokens_checked": [int(t) for t in S], "layers": L,
        "tolerance": {"max_abs": TOL_BF16_ABS, "rel_l2": TOL_BF16_RL2},
        "worst": worst,
        "near_tie_tokens_total": int(sum(r["near_ties"] for r in rows)),
        "route_mismatches_total": int(sum(r["mismatches"] for r in rows)),
        "max_abs_dlogit": max(r["max_abs_dlogit"] for r in rows),
        "mean_unique_experts": float(np.mean([r["unique_experts"] for r in rows])),
        "free_drift_rel_l2_last_layer": rows[-1]["free_drift_rel_l2"],
        "per_layer": rows,
    }
    if n_sample is None:
        summary["mean_repeat_fraction"] = float(np.mean([r["repeat_fraction"] for r in rows]))
    say(f"[stack48 {name}] worst y {worst['y_abs']:.3g} (scaled {worst['y_scaled']:.3g})/"
        f"{worst['y_rl2']:.3g}, out {worst['out_abs']:.3g} (scaled {worst['out_scaled']:.3g})/"
        f"{worst['out_rl2']:.3g}; near ties {summary['near_tie_tokens_total']}, "
        f"mismatches {summary['route_mismatches_total']}, free drift at layer 48 "
        f"{summary['free_drift_rel_l2_last_layer']:.3g}")
    d = _report_dir()
    if d:
        with open(os.path.join(d, f"stack48_{name}.json"), "w") as f:
            json.dump(summary, f, indent=1)
