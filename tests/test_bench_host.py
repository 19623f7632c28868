"""Host-side pieces of bench.py, checked on the CPU: the algorithmic byte and
flop counts behind the roofline (against the per-expert record sizes fixed
by the layer geometry: 3 x 640 x 2560 = 4,915,200 parameters), the
code-only digest that ties the committed PMC summaries to the kernel
sources, and the single-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench
from moe_inputs import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PARAMS = 4_915_200


@pytest.mark.parametrize("name,record", [("decode", 9_830_400), ("stack_int4", 2_764_800),
                                         ("verify_int2", 1_536_000)])
def test_layer_bytes_use_the_record_sizes(name, record):
    cfg = get_config(name)
    assert 3 * cfg.I * cfg.H == PARAMS
    fixed = cfg.E * cfg.H * 2 + 2 * cfg.T * cfg.H * 2       # router weight, x in and out
    assert bench.layer_bytes(cfg, 0) == fixed
    assert bench.layer_bytes(cfg, 75) - fixed == pytest.approx(75 * record, rel=0, abs=1e-6)


def test_gateup_bytes_and_flops_closed_form():
    cfg = get_config("decode")
    U, P = 75, cfg.T * cfg.k
    b, f = bench.gateup_traffic(cfg, U)
    # the weights of the active experts and the token rows; the intermediate
    # the kernel writes is scratch and not counted
    assert b == U * 2 * 640 * 2560 * 2 + 8 * 2560 * 2
    assert f == 2.0 * P * 2 * 640 * 2560
    # gate + up are two thirds of an expert record
    cfg4 = get_config("stack_int4")
    b4, _ = bench.gateup_traffic(cfg4, 1)
    assert b4 - cfg4.T * cfg4.H * 2 == pytest.approx(2_764_800 * 2 / 3)


def test_digest_ignores_comments_not_code():
    src = "int f(int a) {\n  // one\n  return a + 1; /* two */\n}\n"
    same = "int f(int a) {   return a + 1;\n}  // other comment\n"
    other = "int f(int a) { return a + 2; }"
    assert bench._code_only("k.hip", src) == bench._code_only("k.hip", same)
    assert bench._code_only("k.hip", src) != bench._code_only("k.hip", other)
    py = "x = 1  \n# note\ny = 2\n"
    assert bench._code_only("b.py", py) == bench._code_only("b.py", "x = 1\ny = 2")
    assert len(bench.kernel_source_digest()) == 16


@pytest.mark.parametrize("workload", ["decode", "verify_int2", "stack_int4", "prefill",
                                      "prefill_merged"])
def test_traffic_only_for_the_recorded_digest(workload):
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_pmc.txt")
    recorded = None
    with open(path) as f:
        for line in f:
            if line.startswith("kernel_source_digest:"):
                recorded = line.split(":", 1)[1].strip()
    assert recorded
    t = bench.traffic_from_profiles(workload, recorded)
    assert t is not None and t > 0
    assert bench.traffic_from_profiles(workload, "0" * 16) is None


def test_default_run_covers_every_workload():
    assert set(bench.OTHER_WORKLOADS) | {"decode"} == {"tiny", "decode", "prefill", "stack_int4",
                                                      "verify_int2"}
    line = {"value": 1.0, "unit": "tokens/s", "steps": 2, "warmup": 1, "ms_per_step": 1.0,
            "dtype": "bf16", "config": {}, "timing": {}, "layer_hbm": {}, "graph": None,
            "cpu_baseline": None, "oracle_route_check": None, "route_locality": {},
            "roofline": {k: 0 for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                        "kernel", "avg_launch_us", "hbm_frac", "mfma_frac",
                                        "attainable_frac", "kernel_source_digest")}}
    s = bench.summarize(line)
    assert "route_locality" not in s and "kernel_source_digest" not in s["roofline"]
    assert s["roofline"]["attainable_frac"] == 0 and s["oracle_route_check"] is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
