"""Planted mistakes in the C++ oracle must fail its pins.

Each case copies oracle/moe_oracle_c.cpp, changes one expression into a
plausible mistake, builds the copy with g++ into a temporary directory and
runs checks of test_oracle_c.py against it (comparison with the numpy
oracle on every case, equal logits going to the lower index); at least one
must fail.  The mistakes live only in the temporary copies."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import oracle_c as C
from tests import test_oracle_c as T

MUTATIONS = {
    "bias_dropped": ("if (bias) s += bias[e];", ""),
    "ties_to_higher_index": ("(l[f] == l[e] && f < e)", "(l[f] == l[e] && f > e)"),
    "gate_up_swapped": ("a_[i] = g / (1.0 + std::exp(-g)) * u;",
                        "a_[i] = u / (1.0 + std::exp(-u)) * g;"),
    "codes_unsigned": ("if (q >= (1 << (bits - 1))) q -= (1 << bits);", ""),
    "code_order_swapped": ("const int bit = c * bits;", "const int bit = (c ^ 1) * bits;"),
    "wrong_scale_group": ("fp16_to_double(s[c / 32])", "fp16_to_double(s[(c / 32 + 1) % (K / 32)])"),
    "not_renormalized": ("(std::exp(l[ids[static_cast<size_t>(t) * k + j]] - m) / z) / sel;",
                         "(std::exp(l[ids[static_cast<size_t>(t) * k + j]] - m) / z);"),
    "combine_unweighted": ("s += w[static_cast<size_t>(t) * k + j] *", "s += 1.0 *"),
    "fp16_exponent_bias": ("exp - 25)", "exp - 24)"),
}


def _fails(lib) -> bool:
    try:
        for name in T.CASES:
            cfg = T.CASES[name]
            x64, wr64, b64, st, ex, res = T._inputs(cfg)
            got = C.moe_layer_c(x64, wr64, b64, st, cfg.wfmt, cfg.act, cfg.k, res, lib=lib)
            ref = T.O.moe_layer(x64, wr64, b64, ex, cfg.k, residual=res)
            np.testing.assert_array_equal(got.ids, ref.ids)
            T._close(got.w, ref.w, "weights")
            T._close(got.out, ref.out, "out")
        # equal logits (zero router): experts 0..k-1 in order
        cfg = T.CASES["tiny_f32"]
        x64, wr64, _, st, _, _ = T._inputs(cfg)
        got = C.moe_layer_c(x64, np.zeros_like(wr64), None, st, cfg.wfmt, cfg.act, cfg.k, lib=lib)
        np.testing.assert_array_equal(got.ids, np.tile(np.arange(cfg.k), (cfg.T, 1)))
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    with open(C.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    with tempfile.TemporaryDirectory() as d:
        cpp, so = os.path.join(d, "m.cpp"), os.path.join(d, "m.so")
        with open(cpp, "w") as f:
            f.write(src.replace(old, new))
        r = subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-pthread", cpp, "-o",
                            so], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        assert _fails(C.load_from(so)), f"no check caught the planted mistake {name}"


def test_unmutated_copy_passes():
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "m.so")
        r = subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-pthread", C.SRC, "-o",
                            so], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        assert not _fails(C.load_from(so))
