"""The low-bit 16-row-tile FFN kernels on chosen token values.  For int2,
token dwords 1 and 2 of every MFMA fragment are divided by 4 and 16 with an
exponent step before they meet codes masked in place, and the SwiGLU rows
feeding down are staged that way too; for both formats tiles of at most 4
rows use the 4-row layout.  So zero and negative-zero elements, all-zero
rows, small magnitudes and mixed signs must come out of gate/up and down as
the float64 oracle computes them, in tiles of both layouts (at most 4 rows,
and more).  A non-finite token value, in a prescaled dword or not, must make
every output of that token non-finite and leave the other tokens' outputs as
they are.

Expected values: the oracle's SwiGLU intermediate and down projection on the
same expert records ("Agent Field Notes -- full corpus", AFN-001, section
"Phase 1: separate math from acceleration"); the routes are forced (any
top-k ids define the grouping) and the permutation is checked against the
oracle's first."""
import numpy as np
import pytest
import torch

from moe_inputs import CONFIGS
from oracle import moe_oracle as O
from tests.gpu_util import DEV, buffers, check_values, decode, i32, make_case, say, to_act_tensor

pytestmark = pytest.mark.gpu

# low-bit g32 experts, tiled; H = 1024: four k parts of two 128-wide units
# per gate/up wave (a rolled unit and the last one), I = 256: two units in
# down
CFG = CONFIGS[5].with_(T=24, H=1024, E=32, I=256, k=4, layers=1)
WFMTS = ["int2_g32", "int4_g32"]
TINY = 2.0 ** -40


def forced_ids(T):
    """Four distinct experts per token: 4 experts of 6 rows, 7 of 3-4, 5 of
    4-5 and 16 of 1-2, so both tile layouts occur."""
    t = np.arange(T)
    return np.stack([t % 4, 4 + t % 7, 11 + t % 5, 16 + t % 16], axis=1).astype(np.int32)


def special_rows(v, rng):
    """Rows 0-4 of `v` (tokens or pair rows): all zero, negative zeros every
    third element, small magnitudes, zeros every other element, and values
    on a coarse grid with both signs."""
    v = v.copy()
    v[0] = 0.0
    v[1, ::3] = -0.0
    v[2] *= TINY
    v[3, ::2] = 0.0
    v[4] = np.round(v[4] * 4.0) / 4.0
    return O.round_to_bf16(v)


def poison(v, rows):
    """+inf in a dword-1 position (k % 8 == 2, prescaled by 1/4), -inf in a
    dword-0 position (k % 8 == 0, not prescaled), NaN in a dword-2 position
    (k % 8 == 5, prescaled by 1/16)."""
    v = v.copy()
    v[rows[0], 8 * 3 + 2] = np.inf
    v[rows[1], 8 * 5 + 0] = -np.inf
    v[rows[2], 8 * 7 + 5] = np.nan
    return v


def rel_check(got, ref, what):
    """Rows of small values: error relative to the row's largest value."""
    scale = np.abs(ref).max()
    assert scale > 0, what
    err = float(np.abs(got - ref).max()) / scale
    assert err <= 2e-2, f"{what}: relative error {err:.3g}"
    return err


@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("poisoned", [False, True], ids=["finite", "nonfinite"])
def test_lowbit_gateup_special_tokens(poisoned, wfmt):
    cfg = CFG.with_(wfmt=wfmt)
    case = make_case(cfg)
    rng = np.random.default_rng(5)
    ids = forced_ids(cfg.T)
    ref_perm = O.permutation(ids, cfg.E)
    x64 = special_rows(rng.standard_normal((cfg.T, cfg.H)), rng)
    bad = np.array([5, 6, 7]) if poisoned else np.array([], dtype=int)
    if poisoned:
        x64 = poison(x64, bad)
    buf = buffers(cfg, tiled=True)
    say(f"[{wfmt} special values gate/up poisoned={poisoned}] moe_permute on forced ids")
    buf.permute(topk_ids=i32(ids))
    torch.cuda.synchronize()
    assert np.array_equal(buf.sorted_pair.cpu().numpy(), ref_perm.sorted_pair)
    rows_per_expert = np.diff(ref_perm.offsets)[ref_perm.active]
    assert (rows_per_expert <= 4).any() and (rows_per_expert > 4).any()
    say(f"[{wfmt} special values gate/up poisoned={poisoned}] moe_ffn_gate_up")
    buf.ffn_gate_up(to_act_tensor(x64, "bf16"), case.experts(True))
    torch.cuda.synchronize()
    got = decode(buf.h, "bf16")
    tok = ref_perm.sorted_pair // cfg.k                  # token of each permuted row
    A = O.grouped_intermediate(np.where(np.isfinite(x64), x64, 0.0), ref_perm, cfg.k, case.ex_oracle)
    sick = np.isin(tok, bad)
    if poisoned:
        assert not np.isfinite(got[sick]).any(), "a non-finite token produced finite outputs"
    fine = ~sick & (tok != 2)
    stats = check_values(got[fine], A[fine], "bf16", "h")
    small = tok == 2
    rel = rel_check(got[small], A[small], "h (small token)")
    zero = tok == 0
    assert (got[zero] == 0).all(), "an all-zero token gave nonzero outputs"
    say(f"[{wfmt} special values gate/up poisoned={poisoned}] h {stats}, small-token rel {rel:.3g}")


@pytest.mark.parametrize("wfmt", WFMTS)
@pytest.mark.parametrize("poisoned", [False, True], ids=["finite", "nonfinite"])
def test_lowbit_down_special_rows(poisoned, wfmt):
    cfg = CFG.with_(wfmt=wfmt)
    case = make_case(cfg)
    rng = np.random.default_rng(6)
    ids = forced_ids(cfg.T)
    ref_perm = O.permutation(ids, cfg.E)
    P = cfg.T * cfg.k
    tok = ref_perm.sorted_pair // cfg.k
    # intermediate rows in permuted order; the special rows are those of
    # tokens 0-4 (token t's rows get pattern t)
    A = O.round_to_bf16(0.5 * rng.standard_normal((P, cfg.I)))
    for t in range(5):
        rows = np.nonzero(tok == t)[0]
        pat = special_rows(np.tile(0.5 * rng.standard_normal((1, cfg.I)), (5, 1)), rng)[t]
        A[rows] = pat
    bad_rows = np.nonzero(np.isin(tok, [5, 6, 7]))[0] if poisoned else np.array([], dtype=int)
    if poisoned:
        # the three kinds of poison() in turn over the rows of tokens 5-7
        kinds = [(8 * 3 + 2, np.inf), (8 * 5 + 0, -np.inf), (8 * 7 + 5, np.nan)]
        for i, r in enumerate(bad_rows):
            c, v = kinds[i % 3]
            A[r, c] = v
    buf = buffers(cfg, tiled=True)
    say(f"[{wfmt} special values down poisoned={poisoned}] moe_permute + moe_ffn_down")
    buf.permute(topk_ids=i32(ids))
    buf.ffn_down(case.experts(True), h=to_act_tensor(A, "bf16"))
    torch.cuda.synchronize()
    got = decode(buf.y, "bf16")
    Y = O.grouped_down(np.where(np.isfinite(A), A, 0.0), ref_perm, case.ex_oracle)
    sick = np.zeros(P, dtype=bool)
    sick[bad_rows] = True
    if poisoned:
        assert not np.isfinite(got[sick]).any(), "a non-finite row produced finite outputs"
    fine = ~sick & (tok != 2)
    stats = check_values(got[fine], Y[fine], "bf16", "y")
    small = tok == 2
    rel = rel_check(got[small], Y[small], "y (small rows)")
    zero = tok == 0
    assert (got[zero] == 0).all(), "all-zero rows gave nonzero outputs"
    say(f"[{wfmt} special values down poisoned={poisoned}] y {stats}, small-row rel {rel:.3g}")
