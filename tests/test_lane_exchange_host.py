"""Host model of the router top-k's wave reductions (no GPU needed).

The top-k kernel reduces over the 64 lanes of a wave in six exchange steps:
two DPP quad permutations, the DPP half-row and row mirrors, and the
v_permlane16_swap / v_permlane32_swap pair.  This test reads the four DPP
control words from the kernel source, applies them with the lane semantics
of the gfx9 DPP controls (quad_perm selects a lane within each group of 4;
row_half_mirror reverses each group of 8; row_mirror each row of 16) and of
the two swaps (lanes l and l ^ 16, then l and l ^ 32, trade values), and
checks that after the six steps every lane has met every other lane: a
wrong control word (a pairing inside an already-reduced group) leaves some
lanes out and fails here.
"""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROUTE = os.path.join(ROOT, "sparse_mixture_experts_15_amd", "csrc", "route.hip")


def _dpp_controls():
    src = open(ROUTE).read()
    m = re.search(r"ctrl = S == 0 \? (0x[0-9A-Fa-f]+) : S == 1 \? (0x[0-9A-Fa-f]+) : "
                  r"S == 2 \? (0x[0-9A-Fa-f]+) : (0x[0-9A-Fa-f]+);", src)
    assert m, "DPP control words not found in route.hip"
    return [int(v, 16) for v in m.groups()]


def _dpp_source_lane(ctrl, lane):
    """Lane whose value `lane` receives under a gfx9 DPP control word."""
    if ctrl <= 0xFF:                        # quad_perm
        sel = (ctrl >> (2 * (lane & 3))) & 3
        return (lane & ~3) | sel
    if ctrl == 0x140:                       # row_mirror: reverse within 16 lanes
        return (lane & ~15) | (15 - (lane & 15))
    if ctrl == 0x141:                       # row_half_mirror: reverse within 8 lanes
        return (lane & ~7) | (7 - (lane & 7))
    raise AssertionError(f"unmodelled DPP control 0x{ctrl:x}")


def _partners(step, ctrls):
    if step < 4:
        return [_dpp_source_lane(ctrls[step], l) for l in range(64)]
    off = 16 if step == 4 else 32
    return [l ^ off for l in range(64)]


def test_six_steps_reach_every_lane():
    ctrls = _dpp_controls()
    # each lane's set of lanes whose values it has combined
    seen = [{l} for l in range(64)]
    for step in range(6):
        p = _partners(step, ctrls)
        # every step pairs lanes symmetrically, so both lanes of a pair end
        # with the same combined value
        assert all(p[p[l]] == l and p[l] != l for l in range(64)), f"step {step} not a pairing"
        seen = [seen[l] | seen[p[l]] for l in range(64)]
    assert all(s == set(range(64)) for s in seen)


def test_argmax_model_matches_a_plain_argmax():
    """The reduction's combine (larger score, then lower index) over the six
    steps gives every lane the plain argmax, ties to the lower index."""
    ctrls = _dpp_controls()
    rng = np.random.default_rng(0)
    for trial in range(200):
        v = rng.integers(0, 6, size=64).astype(float)   # many exact ties
        if trial % 3 == 0:
            v[rng.integers(0, 64, size=5)] = -np.inf
        val = v.copy()
        idx = np.arange(64)
        for step in range(6):
            p = _partners(step, ctrls)
            ov, oi = val[p], idx[p]
            take = (ov > val) | ((ov == val) & (oi < idx))
            val = np.where(take, ov, val)
            idx = np.where(take, oi, idx)
        best = int(np.argmax(v))   # first (lowest) index among the maxima
        assert (idx == best).all() and (val == v[best]).all()
