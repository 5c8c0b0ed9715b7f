"""Exact ties on the GPU router: the lower expert index wins.

Router rows (and correction biases) are planted in groups of three
identical copies, so three experts have bit-identical selection scores on
every token, and k is chosen so that the top-k boundary splits such a
group (k = 8 = 3 + 3 + 2 for GLM-4.5-shaped routing, k = 2 for GLaM-shaped
routing).  The GLaM study note's TopK does not say which of equal scores
wins; the reading here is the lower expert index (as the oracle does).  On
these tokens the oracle's boundary gap is exactly zero, so the usual
1e-6 tie exemption would excuse any choice: here none is allowed, the GPU's
indices must equal the oracle's bit for bit.  Both router paths run: the
fp64 dot-product router (T <= 256) and the split-plane MFMA router.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import check_dispatch_props, gpu_permute, new_layer, run_route, to_np

pytestmark = pytest.mark.gpu

S = workloads.shrink
CASES = {
    "sigmoid_gemm_router": S(workloads.GLM45_PREFILL, T=600, D=264, F=64, F_shared=0),
    "sigmoid_small_router": S(workloads.GLM45_PREFILL, T=64, D=264, F=64, F_shared=0),
    "softmax_gemm_router": S(workloads.GLAM_4K, T=700, D=264, F=64),
    "softmax_small_router": S(workloads.GLAM_4K, T=200, D=264, F=64),
    "grouped_sigmoid": S(workloads.GLM45_PREFILL, T=600, D=264, F=64,
                         F_shared=0).replace(n_group=8, topk_group=4),
}


def _plant_triples(t, M):
    """Rows 3q, 3q+1, 3q+2 of W_r (and of the bias) become copies of row 3q."""
    src = torch.arange(M, device=t["W_r"].device) // 3 * 3
    t["W_r"] = t["W_r"][src].contiguous()
    if t.get("bias") is not None:
        t["bias"] = t["bias"][src].contiguous()
    return t


@pytest.mark.parametrize("name", list(CASES))
def test_planted_exact_ties_lower_index_wins(name):
    cfg = CASES[name]
    t = _plant_triples(workloads.generate(cfg, seed=5, device="cuda"), cfg.M)
    h = workloads.host_inputs(t)
    L = new_layer(cfg)
    idx_g, w_g = run_route(L, L.desc, t)
    torch.cuda.synchronize()
    idx_gh = to_np(idx_g).reshape(cfg.T, cfg.k)
    idx_o, w_o, gap_o, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"], want_sel=True)
    tied = gap_o == 0.0
    # the plant works: most tokens have an exact tie at the top-k boundary
    assert tied.mean() > 0.9, f"only {tied.mean():.2f} of tokens tie exactly"
    assert np.array_equal(idx_gh, idx_o), (
        f"tie rule broken on tokens {np.nonzero((idx_gh != idx_o).any(axis=1))[0][:8]}")
    err = np.abs(to_np(w_g).reshape(cfg.T, cfg.k).astype(np.float64) - w_o).max()
    assert err <= 1e-5 * cfg.alpha
    # the dispatch of these indices is then bit-exact as well
    pg = {k: to_np(v) for k, v in gpu_permute(L, L.desc, idx_g).items()}
    check_dispatch_props(cfg, idx_gh, pg)
    disp_o = oracle.dispatch(cfg.T, cfg.k, cfg.M, idx_o)
    for key in disp_o:
        assert (pg[key] == disp_o[key]).all(), key
