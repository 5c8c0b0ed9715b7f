"""Pins of the CPU oracle against what the pages and the mathematics fix:
page-printed integers, brute force, library routines, closed forms and
invariants.  Nothing here compares the oracle with itself or with the GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import special

import oracle
import workloads
from tests.helpers import (all_experts_dense, dense_gelu, dense_swiglu, rms,
                           scatter_dense_weights, widen)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _host(cfg, seed=0):
    return workloads.host_inputs(workloads.generate(cfg, seed=seed, device="cpu"))


def _small(cfg, T=24, D=40, F=24, Fs=None):
    return workloads.shrink(cfg, T=T, D=D, F=F, F_shared=Fs)


SMALL_CFGS = [
    workloads.GLAM_TINY_FP32,
    _small(workloads.GLAM_4K),
    _small(workloads.GLM45_PREFILL),
    _small(workloads.GLM5_ZIPF),
    _small(workloads.GLM45_DECODE, T=8),
]
SMALL_IDS = ["tiny_fp32", "glam_small", "glm45_small", "glm5_small", "decode_small"]


# ---------------------------------------------------------------- page counts

def test_glm5_shared_expert_parameter_count():
    g = json.load(open(os.path.join(GOLDEN, "glm5_shared_expert_params.json")))
    D, F = g["hidden_size"], g["shared_width"]
    assert D * F == g["gate_projection"] == g["up_projection"] == g["down_projection"]
    assert oracle.swiglu_params(D, F) == g["per_instance_total"] == 37_748_736
    assert oracle.swiglu_params(D, F) * g["moe_blocks"] == g["all_blocks_total"]
    p = oracle.layer_params(workloads.GLM5_ZIPF)
    assert p["shared"] == g["per_instance_total"]
    # the routers' correction-bias values over all MoE blocks fix M = 256
    assert p["correction_bias"] * g["moe_blocks"] == g["router_correction_bias_values_all_blocks"]
    assert workloads.GLM5_ZIPF.M == 256


def test_glm45_shapes_match_page():
    g = json.load(open(os.path.join(GOLDEN, "glm45_shapes.json")))
    c = workloads.GLM45_PREFILL
    assert (c.M, c.k, c.D, c.F, c.F_shared) == (
        g["routed_experts_355B"], g["active_per_token"], g["hidden_size_355B"],
        g["expert_width"], g["expert_width"] * g["shared_experts"])
    assert c.alpha == g["routed_scaling_factor_355B"] and c.eps == g["renorm_eps"]
    assert oracle.layer_params(c)["routed_per_expert"] == 3 * 5120 * 1536 == 23_592_960


# ------------------------------------------------------------------- router

def _logits_np(h, cfg):
    return widen(h["x"]) @ h["W_r"].astype(np.float64).T


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=SMALL_IDS)
def test_logits_match_numpy_matmul(cfg):
    h = _host(cfg)
    _, _, _, lg = oracle.route(cfg, h["x"], h["W_r"], h["bias"], want_logits=True)
    ref = _logits_np(h, cfg)
    assert np.allclose(lg, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def _brute_topk(sel, k):
    """Max-sum k-subset; among equal sums the lexicographically smallest
    sorted tuple (lower expert index wins an exact tie)."""
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(len(sel)), k):
        s = math.fsum(sel[i] for i in sub)
        if s > best_sum or (s == best_sum and sub < best):
            best, best_sum = sub, s
    return best


@pytest.mark.parametrize("scorer,M,k", [("softmax", 8, 2), ("softmax", 7, 3),
                                        ("sigmoid", 10, 3), ("sigmoid", 9, 4),
                                        ("sigmoid", 6, 6), ("softmax", 5, 1)])
def test_topk_bruteforce(scorer, M, k):
    base = workloads.GLAM_4K if scorer == "softmax" else workloads.GLM45_PREFILL
    cfg = base.replace(T=16, D=24, M=M, F=8, k=k, F_shared=0)
    h = _host(cfg, seed=3)
    # plant exact ties: duplicate router rows (and bias) give bit-equal scores
    h["W_r"][M - 1] = h["W_r"][0]
    if h["bias"] is not None:
        h["bias"][M - 1] = h["bias"][0]
    idx, _, gap = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    lg = _logits_np(h, cfg)
    for t in range(cfg.T):
        if scorer == "softmax":
            sel = lg[t]                      # softmax is strictly increasing in the logit
        else:
            sel = special.expit(lg[t]) + h["bias"].astype(np.float64)
        assert tuple(idx[t]) == _brute_topk(list(sel), k)
        score = special.softmax(lg[t]) if scorer == "softmax" else sel
        srt = np.sort(score)[::-1]
        if k < M:
            assert gap[t] == pytest.approx(srt[k - 1] - srt[k], abs=1e-12)
        if k == M:
            assert math.isinf(gap[t])


def _sel_np(h, cfg):
    lg = _logits_np(h, cfg)
    if cfg.scorer == "softmax":
        return lg
    return special.expit(lg) + (h["bias"].astype(np.float64) if h["bias"] is not None else 0.0)


@pytest.mark.parametrize("scorer,M,ng,tg,k", [("sigmoid", 12, 4, 2, 3), ("sigmoid", 12, 3, 1, 4),
                                               ("softmax", 10, 5, 3, 2), ("sigmoid", 8, 4, 4, 3)])
def test_group_limited_topk_bruteforce(scorer, M, ng, tg, k):
    """Groups of M/ng consecutive experts, a group's score the largest
    selection score in it, the tg best groups kept (numpy stable argsort),
    then the brute-force top-k among the kept groups' experts."""
    base = workloads.GLAM_4K if scorer == "softmax" else workloads.GLM45_PREFILL
    cfg = base.replace(T=20, D=24, M=M, F=8, k=k, F_shared=0, n_group=ng, topk_group=tg)
    h = _host(cfg, seed=5)
    idx, _, gap = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    sel = _sel_np(h, cfg)
    gs = M // ng
    for t in range(cfg.T):
        gmax = sel[t].reshape(ng, gs).max(axis=1)
        kept = np.argsort(-gmax, kind="stable")[:tg]
        cand = [e for e in range(M) if e // gs in set(kept.tolist())]
        sub = _brute_topk([sel[t][e] for e in cand], k)
        assert tuple(idx[t]) == tuple(sorted(cand[i] for i in sub))
        assert all(e // gs in set(kept.tolist()) for e in idx[t])
        # the gap covers the group boundary too
        if tg < ng:
            srt = np.sort(gmax)[::-1]
            assert gap[t] <= srt[tg - 1] - srt[tg] + 1e-12


@pytest.mark.parametrize("ng,tg", [(1, 1), (0, 0), (4, 4)])
def test_grouping_that_keeps_every_group_changes_nothing(ng, tg):
    cfg = _small(workloads.GLM45_PREFILL).replace(M=16, n_group=ng, topk_group=tg)
    h = _host(cfg, seed=6)
    idx_g, w_g, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    idx_0, w_0, _ = oracle.route(cfg.replace(n_group=0, topk_group=0), h["x"], h["W_r"], h["bias"])
    assert (idx_g == idx_0).all() and (w_g == w_0).all()


def test_group_limited_planted_example():
    """Group 0 holds the best single expert; groups 1 and 2 hold the next
    best ones.  One kept group and k = 2 must take expert 0 and the best
    other expert of group 0, not the overall second best."""
    cfg = workloads.GLM45_PREFILL.replace(T=1, D=6, M=6, F=8, k=2, F_shared=0, n_group=3,
                                          topk_group=1, renorm=True, alpha=1.0)
    x = np.zeros((1, 6), np.uint16)
    x[0, 0] = 0x3F80                               # bf16 1.0
    W_r = np.zeros((6, 6), np.float32)
    W_r[:, 0] = [3.0, -2.0, 2.5, 2.4, 2.3, 2.2]   # logits = first column
    bias = np.zeros(6, np.float32)
    idx, w, _ = oracle.route(cfg, x, W_r, bias)
    assert tuple(idx[0]) == (0, 1)
    # ungrouped, the two best experts are 0 and 2
    idx2, _, _ = oracle.route(cfg.replace(n_group=0, topk_group=0), x, W_r, bias)
    assert tuple(idx2[0]) == (0, 2)
    s = special.expit([3.0, -2.0])
    assert np.allclose(w[0], s / s.sum(), rtol=1e-15)


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=SMALL_IDS)
def test_exactly_k_distinct_ascending(cfg):
    h = _host(cfg)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    assert idx.shape == (cfg.T, cfg.k)
    assert ((idx >= 0) & (idx < cfg.M)).all()
    assert (np.diff(idx, axis=1) > 0).all()     # distinct and ascending


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=SMALL_IDS)
def test_renormalised_weights_sum_to_alpha(cfg):
    h = _host(cfg)
    _, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    assert np.abs(w.sum(axis=1) - cfg.alpha).max() <= 1e-12 * cfg.alpha
    assert (w > 0).all()


def test_alpha_zero_gives_zero_weights():
    cfg = _small(workloads.GLM45_PREFILL).replace(alpha=0.0)
    h = _host(cfg)
    _, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    assert (w == 0).all()


def test_softmax_top2_closed_form():
    # renormalised top-2 softmax: w_first = 1 / (1 + exp(l_second - l_first))
    cfg = _small(workloads.GLAM_4K, T=32)
    h = _host(cfg, seed=5)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    lg = _logits_np(h, cfg)
    for t in range(cfg.T):
        a, b = idx[t]
        assert w[t, 0] == pytest.approx(special.expit(lg[t, a] - lg[t, b]), abs=1e-13)
        assert w[t, 1] == pytest.approx(special.expit(lg[t, b] - lg[t, a]), abs=1e-13)


def test_softmax_weights_ignore_unselected_logits():
    # renormalised softmax weights depend only on the selected logits
    cfg = _small(workloads.GLAM_4K, T=16)
    h = _host(cfg, seed=6)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    Wr2 = h["W_r"].copy()
    unused = [e for e in range(cfg.M) if not (idx == e).any()]
    assert unused
    Wr2[unused] *= 0.25                    # shrinks only unselected logits toward 0 ...
    idx2, w2, _ = oracle.route(cfg, h["x"], Wr2, None)
    keep = (idx2 == idx).all(axis=1)       # ... where the selection stays the same
    assert keep.sum() >= cfg.T // 2
    assert np.allclose(w2[keep], w[keep], rtol=0, atol=1e-13)


def test_sigmoid_weights_use_unbiased_scores():
    cfg = _small(workloads.GLM45_PREFILL, T=16)
    h = _host(cfg, seed=7)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    # a uniform bias shift changes neither the selection nor the weights
    idx2, w2, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"] + np.float32(0.75))
    assert (idx2 == idx).all() and np.allclose(w2, w, rtol=0, atol=1e-14)
    # weight ratios equal ratios of the plain sigmoid scores (scipy expit)
    lg = _logits_np(h, cfg)
    for t in range(cfg.T):
        s = special.expit(lg[t, idx[t]])
        assert np.allclose(w[t] / w[t, 0], s / s[0], rtol=1e-12)
    # a bias large enough to force an expert in does not enter its weight
    forced = int(np.argmin(lg.mean(axis=0)))
    b3 = h["bias"].copy()
    b3[forced] = 50.0
    idx3, w3, _ = oracle.route(cfg, h["x"], h["W_r"], b3)
    for t in range(cfg.T):
        j = list(idx3[t]).index(forced)
        s = special.expit(lg[t, idx3[t]])
        assert w3[t, j] == pytest.approx(cfg.alpha * s[j] / s.sum(), rel=1e-12)


def test_eps_keeps_underflowing_scores_finite():
    # all logits -800: every sigmoid score is 0 in fp64, eps turns 0/0 into 0
    cfg = workloads.GLM45_PREFILL.replace(T=2, D=8, M=6, F=8, k=3, F_shared=0, dtype="f32")
    x = np.ones((2, 8), np.float32)
    W_r = np.full((6, 8), -100.0, np.float32)
    bias = np.zeros(6, np.float32)
    idx, w, _ = oracle.route(cfg, x, W_r, bias)
    assert (w == 0).all() and np.isfinite(w).all()
    assert (idx == np.array([0, 1, 2])).all()         # all tied: lowest indices
    # scores near 1e-20: eps is of the same size as each score, so every
    # weight is alpha * s / (3 s + 1e-20), about alpha / 4 (not alpha / 3)
    l0 = math.log(1e-20)
    W_r = np.full((6, 8), np.float32(l0 / 8), np.float32)
    idx, w, _ = oracle.route(cfg, x, W_r, bias)
    s = special.expit(float(np.float32(l0 / 8)) * 8)
    assert np.allclose(w, cfg.alpha * s / (3 * s + 1e-20), rtol=1e-9)
    assert np.allclose(w, cfg.alpha / 4, rtol=1e-3)


def test_no_renorm_weights_are_scaled_scores():
    cfg = _small(workloads.GLAM_4K, T=8).replace(renorm=False, alpha=1.5)
    h = _host(cfg)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], None)
    lg = _logits_np(h, cfg)
    p = special.softmax(lg, axis=1)
    assert np.allclose(w, 1.5 * np.take_along_axis(p, idx, axis=1), rtol=1e-12)


# ----------------------------------------------------------------- dispatch

def _random_routing(T, M, k, rng, sentinel_frac=0.0):
    idx = np.stack([np.sort(rng.choice(M, size=k, replace=False)) for _ in range(T)])
    if sentinel_frac:
        drop = rng.random(idx.shape) < sentinel_frac
        idx[drop] = M
    return idx.astype(np.int32)


@pytest.mark.parametrize("T,M,k,drop", [(1, 1, 1, 0.0), (37, 8, 2, 0.0), (300, 160, 8, 0.0),
                                        (64, 256, 8, 0.1), (50, 5, 5, 0.3), (0, 4, 2, 0.0)])
def test_dispatch_against_numpy_stable_sort(T, M, k, drop):
    rng = np.random.default_rng(T * 1000 + M)
    idx = _random_routing(T, M, k, rng, drop) if T else np.zeros((0, k), np.int32)
    d = oracle.dispatch(T, k, M, idx)
    flat = idx.reshape(-1)
    valid = flat < M
    assert (d["counts"] == np.bincount(flat[valid], minlength=M)).all()
    assert d["offsets"][0] == 0 and d["offsets"][-1] == valid.sum()
    assert (np.diff(d["offsets"]) == d["counts"]).all()
    order = np.argsort(flat, kind="stable")[: valid.sum()]   # library stable sort
    S = valid.sum()
    assert (d["sorted_slot"][:S] == order).all()
    assert (d["sorted_token"][:S] == order // k).all()
    assert (d["sorted_slot"][S:] == -1).all() and (d["sorted_token"][S:] == -1).all()
    # slot_row inverts sorted_slot; dropped slots map to -1
    assert (d["slot_row"][order] == np.arange(S)).all()
    assert (d["slot_row"][~valid] == -1).all()
    # tokens strictly increase inside every expert's rows
    for e in range(M):
        a, b = d["offsets"][e], d["offsets"][e + 1]
        assert (np.diff(d["sorted_token"][a:b]) > 0).all()


# ------------------------------------------------------------- layer output

@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=SMALL_IDS)
def test_sparse_equals_masked_dense(cfg):
    """y = sum over ALL experts of (weight, zero unless selected) * E_e(x)
    + E_sh(x), with every expert evaluated by numpy matmuls."""
    h = _host(cfg, seed=1)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], h["b1"], h["W2"], h["b2"],
                     h["Wsh_gu"], h["Wsh_dn"])
    E = all_experts_dense(cfg, h)
    ref = np.einsum("tm,tmd->td", scatter_dense_weights(cfg.T, cfg.M, idx, w), E)
    if cfg.F_shared:
        ref += dense_swiglu(widen(h["x"]), widen(h["Wsh_gu"]), widen(h["Wsh_dn"]))
    assert np.abs(y - ref).max() <= 1e-12 * max(1.0, rms(ref)) * 10


@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=SMALL_IDS)
def test_per_slot_outputs_and_shared_part(cfg):
    h = _host(cfg, seed=2)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    y, slots, sh = oracle.layer(cfg, h["x"], idx, w, h["W1"], h["b1"], h["W2"], h["b2"],
                                h["Wsh_gu"], h["Wsh_dn"], want_slots=True, want_shared=True)
    E = all_experts_dense(cfg, h)
    for t in range(cfg.T):
        for j in range(cfg.k):
            assert np.allclose(slots[t, j], w[t, j] * E[t, idx[t, j]], rtol=1e-11, atol=1e-12)
    assert np.allclose(y, slots.sum(axis=1) + sh, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("scorer,act", [("softmax", "gelu"), ("sigmoid", "swiglu"),
                                        ("softmax", "swiglu"), ("sigmoid", "gelu")])
def test_single_expert_collapses_to_dense_ffn(scorer, act):
    base = workloads.GLAM_TINY_FP32 if act == "gelu" else workloads.GLM45_PREFILL
    cfg = base.replace(T=12, D=32, M=1, F=20, k=1, F_shared=0, scorer=scorer, act=act,
                       alpha=2.5 if scorer == "sigmoid" else 1.0,
                       router_bias_std=0.3 if scorer == "sigmoid" else 0.0)
    h = _host(cfg, seed=4)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    assert (idx == 0).all()
    # s + 1e-20 rounds to s, so the weight is alpha up to the last bit
    assert np.allclose(w, cfg.alpha, rtol=4e-16, atol=0)
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], h["b1"], h["W2"], h["b2"])
    X = widen(h["x"])
    if act == "gelu":
        ref = dense_gelu(X, widen(h["W1"])[0], None if h["b1"] is None else widen(h["b1"])[0],
                         widen(h["W2"])[0], None if h["b2"] is None else widen(h["b2"])[0])
    else:
        ref = dense_swiglu(X, widen(h["W1"])[0], widen(h["W2"])[0])
    assert np.allclose(y, cfg.alpha * ref, rtol=1e-12, atol=1e-12)


def test_dense_prefix_layer_is_one_swiglu():
    # the dense prefix workload: one expert, top-1 softmax, alpha 1: the gate
    # weight is 1 exactly and the layer is a plain SwiGLU of the expert's width
    cfg = workloads.shrink(workloads.GLM45_DENSE, T=9, D=32, F=24)
    h = _host(cfg, seed=5)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    assert (idx == 0).all() and (w == 1.0).all()
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], None, h["W2"], None)
    ref = dense_swiglu(widen(h["x"]), widen(h["W1"])[0], widen(h["W2"])[0])
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_alpha_zero_leaves_plain_shared_swiglu():
    cfg = _small(workloads.GLM45_PREFILL).replace(alpha=0.0)
    h = _host(cfg, seed=8)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], None, h["W2"], None, h["Wsh_gu"], h["Wsh_dn"])
    ref = dense_swiglu(widen(h["x"]), widen(h["Wsh_gu"]), widen(h["Wsh_dn"]))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_two_shared_experts_equal_one_wider_swiglu():
    # N shared experts are one SwiGLU of width N * d_moe: stacking two width-F
    # experts (gates, then ups; downs side by side) equals summing them
    c1 = _small(workloads.GLM45_PREFILL, T=10, D=32, F=16, Fs=16)
    c2 = c1.replace(F_shared=32)
    ha, hb = _host(c1, seed=10), _host(c1, seed=11)
    Fs = 16
    gu = np.concatenate([ha["Wsh_gu"][:Fs], hb["Wsh_gu"][:Fs], ha["Wsh_gu"][Fs:],
                         hb["Wsh_gu"][Fs:]])
    dn = np.ascontiguousarray(np.concatenate([ha["Wsh_dn"], hb["Wsh_dn"]], axis=1))
    for t in range(c1.T):
        wide = oracle.shared(c2, ha["x"], t, gu, dn)
        two = oracle.shared(c1, ha["x"], t, ha["Wsh_gu"], ha["Wsh_dn"]) + \
            oracle.shared(c1, ha["x"], t, hb["Wsh_gu"], hb["Wsh_dn"])
        assert np.allclose(wide, two, rtol=1e-12, atol=1e-13)


def test_expert_relabelling_leaves_output_unchanged():
    cfg = _small(workloads.GLM45_PREFILL, T=12)
    h = _host(cfg, seed=12)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], None, h["W2"], None, h["Wsh_gu"], h["Wsh_dn"])
    perm = np.random.default_rng(0).permutation(cfg.M)      # new id of old expert e
    inv = np.argsort(perm)
    g = {k: v for k, v in h.items()}
    for key in ("W_r", "bias", "W1", "W2"):
        g[key] = np.ascontiguousarray(h[key][inv])
    idx2, w2, _ = oracle.route(cfg, g["x"], g["W_r"], g["bias"])
    assert (np.sort(inv[idx2], axis=1) == idx).all()
    y2 = oracle.layer(cfg, g["x"], idx2, w2, g["W1"], None, g["W2"], None, g["Wsh_gu"], g["Wsh_dn"])
    assert np.allclose(y2, y, rtol=1e-12, atol=1e-13)


def test_tokens_are_independent():
    cfg = _small(workloads.GLAM_4K, T=16)
    h = _host(cfg, seed=13)
    idx, w, y = oracle.forward(cfg, h, tokens=[5])
    h2 = dict(h)
    x2 = h["x"].copy()
    x2[np.arange(cfg.T) != 5] = x2[::-1][np.arange(cfg.T) != 5]
    h2["x"] = x2
    idx2, w2, y2 = oracle.forward(cfg, h2, tokens=[5])
    assert (idx == idx2).all() and (w == w2).all() and (y == y2).all()


def test_forward_matches_route_then_layer():
    cfg = _small(workloads.GLM5_ZIPF, T=10)
    h = _host(cfg, seed=14)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    y = oracle.layer(cfg, h["x"], idx, w, h["W1"], None, h["W2"], None, h["Wsh_gu"], h["Wsh_dn"])
    toks = np.array([7, 0, 3])
    i2, w2, y2 = oracle.forward(cfg, h, tokens=toks)
    assert (i2 == idx[toks]).all() and (w2 == w[toks]).all() and (y2 == y[toks]).all()


def test_dropped_slot_contributes_nothing():
    cfg = _small(workloads.GLM45_PREFILL, T=6)
    h = _host(cfg, seed=15)
    idx, w, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    idx_d = idx.copy()
    idx_d[:, 0] = cfg.M                       # sentinel: the extra one-hot class
    cfg0 = cfg.replace(F_shared=0)
    y_d, slots = oracle.layer(cfg0, h["x"], idx_d, w, h["W1"], None, h["W2"], None,
                              want_slots=True)
    assert (slots[:, 0] == 0).all()
    E = all_experts_dense(cfg0, h)
    ref = sum(w[:, j:j + 1] * E[np.arange(cfg.T), idx[:, j]] for j in range(1, cfg.k))
    assert np.allclose(y_d, ref, rtol=1e-12, atol=1e-13)


def test_gelu_is_the_erf_form():
    # tanh-approximate GELU differs by ~1e-3 near |z| ~ 2; the oracle must
    # reproduce scipy's erf-based Phi, not the approximation
    cfg = workloads.GLAM_TINY_FP32.replace(T=1, D=1, M=1, F=1, k=1, ffn_bias_std=0.0)
    for z in (-3.0, -2.0, -0.5, 0.0, 0.7, 2.0):
        h = {"x": np.array([[1.0]], np.float32), "W1": np.array([[[z]]], np.float32),
             "W2": np.array([[[1.0]]], np.float32)}
        y = oracle.expert(cfg, h["x"], 0, 0, h["W1"], None, h["W2"], None)
        zf = float(np.float32(z))            # the weight is stored in fp32
        assert y[0] == pytest.approx(zf * special.ndtr(zf), abs=1e-15)


# ------------------------------------------------------------- the gradient
#
# The backward is pinned to the forward definition by central finite
# differences of L = sum(dy * y): inputs are multiples of 2^-8 and the step
# is 2^-12, so x +- h is exact in fp32 storage, the forward runs in fp64 and
# the difference quotient's truncation error (~h^2) is ~1e-7.  Entries whose
# perturbation changes the top-k selection are skipped (the selection is
# piecewise constant and passes no gradient).

_FD_H = 2.0 ** -12


def _q(rng, shape, std):
    """fp32 normal draws rounded to multiples of 2^-8 (exact in fp32)."""
    return (np.round(rng.normal(0.0, std, shape) * 256.0) / 256.0).astype(np.float32)


def _fd_case(scorer, act, M, k, T=4, D=6, F=4, Fs=0, renorm=True, alpha=1.0, biases=False,
             n_group=0, topk_group=0, seed=0):
    cfg = workloads.MoEConfig(name="fd", T=T, D=D, M=M, F=F, k=k, scorer=scorer, act=act,
                              F_shared=Fs, dtype="f32", renorm=renorm, alpha=alpha,
                              n_group=n_group, topk_group=topk_group)
    rng = np.random.default_rng(seed)
    G = 2 if act == "swiglu" else 1
    h = {"x": _q(rng, (T, D), 1.0), "W_r": _q(rng, (M, D), 1.0),
         "bias": _q(rng, (M,), 0.3) if scorer == "sigmoid" else None,
         "W1": _q(rng, (M, G * F, D), 0.5), "W2": _q(rng, (M, D, F), 0.5),
         "b1": _q(rng, (M, F), 0.3) if biases else None,
         "b2": _q(rng, (M, D), 0.3) if biases else None,
         "Wsh_gu": _q(rng, (2 * Fs, D), 0.5) if Fs else None,
         "Wsh_dn": _q(rng, (D, Fs), 0.5) if Fs else None}
    dy = rng.normal(0.0, 1.0, (T, D))
    return cfg, h, dy


def _loss(cfg, h, dy):
    idx, _, y = oracle.forward(cfg, h)
    return float((dy * y).sum()), idx


FD_CASES = {
    "swiglu_sigmoid_shared": dict(scorer="sigmoid", act="swiglu", M=5, k=2, Fs=3, alpha=2.5),
    "gelu_softmax_biases": dict(scorer="softmax", act="gelu", M=4, k=2, biases=True),
    "swiglu_sigmoid_norenorm": dict(scorer="sigmoid", act="swiglu", M=4, k=1, renorm=False,
                                    alpha=1.5),
    "gelu_softmax_norenorm_k3": dict(scorer="softmax", act="gelu", M=5, k=3, renorm=False),
    "swiglu_sigmoid_groups": dict(scorer="sigmoid", act="swiglu", M=6, k=2, n_group=3,
                                  topk_group=2, Fs=2),
}


@pytest.mark.parametrize("name", list(FD_CASES))
def test_backward_matches_finite_differences(name):
    cfg, h, dy = _fd_case(**FD_CASES[name])
    g = oracle.backward(cfg, h, dy)
    _, idx0 = _loss(cfg, h, dy)
    names = [("x", "dx"), ("W_r", "dW_r"), ("W1", "dW1"), ("W2", "dW2"), ("b1", "db1"),
             ("b2", "db2"), ("Wsh_gu", "dWsh_gu"), ("Wsh_dn", "dWsh_dn")]
    checked = skipped = 0
    for pname, gname in names:
        if h.get(pname) is None:
            assert gname not in g
            continue
        a = h[pname]
        flat = a.reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            flat[i] = v + np.float32(_FD_H)
            lp, ip = _loss(cfg, h, dy)
            flat[i] = v - np.float32(_FD_H)
            lm, im = _loss(cfg, h, dy)
            flat[i] = v
            if not (np.array_equal(ip, idx0) and np.array_equal(im, idx0)):
                skipped += 1
                continue
            fd = (lp - lm) / (2 * _FD_H)
            an = g[gname].reshape(-1)[i]
            assert abs(fd - an) <= 2e-5 * (1.0 + abs(fd)), (pname, i, fd, an)
            checked += 1
    assert checked > 20 * skipped


def test_backward_load_statistics():
    cfg, h, dy = _fd_case(scorer="sigmoid", act="swiglu", M=6, k=2, T=9, Fs=2)
    g = oracle.backward(cfg, h, dy)
    idx, _, _, logits = oracle.route(cfg, h["x"], h["W_r"], h["bias"], want_logits=True)
    assert (g["load_count"] == np.bincount(idx.reshape(-1), minlength=cfg.M)).all()
    assert g["load_count"].sum() == cfg.T * cfg.k
    assert np.allclose(g["load_score"], special.expit(logits).sum(axis=0), rtol=1e-13)
    cfg, h, dy = _fd_case(scorer="softmax", act="gelu", M=5, k=2, T=7)
    g = oracle.backward(cfg, h, dy)
    _, _, _, logits = oracle.route(cfg, h["x"], h["W_r"], None, want_logits=True)
    assert np.allclose(g["load_score"], special.softmax(logits, axis=1).sum(axis=0), rtol=1e-13)
    assert np.isclose(g["load_score"].sum(), cfg.T, rtol=1e-13)


def test_backward_alpha_zero_is_shared_swiglu_only():
    """alpha = 0 zeroes every routed weight: the routed experts and the
    router receive no gradient, and dx is a plain SwiGLU's input gradient
    (numpy matmuls)."""
    cfg, h, dy = _fd_case(scorer="sigmoid", act="swiglu", M=5, k=2, Fs=3, alpha=0.0, T=5)
    g = oracle.backward(cfg, h, dy)
    for key in ("dW1", "dW2", "dW_r"):
        assert not g[key].any(), key
    x = h["x"].astype(np.float64)
    Wg, Wu = h["Wsh_gu"][:3].astype(np.float64), h["Wsh_gu"][3:].astype(np.float64)
    Wd = h["Wsh_dn"].astype(np.float64)
    a, b = x @ Wg.T, x @ Wu.T
    sg = special.expit(a)
    dh = dy @ Wd
    da = dh * b * sg * (1 + a * (1 - sg))
    db = dh * a * sg
    assert np.allclose(g["dx"], da @ Wg + db @ Wu, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dWsh_dn"], dy.T @ (a * sg * b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_backward_expert_selection_is_a_slice(act):
    """Keeping only some experts' weight gradients (for layers too large to
    hold all M in fp64) returns exactly those experts' slices of the full
    gradient, in list order, and leaves every other output unchanged."""
    cfg, h, dy = _fd_case(scorer="sigmoid" if act == "swiglu" else "softmax", act=act, M=6, k=2,
                          T=11, Fs=2 if act == "swiglu" else 0, biases=act == "gelu")
    full = oracle.backward(cfg, h, dy)
    pick = [4, 0, 3]
    part = oracle.backward(cfg, h, dy, experts=pick)
    for key in full:
        if key in ("dW1", "dW2", "db1", "db2"):
            assert part[key].shape == (len(pick),) + full[key].shape[1:]
            assert np.array_equal(part[key], full[key][pick]), key
        else:
            assert np.array_equal(part[key], full[key]), key
