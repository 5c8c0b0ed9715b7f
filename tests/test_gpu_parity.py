"""GPU parity: every stage of the HIP path against the CPU oracle on the
same seeded inputs, through the C ABI.

Integers (top-k indices, counts, offsets, permutation) are bit-exact except
tie-exempt tokens; the layer output is within max|err| <= 2e-2 * RMS(oracle)
for bf16 layers (fp32 output) and 1e-4 * RMS for the fp32 layer, and a bf16
output is bitwise the rounding of that fp32 result.  Sizes span several
128-row tiles with ragged row, column and reduction tails.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from sparse_mixture_experts_15_amd import binding as B
from tests.gpu_util import (COMPACT_REL, PLAIN_MIN_WIDTH, assert_rounded_from,
                            check_dispatch_props, check_float, check_route, check_tie_exempt,
                            dev_i32, forward,
                            gpu_permute, new_layer, rounding_bounds, run_route, tiled_weights,
                            to_np, uses_compact_rows, y_plain)

pytestmark = pytest.mark.gpu

S = workloads.shrink
PARITY = {
    # the tiny fp32 layer at its own size
    "tiny_fp32": workloads.GLAM_TINY_FP32,
    # GLaM-shaped routing (64 experts, softmax top-2) at small D/F; ragged K and N tails
    "glam_small": S(workloads.GLAM_4K, T=700, D=264, F=200),
    # few experts so each spans several 128-row tiles with a ragged last tile
    "glam_tiles": S(workloads.GLAM_4K, T=700, D=264, F=200).replace(M=4),
    # GLM-4.5 routing (160 experts, biased sigmoid top-8, alpha 2.5) + shared expert
    "glm45_small": S(workloads.GLM45_PREFILL, T=333, D=264, F=200, F_shared=136),
    # GLM-5 Zipf routing (256 experts) + shared expert
    "glm5_small": S(workloads.GLM5_ZIPF, T=520, D=200, F=72, F_shared=136),
    # decode shape: 64 tokens over 160 experts
    "decode_small": S(workloads.GLM45_DECODE, T=64, D=264, F=200, F_shared=200),
    # mid-size widths (>= 512), where the plain 2e-2 * RMS bar is asserted too
    "glm45_mid": S(workloads.GLM45_PREFILL, T=256, D=1024, F=512, F_shared=512),
    "glam_mid": S(workloads.GLAM_4K, T=512, D=512, F=1024).replace(M=8),
    # ~200 rows per expert under Zipf routing: one 256-row tile per expert
    "glm5_rows": S(workloads.GLM5_ZIPF, T=600, D=320, F=136, F_shared=136).replace(M=24),
    # more than 1024 tokens: the three-kernel dispatch (smaller batches take
    # the one-workgroup dispatch)
    "glm45_t1500": S(workloads.GLM45_PREFILL, T=1500, D=64, F=48, F_shared=48),
    # group-limited routing: 8 groups of 20 experts, the best 4 kept
    "glm45_grouped": S(workloads.GLM45_PREFILL, T=333, D=264, F=200,
                       F_shared=136).replace(n_group=8, topk_group=4),
    # softmax scorer with 8 groups of 8 experts, the best 2 kept
    "glam_grouped": S(workloads.GLAM_4K, T=700, D=264, F=200).replace(n_group=8, topk_group=2),
    # fp32 SwiGLU layer with a shared expert (fp32 path of every epilogue)
    "fp32_swiglu": S(workloads.GLM45_PREFILL, T=150, D=96, F=40, F_shared=48).replace(dtype="f32"),
}


def _stage_parity(cfg, seed=0, tiled=False, **tuning):
    """Every stage against the oracle.  Float stages are checked on fp32
    outputs (the computation before the output's final rounding) at the plain
    bar; for a bf16 layer the bf16 output is then checked bitwise to be the
    round-to-nearest-even of the fp32 result, so the two together pin it."""
    t = workloads.generate(cfg, seed=seed, device="cuda")
    h = workloads.host_inputs(t)
    bf = cfg.dtype == "bf16"
    layout = "tiled" if tiled else "rows"
    L = new_layer(cfg, out_dtype="f32", weight_layout=layout, **tuning)
    d = L.desc
    if tiled:   # the GPU gets the tiled copies; the oracle keeps the row-major h
        t = tiled_weights(L, t)
    T, k, M, D = cfg.T, cfg.k, cfg.M, cfg.D

    # router
    idx_g, w_g = run_route(L, d, t)
    idx_o, w_o, gap_o, logits_o, sel_o = oracle.route(cfg, h["x"], h["W_r"], h["bias"],
                                                      want_logits=True, want_sel=True)
    idx_gh = to_np(idx_g).reshape(T, k)
    w_gh = to_np(w_g)
    mism = check_route(cfg, idx_gh, w_gh, idx_o, w_o, gap_o, sel_o)

    # dispatch of the GPU's own indices
    pg = {kk: to_np(v) for kk, v in gpu_permute(L, d, idx_g).items()}
    check_dispatch_props(cfg, idx_gh, pg)
    disp_o = oracle.dispatch(T, k, M, idx_o)
    if not mism.any():
        for key in disp_o:
            assert (pg[key] == disp_o[key]).all(), key

    # expert FFNs on the oracle's dispatch and weights
    y_o, slots_o, sh_o = oracle.layer(cfg, h["x"], idx_o, w_o, h["W1"], h["b1"], h["W2"],
                                      h["b2"], h["Wsh_gu"], h["Wsh_dn"], want_slots=True,
                                      want_shared=True)
    dev = {kk: torch.from_numpy(v).cuda() for kk, v in disp_o.items()}
    w_dev = torch.from_numpy(w_o.astype(np.float32).reshape(-1)).cuda()
    O = torch.zeros(T * k * D, dtype=torch.float32, device="cuda")
    B.moe_expert_ffn(L.handle, d, t["x"], dev["sorted_token"], dev["sorted_slot"],
                     dev["offsets"], w_dev, t["W1"], t["b1"], t["W2"], t["b2"], O, L.ws)
    nrow = int(disp_o["offsets"][-1])
    ss = disp_o["sorted_slot"][:nrow]
    O_exp = slots_o.reshape(T * k, D)[ss]
    O_got = to_np(O).reshape(T * k, D)[:nrow]
    bnd, bsh = rounding_bounds(cfg, h, idx_o, w_o)
    check_float(cfg, O_got, O_exp, "expert rows O", bound=bnd.reshape(T * k, D)[ss],
                plain=cfg.F >= PLAIN_MIN_WIDTH)

    # shared expert
    Ysh = None
    if cfg.F_shared:
        Ysh = torch.zeros(T * D, dtype=torch.float32, device="cuda")
        B.moe_shared_expert(L.handle, d, t["x"], t["Wsh_gu"], t["Wsh_dn"], Ysh, L.ws)
        check_float(cfg, to_np(Ysh).reshape(T, D), sh_o, "shared expert Ysh", bound=bsh,
                    plain=cfg.F_shared >= PLAIN_MIN_WIDTH)

    # combine, fp32 output: the plain bar (narrow reduced shapes: the bound)
    y = torch.zeros(T * D, dtype=torch.float32, device="cuda")
    B.moe_combine(L.handle, d, O, dev["slot_row"], Ysh, y)
    ybnd = bnd.sum(axis=1) + (bsh if bsh is not None else 0.0)
    wide = y_plain(cfg)
    check_float(cfg, to_np(y).reshape(T, D), y_o, "combine y", bound=ybnd, plain=wide)

    # whole layer, shared expert on a second stream, fp32 output (its expert
    # and shared rows compact for bf16 layers: up to 2^-11 |O| more per slot
    # and 2^-11 |Ysh| for the shared row)
    aux = torch.cuda.Stream()
    y_f = forward(L, t, aux=aux)
    torch.cuda.synchronize()
    keep = ~mism
    fbnd = ybnd
    if uses_compact_rows(cfg):
        fbnd = ybnd + COMPACT_REL * np.abs(slots_o).sum(axis=1)
        if sh_o is not None:
            fbnd = fbnd + COMPACT_REL * np.abs(sh_o)
    check_float(cfg, to_np(y_f).reshape(T, D)[keep], y_o[keep], "forward y", bound=fbnd[keep],
                plain=wide)
    # tie-exempt tokens: the oracle on the GPU's own selection
    check_tie_exempt(cfg, h, mism, idx_gh, w_gh, to_np(y_f).reshape(T, D), logits_o, idx_o, w_o,
                     float(np.sqrt(np.mean(y_o * y_o))), "forward y", plain=wide,
                     compact=uses_compact_rows(cfg))
    if not bf:
        return L, t, y_f

    # the same layer with bf16 output: bitwise the rounding of the fp32 y
    Lb = new_layer(cfg, out_dtype="bf16", weight_layout=layout, **tuning)
    yb = torch.zeros(T * D, dtype=torch.bfloat16, device="cuda")
    B.moe_combine(Lb.handle, Lb.desc, O, dev["slot_row"], Ysh, yb)
    y_fb = forward(Lb, t, aux=aux)
    torch.cuda.synchronize()
    assert_rounded_from(yb, y, "combine y (bf16)")
    assert_rounded_from(y_fb, y_f, "forward y (bf16)")
    return Lb, t, y_fb


@pytest.mark.parametrize("name", list(PARITY))
def test_stage_parity(name):
    _stage_parity(PARITY[name])


@pytest.mark.parametrize("name", ["glam_small", "glam_tiles", "glm45_small", "glm5_small",
                                  "decode_small", "glm45_mid", "glam_mid", "glm5_rows"])
def test_stage_parity_tiled_weights(name):
    """Every GEMM reading the tiled weight copies (moe_tile_weights)."""
    _stage_parity(PARITY[name], tiled=True)


@pytest.mark.parametrize("name", ["glm45_small", "tiny_fp32", "glam_tiles", "decode_small"])
def test_forward_deterministic_and_stream_invariant(name):
    cfg = PARITY[name]
    t = workloads.generate(cfg, seed=1, device="cuda")
    L = new_layer(cfg)
    aux = torch.cuda.Stream()
    y1 = forward(L, t, aux=aux)
    y2 = forward(L, t, aux=aux)
    y3 = forward(L, t, aux=None)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1,
                       y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2)
    assert torch.equal(y1, y3)
    # the stage calls chained on the GPU's own outputs (fp32 expert rows)
    # reproduce the forward with fp32 rows bitwise
    L = new_layer(cfg, rows_format="fp32")
    y1 = forward(L, t, aux=aux)
    d = L.desc
    idx, w = run_route(L, d, t)
    p = gpu_permute(L, d, idx)
    O = torch.empty(cfg.T * cfg.k * cfg.D, dtype=torch.float32, device="cuda")
    B.moe_expert_ffn(L.handle, d, t["x"], p["sorted_token"], p["sorted_slot"], p["offsets"],
                     w, t["W1"], t["b1"], t["W2"], t["b2"], O, L.ws)
    Ysh = None
    if cfg.F_shared:
        Ysh = torch.empty(cfg.T * cfg.D, dtype=torch.float32, device="cuda")
        B.moe_shared_expert(L.handle, d, t["x"], t["Wsh_gu"], t["Wsh_dn"], Ysh, L.ws)
    y4 = torch.empty_like(y1)
    B.moe_combine(L.handle, d, O, p["slot_row"], Ysh, y4)
    torch.cuda.synchronize()
    assert torch.equal(y1, y4)


def _row_sums(cfg, L, t, On, sr):
    """Per token: the sum of |row| over the compact rows the combine adds
    (its routed rows On via slot_row, and its shared row, computed by the
    shared-expert stage in fp32) and the sum of those rows' largest
    magnitudes."""
    tot = np.zeros((cfg.T, cfg.D))
    rowmax = np.zeros(cfg.T)
    for j in range(cfg.k):
        ok = sr[:, j] >= 0
        tot[ok] += On[sr[ok, j]]
        rowmax[ok] += On[sr[ok, j]].max(axis=1)
    if cfg.F_shared:
        Ysh = torch.zeros(cfg.T * cfg.D, dtype=torch.float32, device="cuda")
        B.moe_shared_expert(L.handle, L.desc, t["x"], t["Wsh_gu"], t["Wsh_dn"], Ysh, L.ws)
        torch.cuda.synchronize()
        Ya = np.abs(to_np(Ysh).reshape(cfg.T, cfg.D).astype(np.float64))
        tot += Ya
        rowmax += Ya.max(axis=1)
    return tot, rowmax


@pytest.mark.parametrize("name", ["glm45_small", "glam_tiles", "glm45_mid", "glam_mid",
                                  "glm5_rows", "glm5_small"])
def test_compact_rows_within_fp16_rounding(name):
    """The forward with compact expert rows against the same forward with
    fp32 rows: per output element the difference stays within the compact
    format's rounding of every routed and shared row it sums, 2^-11 |O_j| (relative
    error of one fp16 rounding after an exact power-of-two scale), plus the
    two fp32 sums' own rounding and fp16 underflow of values far below
    their group's largest."""
    cfg = PARITY[name]
    t = workloads.generate(cfg, seed=3, device="cuda")
    aux = torch.cuda.Stream()
    # a separate shared expert: a merged one keeps fp32 rows
    L32 = new_layer(cfg, out_dtype="f32", rows_format="fp32", shared_mode="separate")
    Lc = new_layer(cfg, out_dtype="f32", rows_format="compact", shared_mode="separate")
    y32 = forward(L32, t, aux=aux)
    yc = forward(Lc, t, aux=aux)
    d = L32.desc
    idx, w = run_route(L32, d, t)
    p = gpu_permute(L32, d, idx)
    S = cfg.T * cfg.k
    O = torch.zeros(S * cfg.D, dtype=torch.float32, device="cuda")
    B.moe_expert_ffn(L32.handle, d, t["x"], p["sorted_token"], p["sorted_slot"], p["offsets"],
                     w, t["W1"], t["b1"], t["W2"], t["b2"], O, L32.ws)
    torch.cuda.synchronize()
    On = np.abs(to_np(O).reshape(S, cfg.D).astype(np.float64))
    sr = to_np(p["slot_row"]).reshape(cfg.T, cfg.k)
    tot, rowmax = _row_sums(cfg, L32, t, On, sr)
    a32 = to_np(y32).reshape(cfg.T, cfg.D).astype(np.float64)
    ac = to_np(yc).reshape(cfg.T, cfg.D).astype(np.float64)
    allow = (COMPACT_REL * tot + 2 * (cfg.k + 1) * 2.0 ** -24 * (tot + np.abs(a32))
             + 2.0 ** -38 * rowmax[:, None])
    err = np.abs(ac - a32)
    assert np.isfinite(ac).all()
    worst = float((err - allow).max())
    assert worst <= 0.0, f"compact rows differ beyond their rounding by {worst:.3e}"
    # and they are not simply fp32: some element moved
    assert (err > 0).any()


def test_compact_rows_extreme_magnitudes():
    """Compact rows across the exponent range: experts whose down weights
    are scaled by 2^40 or 2^-40 (exact in bf16) or zeroed give expert rows
    from ~1e11 to ~1e-13 and all-zero scale groups in one layer; the
    compact forward stays within its rounding of the fp32-rows forward."""
    cfg = PARITY["glm45_small"]
    t = workloads.generate(cfg, seed=5, device="cuda")
    W2 = t["W2"].clone().view(cfg.M, cfg.D, cfg.F)
    e = torch.arange(cfg.M, device="cuda")
    scale = torch.where(e % 3 == 0, 2.0 ** 40, torch.where(e % 3 == 1, 2.0 ** -40, 1.0))
    scale = torch.where(e % 7 == 0, 0.0, scale)
    t["W2"] = (W2.float() * scale[:, None, None]).to(torch.bfloat16).reshape(-1).contiguous()
    aux = torch.cuda.Stream()
    outs = {}
    for rf in ("fp32", "compact"):
        L = new_layer(cfg, out_dtype="f32", rows_format=rf, shared_mode="separate")
        outs[rf] = (L, forward(L, t, aux=aux))
    L32 = outs["fp32"][0]
    d = L32.desc
    idx, w = run_route(L32, d, t)
    p = gpu_permute(L32, d, idx)
    S = cfg.T * cfg.k
    O = torch.zeros(S * cfg.D, dtype=torch.float32, device="cuda")
    B.moe_expert_ffn(L32.handle, d, t["x"], p["sorted_token"], p["sorted_slot"], p["offsets"],
                     w, t["W1"], t["b1"], t["W2"], t["b2"], O, L32.ws)
    torch.cuda.synchronize()
    On = np.abs(to_np(O).reshape(S, cfg.D).astype(np.float64))
    assert On.max() > 1e9 and On[On > 0].min() < 1e-9, "the layer does not span the range"
    sr = to_np(p["slot_row"]).reshape(cfg.T, cfg.k)
    tot, rowmax = _row_sums(cfg, L32, t, On, sr)
    a32 = to_np(outs["fp32"][1]).reshape(cfg.T, cfg.D).astype(np.float64)
    ac = to_np(outs["compact"][1]).reshape(cfg.T, cfg.D).astype(np.float64)
    assert np.isfinite(ac).all()
    allow = (COMPACT_REL * tot + 2 * (cfg.k + 1) * 2.0 ** -24 * (tot + np.abs(a32))
             + 2.0 ** -38 * rowmax[:, None])
    worst = float((np.abs(ac - a32) - allow).max())
    assert worst <= 0.0, f"compact rows differ beyond their rounding by {worst:.3e}"


# ------------------------------------------------------------------ edges

# Every bf16 tile height on every GEMM (the library picks one per shape; the
# descriptor's tile_rows forces the others), covering both activations, the
# grouped and dense GEMMs and every epilogue, and every workgroup order.
@pytest.mark.parametrize("bm", [64, 128, 160, 256])
@pytest.mark.parametrize("name", ["glam_tiles", "glm45_small", "glam_mid"])
def test_tile_heights(name, bm):
    _stage_parity(PARITY[name], tile_rows=bm)


# The same on the tiled weight copies: 64-row tiles read half of each 256-row
# weight block.
@pytest.mark.parametrize("bm", [64, 128, 160, 256])
@pytest.mark.parametrize("name", ["glam_tiles", "glm45_small"])
def test_tile_heights_tiled(name, bm):
    _stage_parity(PARITY[name], tiled=True, tile_rows=bm)


@pytest.mark.parametrize("order", ["xcd_groups", "hardware", "xcd_slices"])
@pytest.mark.parametrize("name", ["glm45_small", "glm5_rows"])
def test_tile_orders(name, order):
    _stage_parity(PARITY[name], tile_order=order, group_m=2)


EDGE = {
    "single_token": S(workloads.GLM45_PREFILL, T=1, D=64, F=48, F_shared=48),
    "k_equals_m": S(workloads.GLM45_PREFILL, T=40, D=64, F=48, F_shared=0).replace(M=6, k=6),
    "one_expert_top1": S(workloads.GLAM_4K, T=130, D=72, F=56).replace(M=1, k=1),
    "dense_prefix_swiglu": S(workloads.GLM45_DENSE, T=300, D=96, F=200),
    "switch_top1": S(workloads.GLAM_4K, T=300, D=128, F=64).replace(M=16, k=1),
    "alpha_zero": S(workloads.GLM45_PREFILL, T=50, D=64, F=48, F_shared=32).replace(alpha=0.0),
    "no_renorm_softmax": S(workloads.GLAM_4K, T=90, D=64, F=40).replace(renorm=False, alpha=1.5),
    "no_renorm_sigmoid": S(workloads.GLM45_PREFILL, T=90, D=64, F=40, F_shared=0).replace(renorm=False),
    "max_k16": S(workloads.GLM5_ZIPF, T=70, D=64, F=32, F_shared=0).replace(k=16),
    "many_experts_1024": S(workloads.GLM45_PREFILL, T=200, D=64, F=16, F_shared=0).replace(M=1024, k=4),
    "k_tail_8": S(workloads.GLM45_PREFILL, T=100, D=8, F=8, F_shared=8),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_parity(name):
    _stage_parity(EDGE[name])


def test_empty_batch_is_noop():
    cfg = S(workloads.GLM45_PREFILL, T=0, D=64, F=48, F_shared=48)
    t = workloads.generate(cfg.replace(T=4), seed=0, device="cuda")
    L = new_layer(cfg)
    y = torch.full((4 * 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    B.moe_forward(L.handle, L.desc, t["x"][:0], t["W_r"], t["bias"], t["W1"], None, t["W2"],
                  None, t["Wsh_gu"], t["Wsh_dn"], y[:0], L.ws)
    torch.cuda.synchronize()
    assert (y.float() == 7.0).all()


# T = 260 takes the one-workgroup dispatch, T = 1500 the three-kernel one.
@pytest.mark.parametrize("T", [260, 1500])
def test_dropped_slots_in_permute_and_combine(T):
    cfg = S(workloads.GLM45_PREFILL, T=T, D=64, F=48, F_shared=0)
    t = workloads.generate(cfg, seed=3, device="cuda")
    h = workloads.host_inputs(t)
    L = new_layer(cfg)
    idx_o, w_o, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    idx_d = idx_o.copy()
    rng = np.random.default_rng(0)
    drop = rng.random(idx_d.shape) < 0.2
    idx_d[drop] = cfg.M                                # the extra one-hot class
    pg = {kk: to_np(v) for kk, v in
          gpu_permute(L, L.desc, torch.from_numpy(idx_d.reshape(-1)).cuda()).items()}
    disp = oracle.dispatch(cfg.T, cfg.k, cfg.M, idx_d)
    for key in disp:
        assert (pg[key] == disp[key]).all(), key
    # combine skips dropped slots: the fp32 sum in slot order is an exact
    # sequence of IEEE additions, reproduced bitwise by numpy's float32 adds
    # in the same order; the bf16 output is its rounding
    O = torch.randn(cfg.T * cfg.k * cfg.D, device="cuda")
    sr_dev = torch.from_numpy(disp["slot_row"]).cuda()
    Lf = new_layer(cfg, out_dtype="f32")
    y32 = torch.empty(cfg.T * cfg.D, dtype=torch.float32, device="cuda")
    B.moe_combine(Lf.handle, Lf.desc, O, sr_dev, None, y32)
    y = torch.empty(cfg.T * cfg.D, dtype=torch.bfloat16, device="cuda")
    B.moe_combine(L.handle, L.desc, O, sr_dev, None, y)
    On = to_np(O).reshape(-1, cfg.D)
    sr = disp["slot_row"].reshape(cfg.T, cfg.k)
    ref = np.zeros((cfg.T, cfg.D), np.float32)
    for tt in range(cfg.T):
        for j in range(cfg.k):
            if sr[tt, j] >= 0:
                ref[tt] += On[sr[tt, j]]
    assert np.array_equal(to_np(y32).reshape(cfg.T, cfg.D), ref), "combine, drops"
    assert_rounded_from(y, y32, "combine, drops (bf16)")


def test_small_workspace_rejected_before_launch():
    cfg = PARITY["glm45_small"]
    t = workloads.generate(cfg, seed=0, device="cuda")
    L = new_layer(cfg)
    y = torch.full((cfg.T * cfg.D,), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoEError) as ei:
        B.moe_forward(L.handle, L.desc, t["x"], t["W_r"], t["bias"], t["W1"], None, t["W2"],
                      None, t["Wsh_gu"], t["Wsh_dn"], y, L.ws[:1024])
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (y.float() == 3.0).all()
