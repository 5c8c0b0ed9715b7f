"""The tiled weight layout (moe_tile_weights): its bytes against the layout
the C header defines, written out here with numpy, and the layer on tiled
weights against the layer on row-major weights (bitwise: only where the
GEMM reads each weight from changes, not any arithmetic)."""
import numpy as np
import pytest
import torch

import workloads
from sparse_mixture_experts_15_amd import binding as B
from tests.gpu_util import forward, new_layer, tiled_weights, to_np

pytestmark = pytest.mark.gpu

S = workloads.shrink


def tiled_reference(W, E, rows, n_out, K, swiglu, f_split):
    """The header's definition: per expert, tiles of 256 weight rows (SwiGLU:
    per 64 rows, 32 gate rows and the matching 32 up rows, 128 output columns
    per tile) by K stages of 64; row b, element c of a block at
    b*64 + 8*((c/8) ^ (b % 8)) + c % 8; zeros past the matrix and past K."""
    per = 128 if swiglu else 256
    nt, nk = -(-n_out // per), -(-K // 64)
    W = W.reshape(E, rows, K)
    out = np.zeros((E, nt, nk, 256, 64), dtype=np.uint16)
    c = np.arange(64)
    for n in range(nt):
        for b in range(256):
            if swiglu:
                g, w = divmod(b, 64)
                col = n * per + 32 * g + (w % 32)
                row = col + (f_split if w >= 32 else 0)
            else:
                col = row = n * per + b
            if col >= n_out:
                continue
            pos = 8 * ((c // 8) ^ (b % 8)) + c % 8
            for s in range(nk):
                k = s * 64 + c
                ok = k < K
                out[:, n, s, b, pos[ok]] = W[:, row, k[ok]]
    return out.reshape(-1)


@pytest.mark.parametrize("name,cfg", [
    ("swiglu_ragged", S(workloads.GLM45_PREFILL, T=8, D=200, F=200, F_shared=136).replace(M=3, k=2)),
    ("gelu_ragged", S(workloads.GLAM_4K, T=8, D=136, F=264).replace(M=2)),
])
def test_tile_layout_matches_definition(name, cfg):
    t = workloads.generate(cfg, seed=3, device="cuda")
    L = new_layer(cfg)
    d = L.desc
    sw = cfg.act == "swiglu"
    mats = {"W1": (cfg.M, (2 if sw else 1) * cfg.F, cfg.F, cfg.D, sw, cfg.F),
            "W2": (cfg.M, cfg.D, cfg.D, cfg.F, False, cfg.D)}
    if cfg.F_shared:
        mats["Wsh_gu"] = (1, 2 * cfg.F_shared, cfg.F_shared, cfg.D, True, cfg.F_shared)
        mats["Wsh_dn"] = (1, cfg.D, cfg.D, cfg.F_shared, False, cfg.D)
    for wname, (E, rows, n_out, K, swiglu, f_split) in mats.items():
        got = B.tile_weights(L.handle, d, wname, t[wname])
        torch.cuda.synchronize()
        src = to_np(t[wname].view(torch.int16)).view(np.uint16)
        ref = tiled_reference(src, E, rows, n_out, K, swiglu, f_split)
        g = to_np(got.view(torch.int16)).view(np.uint16)
        assert g.shape == ref.shape, wname
        assert (g == ref).all(), f"{wname}: {(g != ref).sum()} elements differ"


@pytest.mark.parametrize("name,cfg", [
    ("glam_mid", S(workloads.GLAM_4K, T=512, D=512, F=1024).replace(M=8)),
    ("glm45_small", S(workloads.GLM45_PREFILL, T=333, D=264, F=200, F_shared=136)),
    ("glm5_rows", S(workloads.GLM5_ZIPF, T=600, D=320, F=136, F_shared=136).replace(M=24)),
    ("decode_small", S(workloads.GLM45_DECODE, T=64, D=264, F=200, F_shared=200)),
])
def test_tiled_forward_equals_row_major(name, cfg):
    t = workloads.generate(cfg, seed=2, device="cuda")
    L_rows = new_layer(cfg)
    L_tiled = new_layer(cfg, weight_layout="tiled")
    tt = tiled_weights(L_tiled, t)
    aux = torch.cuda.Stream()
    y_rows = forward(L_rows, t, aux=aux)
    y_tiled = forward(L_tiled, tt, aux=aux)
    torch.cuda.synchronize()
    assert torch.equal(y_rows.view(torch.int16), y_tiled.view(torch.int16))
