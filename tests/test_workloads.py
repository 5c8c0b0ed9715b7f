"""Seeded input generator: determinism, shapes, dtypes and the skew recipes."""
import numpy as np
import torch

import oracle
import workloads


def test_configs_shapes():
    c = workloads.CONFIGS
    assert [x.T for x in c] == [64, 4096, 8192, 16384, 64, 8192, 4096, 8192]
    assert [x.M for x in c] == [8, 64, 160, 256, 160, 160, 64, 1]
    assert [x.k for x in c] == [2, 2, 8, 8, 8, 8, 1, 1]
    assert [(x.n_group, x.topk_group) for x in c] == [(0, 0)] * 5 + [(8, 4), (0, 0), (0, 0)]
    assert not workloads.SWITCH_TOP1.renorm
    dense = workloads.GLM45_DENSE
    # the dense prefix layer: one SwiGLU as wide as the MoE layer's active width
    assert (dense.F, dense.F_shared, dense.act) == (8 * 1536 + 1536, 0, "swiglu")
    assert dense.scorer == "softmax" and dense.alpha == 1.0 and dense.renorm
    assert workloads.GLM45_DECODE.D == workloads.GLM45_PREFILL.D
    assert workloads.get("glm45") is workloads.GLM45_PREFILL


def test_generate_deterministic_and_shaped():
    cfg = workloads.shrink(workloads.GLM45_PREFILL, T=16, D=32, F=24)
    a = workloads.generate(cfg, seed=0)
    b = workloads.generate(cfg, seed=0)
    c = workloads.generate(cfg, seed=1)
    for k in workloads.TENSOR_ORDER:
        if a[k] is None:
            assert b[k] is None
            continue
        assert torch.equal(a[k], b[k])
    assert not torch.equal(a["x"], c["x"])
    assert a["x"].dtype == torch.bfloat16 and a["W_r"].dtype == torch.float32
    assert a["W1"].shape == (cfg.M, 2 * cfg.F, cfg.D)
    assert a["W2"].shape == (cfg.M, cfg.D, cfg.F)
    assert a["Wsh_gu"].shape == (2 * cfg.F, cfg.D) and a["Wsh_dn"].shape == (cfg.D, cfg.F)
    assert a["b1"] is None and a["bias"].shape == (cfg.M,)


def test_tensor_streams_are_independent():
    # changing one tensor's shape must not change another tensor's values
    c1 = workloads.shrink(workloads.GLM45_PREFILL, T=16, D=32, F=24)
    c2 = workloads.shrink(workloads.GLM45_PREFILL, T=16, D=32, F=40)
    a, b = workloads.generate(c1), workloads.generate(c2)
    assert torch.equal(a["x"], b["x"]) and torch.equal(a["W_r"], b["W_r"])


def test_std_recipe():
    cfg = workloads.shrink(workloads.GLM45_PREFILL, T=256, D=512, F=256)
    t = workloads.generate(cfg)
    assert abs(t["x"].float().std().item() - 1.0) < 0.02
    assert abs(t["W1"].float().std().item() * np.sqrt(512) - 1.0) < 0.02
    assert abs(t["W2"].float().std().item() * np.sqrt(256) - 1.0) < 0.02
    assert abs(t["bias"].std().item() - np.sqrt(0.1)) < 0.1


def test_fp32_layer_with_biases():
    t = workloads.generate(workloads.GLAM_TINY_FP32)
    assert t["x"].dtype == torch.float32 and t["b1"].shape == (8, 256)
    assert t["b2"].shape == (8, 64) and t["bias"] is None and t["Wsh_gu"] is None
    assert abs(t["b1"].std().item() - 0.1) < 0.02


def test_zipf_router_skews_counts():
    # router rows scaled by (pi(e)+1)^-0.3: popular experts take far more slots
    cfg = workloads.shrink(workloads.GLM5_ZIPF, T=1024, D=256, F=8, F_shared=8)
    h = workloads.host_inputs(workloads.generate(cfg))
    idx, _, _ = oracle.route(cfg, h["x"], h["W_r"], h["bias"])
    counts = np.sort(np.bincount(idx.reshape(-1), minlength=cfg.M))[::-1]
    assert counts[0] > 8 * max(1, np.median(counts))
    norms = np.linalg.norm(h["W_r"], axis=1)
    assert norms.max() / norms.min() > 4.0


def test_host_arrays_keep_bits():
    t = torch.tensor([1.0, -2.5, 3.140625], dtype=torch.bfloat16)
    a = workloads.to_host_array(t)
    assert a.dtype == np.uint16
    assert list(a) == [0x3F80, 0xC020, 0x4049]
