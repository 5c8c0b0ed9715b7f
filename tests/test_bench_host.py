"""Host-side checks of the benchmark script: its algorithmic work counts
for the layer shapes (active FLOPs: 2 D F (G + 1) per routed pair, 6 D F_sh
per token for the shared expert, 2 D M per token for the router; bytes: the
touched experts' weights, shared weights, router weights, x and y), and
that it refuses more than one GPU before touching one."""
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("name,U,tflop,gbytes", [
    ("glam", 64, 2.201, 17.25),     # every expert reached
    ("glm45", 160, 3.492, 7.77),    # all 160 experts reached
    ("glm45", 63, 3.492, 3.19),     # 63 reached
    ("glm5", 256, 11.18, 19.81),
    ("decode", 40, 0.0273, 1.94),
    ("glm45dense", 1, 3.479, 0.5925),   # 6 T D F + the one-expert router
])
def test_layer_work(name, U, tflop, gbytes):
    cfg = workloads.get(name)
    flops, byts = bench.layer_work(cfg, U)
    assert flops / 1e12 == pytest.approx(tflop, rel=2e-3)
    assert byts / 1e9 == pytest.approx(gbytes, rel=5e-3)


def test_default_weight_layout_follows_dtype():
    # the tiled weight copy is bf16 only: fp32 layers default to row-major
    for cfg in workloads.CONFIGS:
        assert bench.default_weight_layout(cfg) == ("tiled" if cfg.dtype == "bf16" else "rows")
    assert bench.default_weight_layout(workloads.get("tiny")) == "rows"


def test_backward_work_counts_all_experts_gradients():
    cfg = workloads.get("glm45")
    w, flops = bench.backward_work(cfg, 68)
    G = 2
    _, by = w["b_wgrad"]
    # every expert's weight gradient is written (zeros for unreached ones)
    assert by >= cfg.M * (G + 1) * cfg.F * cfg.D * 4
    # the gradients of every forward GEMM: twice the forward's active FLOPs
    fwd_gemm = 2 * cfg.T * cfg.k * cfg.D * cfg.F * (G + 1) + 6 * cfg.T * cfg.D * cfg.F_shared
    assert flops >= 2 * fwd_gemm


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_work_credits_only_algorithmic_bytes():
    """Per kernel, only the touched weights, x and y are credited: no hidden
    activations H, no fp32 expert rows O, no shared rows Ysh."""
    cfg = workloads.get("glm45")
    counts = [100] * 68 + [0] * (cfg.M - 68)
    w, U = bench.kernel_work(cfg, counts)
    assert U == 68
    T, D, F, S = cfg.T, cfg.D, cfg.F, cfg.T * cfg.k
    assert w["ffn_up"] == (2.0 * S * D * 2 * F, 68 * 2 * F * D * 2 + T * D * 2)
    assert w["ffn_down"] == (2.0 * S * F * D, 68 * D * F * 2)
    assert w["shared_up"][1] == 2 * cfg.F_shared * D * 2 + T * D * 2
    assert w["shared_down"][1] == D * cfg.F_shared * 2
    assert w["combine"][1] == T * D * 2
    # the up projection is MFMA-bound at this shape: its FLOPs over its bytes
    # exceed the ridge of 2.5 PFLOP/s over 8 TB/s
    fl, by = w["ffn_up"]
    assert fl / by > bench.PEAK_BF16_TFLOPS / bench.PEAK_HBM_GBPS * 1e3


def test_default_workload_is_the_glm45_prefill_layer():
    import argparse
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--config", default="glm45")' in src
    assert workloads.get("glm45").name == "glm45_t8192_d5120_m160_f1536"


def test_routing_stats_of_reached_experts():
    s = bench.routing_stats([0, 4, 0, 2, 6])
    assert s["reached"] == 3 and s["rows_min"] == 2 and s["rows_max"] == 6
    assert s["rows_median"] == 4.0
    assert s["rows_cv"] == pytest.approx(1.632993 / 4, abs=1e-4)   # population std / mean
    assert bench.routing_stats([0, 0]) == {"reached": 0}
