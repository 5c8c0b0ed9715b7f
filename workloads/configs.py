"""Workload descriptions for the sparse MoE feed-forward layer.

Five layer shapes are used throughout: one tiny fp32 layer small enough for
brute force, three prefill layers and one decode layer.  They are taken from
the method's own architecture figures:

* GLaM study note, "Sparse MoE Layer": softmax router over an expert pool,
  top-2 selection, each expert a dense FFN ``W2 s(W1 x + b1) + b2``.
* "Shared Expert" (GLM-4.5 study note), "Overview" / "How it works": 160
  routed experts, 8 active per token, one always-on shared SwiGLU expert,
  hidden size 5120, expert width 1536, routed scaling factor 2.5.
* "GLM-5 Shared expert" inspector page, "Parameters" / "Explanation": hidden
  size 6144, shared SwiGLU width 2048; its 19,200 correction-bias values
  over 75 MoE blocks give 256 routed experts per block.

This module holds shapes and distribution parameters only.  It computes no
part of the layer.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                      # tokens (flattened batch x positions)
    D: int                      # hidden size
    M: int                      # routed experts
    F: int                      # routed expert width
    k: int                      # experts per token
    scorer: str                 # "softmax" | "sigmoid"
    act: str                    # "gelu" | "swiglu"
    F_shared: int = 0           # shared SwiGLU width, 0 = no shared expert
    dtype: str = "bf16"         # x, expert weights, shared weights and y
    renorm: bool = True         # renormalise the selected gate values
    alpha: float = 1.0          # routed scaling factor
    eps: float = 1e-20          # renormalisation epsilon
    router_bias_std: float = 0.0  # selection-only correction bias (sigmoid)
    ffn_bias_std: float = 0.0     # b1/b2 of GELU experts (0 = no biases)
    zipf_gamma: float = 0.0       # router row scale (pi(e)+1)^-gamma, 0 = off
    x_std: float = 1.0
    n_group: int = 0              # expert groups for group-limited routing (0 = none)
    topk_group: int = 0           # groups kept per token

    @property
    def G(self) -> int:
        """Rows of W1 per output column: 2 for SwiGLU (gate, up), 1 for GELU."""
        return 2 if self.act == "swiglu" else 1

    @property
    def has_router_bias(self) -> bool:
        return self.scorer == "sigmoid"

    @property
    def has_ffn_bias(self) -> bool:
        return self.ffn_bias_std > 0.0

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# Tiny GLaM-style layer, fp32 throughout, GELU experts with biases.  Biases
# are N(0, 0.01) read as variance 0.01, so std 0.1.
GLAM_TINY_FP32 = MoEConfig(
    name="glam_tiny_fp32_t64", T=64, D=64, M=8, F=256, k=2,
    scorer="softmax", act="gelu", dtype="f32", ffn_bias_std=0.1)

# GLaM-shaped layer: 64 experts, top-2, GELU D -> 16384 -> D, no biases.
GLAM_4K = MoEConfig(
    name="glam_t4096_d4096_m64_f16384", T=4096, D=4096, M=64, F=16384, k=2,
    scorer="softmax", act="gelu")

# GLM-4.5-shaped prefill layer.  Correction bias N(0, 0.1) read as variance
# 0.1 (std sqrt(0.1)), used only for selection.
GLM45_PREFILL = MoEConfig(
    name="glm45_t8192_d5120_m160_f1536", T=8192, D=5120, M=160, F=1536, k=8,
    scorer="sigmoid", act="swiglu", F_shared=1536, alpha=2.5,
    router_bias_std=math.sqrt(0.1))

# GLM-5-shaped layer with Zipf-skewed router rows; correction bias zero so
# the skew comes from the router weights alone.
GLM5_ZIPF = MoEConfig(
    name="glm5_t16384_d6144_m256_f2048_zipf", T=16384, D=6144, M=256, F=2048,
    k=8, scorer="sigmoid", act="swiglu", F_shared=2048, alpha=1.0,
    router_bias_std=0.0, zipf_gamma=0.3)

# Decode-shaped GLM-4.5 layer: 64 tokens (batch 64 x 1 position).
GLM45_DECODE = GLM45_PREFILL.replace(name="glm45_decode_t64_d5120_m160_f1536", T=64)

# The GLM-4.5 prefill layer with group-limited routing (the router's optional
# masking by expert group): 8 groups of 20 experts, the best 4 kept.  The
# page gives no group counts; these exercise the variant at full size.
GLM45_GROUPED = GLM45_PREFILL.replace(name="glm45_grouped_t8192_d5120_m160_f1536_g8k4",
                                      n_group=8, topk_group=4)

# Switch-style top-1 routing (the GLaM note's related-work table: top-1
# sparse FFN routing) through the same kernels, at the GLaM layer's shape.
# The gate value is the router probability itself: with one expert, the
# renormalised weight would always be 1.
SWITCH_TOP1 = GLAM_4K.replace(name="switch_top1_t4096_d4096_m64_f16384", k=1, renorm=False)

# A dense prefix layer of the GLM-4.5-shaped model (the "Shared Expert" note,
# "How it works": the first blocks hold one wide SwiGLU and no shared
# expert) through the same kernels: one expert, top-1, softmax, so the gate
# weight is exactly 1 and the layer is that plain SwiGLU.  The page gives no
# width; this takes the MoE layer's active width per token (8 x 1536 routed
# + 1536 shared = 13,824), so both layers do the same work per token.
GLM45_DENSE = GLM45_PREFILL.replace(
    name="glm45_dense_t8192_d5120_f13824", M=1, k=1, F=13824, F_shared=0,
    scorer="softmax", alpha=1.0, router_bias_std=0.0)

CONFIGS = [GLAM_TINY_FP32, GLAM_4K, GLM45_PREFILL, GLM5_ZIPF, GLM45_DECODE, GLM45_GROUPED,
           SWITCH_TOP1, GLM45_DENSE]
BY_NAME = {c.name: c for c in CONFIGS}
# Short aliases used by the harness command line.
ALIASES = {
    "tiny": GLAM_TINY_FP32, "glam": GLAM_4K, "glm45": GLM45_PREFILL,
    "glm5": GLM5_ZIPF, "decode": GLM45_DECODE, "glm45g": GLM45_GROUPED,
    "switch": SWITCH_TOP1, "glm45dense": GLM45_DENSE,
}


def get(name: str) -> MoEConfig:
    if name in ALIASES:
        return ALIASES[name]
    return BY_NAME[name]


def shrink(cfg: MoEConfig, T: int, D: int, F: int, F_shared: int | None = None,
           name: str | None = None) -> MoEConfig:
    """Same routing structure (M, k, scorer, alpha, bias and skew recipe) at
    a smaller T, D and F, for tests the oracle finishes in seconds."""
    if F_shared is None:
        F_shared = F if cfg.F_shared else 0
    return cfg.replace(name=name or f"{cfg.name}_shrunk_t{T}_d{D}_f{F}",
                       T=T, D=D, F=F, F_shared=F_shared)
