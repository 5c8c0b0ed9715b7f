"""Seeded synthetic inputs for the MoE layer.

Both the HIP path and the CPU oracle consume what this module produces; it
holds no part of the layer's arithmetic.  Recipe:

* one independent torch generator per tensor, seeded ``seed*16 + i`` with i
  the tensor's position in ``TENSOR_ORDER`` (the Zipf permutation uses
  i = 9);
* values are fp32 draws from N(0, 1) scaled by the tensor's std, then
  rounded to nearest-even into the storage dtype;
* std = 1/sqrt(fan_in): D for the router, W1 and the shared gate/up weights,
  F (or F_shared) for W2 and the shared down weights; x has std 1;
* Zipf-skewed router: row e is scaled by (pi(e)+1)^-gamma, pi a seeded
  permutation of the experts, so expert popularity falls off as a power law.

Large tensors are drawn one leading slice at a time so peak memory stays
near the tensor's own size.  Draws on a CUDA device and on the CPU use
different generators and give different (equally valid) values; a test
always hands the oracle a host copy of the exact tensors the GPU used.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .configs import MoEConfig

TENSOR_ORDER = ("x", "W_r", "bias", "W1", "b1", "W2", "b2", "Wsh_gu", "Wsh_dn")
_PERM_STREAM = 9

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(cfg: MoEConfig) -> torch.dtype:
    return _TORCH_DTYPE[cfg.dtype]


def _gen(seed: int, i: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + i)
    return g


def _normal(shape, std: float, dtype, g: torch.Generator, device) -> torch.Tensor:
    """N(0, std^2) in fp32, rounded to ``dtype``; drawn slice by slice along
    dim 0 for tensors with more than two dimensions."""
    out = torch.empty(shape, dtype=dtype, device=device)
    if len(shape) >= 3:
        for e in range(shape[0]):
            z = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
            out[e].copy_(z.mul_(std))
            del z
    else:
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.copy_(z.mul_(std))
    return out


def generate(cfg: MoEConfig, seed: int = 0, device="cpu") -> dict:
    """All layer inputs for ``cfg`` as torch tensors on ``device``.

    Keys: x[T,D], W_r[M,D] (fp32), bias[M] (fp32, sigmoid scorer only),
    W1[M,G*F,D] (SwiGLU: gate rows then up rows), b1[M,F], W2[M,D,F],
    b2[M,D] (biased GELU experts only), Wsh_gu[2*F_sh,D] (gate rows then up
    rows), Wsh_dn[D,F_sh] (shared expert only).  Absent tensors map to None.
    """
    dev = torch.device(device)
    dt = torch_dtype(cfg)
    T, D, M, F, G, Fs = cfg.T, cfg.D, cfg.M, cfg.F, cfg.G, cfg.F_shared
    t = {}
    t["x"] = _normal((T, D), cfg.x_std, dt, _gen(seed, 0, dev), dev)

    W_r = _normal((M, D), 1.0 / math.sqrt(D), torch.float32, _gen(seed, 1, dev), dev)
    if cfg.zipf_gamma > 0.0:
        gp = torch.Generator(device="cpu")
        gp.manual_seed(seed * 16 + _PERM_STREAM)
        perm = torch.randperm(M, generator=gp)
        scale = (perm.to(torch.float64) + 1.0).pow(-cfg.zipf_gamma).to(torch.float32)
        W_r.mul_(scale.to(dev)[:, None])
    t["W_r"] = W_r

    if cfg.has_router_bias:
        if cfg.router_bias_std > 0.0:
            t["bias"] = _normal((M,), cfg.router_bias_std, torch.float32, _gen(seed, 2, dev), dev)
        else:
            t["bias"] = torch.zeros(M, dtype=torch.float32, device=dev)
    else:
        t["bias"] = None

    t["W1"] = _normal((M, G * F, D), 1.0 / math.sqrt(D), dt, _gen(seed, 3, dev), dev)
    t["b1"] = (_normal((M, F), cfg.ffn_bias_std, dt, _gen(seed, 4, dev), dev)
               if cfg.has_ffn_bias else None)
    t["W2"] = _normal((M, D, F), 1.0 / math.sqrt(F), dt, _gen(seed, 5, dev), dev)
    t["b2"] = (_normal((M, D), cfg.ffn_bias_std, dt, _gen(seed, 6, dev), dev)
               if cfg.has_ffn_bias else None)
    if Fs > 0:
        t["Wsh_gu"] = _normal((2 * Fs, D), 1.0 / math.sqrt(D), dt, _gen(seed, 7, dev), dev)
        t["Wsh_dn"] = _normal((D, Fs), 1.0 / math.sqrt(Fs), dt, _gen(seed, 8, dev), dev)
    else:
        t["Wsh_gu"] = None
        t["Wsh_dn"] = None
    return t


def to_host_array(t: torch.Tensor | None):
    """Host numpy copy with the storage bits unchanged: bf16 becomes a uint16
    array of the raw bit patterns, fp32 stays float32, int32 stays int32."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_inputs(tensors: dict) -> dict:
    return {k: to_host_array(v) for k, v in tensors.items()}
