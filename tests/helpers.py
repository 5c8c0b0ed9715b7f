"""Test-side helpers: storage conversion and textbook dense building blocks
written with numpy / scipy library routines, used to pin the oracle against
something other than itself."""
from __future__ import annotations

import numpy as np
from scipy import special


def widen(a):
    """Host array (float32, or uint16 holding bf16 bits) -> float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def np_silu(z):
    return z * special.expit(z)


def np_gelu(z):
    return 0.5 * z * (1.0 + special.erf(z / np.sqrt(2.0)))


def dense_swiglu(X, Wgu, Wdn):
    """Batched SwiGLU with numpy matmuls: X[n,D], Wgu[2F,D] (gate rows then
    up rows), Wdn[D,F] -> [n,D]."""
    F = Wdn.shape[1]
    Z = X @ Wgu.T
    return (np_silu(Z[:, :F]) * Z[:, F:]) @ Wdn.T


def dense_gelu(X, W1, b1, W2, b2):
    Z = X @ W1.T
    if b1 is not None:
        Z = Z + b1
    Y = np_gelu(Z) @ W2.T
    if b2 is not None:
        Y = Y + b2
    return Y


def all_experts_dense(cfg, h):
    """Every expert applied to every token: [T, M, D] in fp64 (the work a
    sparse layer avoids), computed with numpy matmuls."""
    X = widen(h["x"])
    W1, W2 = widen(h["W1"]), widen(h["W2"])
    b1, b2 = widen(h.get("b1")), widen(h.get("b2"))
    out = np.zeros((cfg.T, cfg.M, cfg.D))
    for e in range(cfg.M):
        if cfg.act == "swiglu":
            out[:, e, :] = dense_swiglu(X, W1[e], W2[e])
        else:
            out[:, e, :] = dense_gelu(X, W1[e], None if b1 is None else b1[e],
                                      W2[e], None if b2 is None else b2[e])
    return out


def scatter_dense_weights(T, M, idx, w):
    """[T,k] routing -> [T,M] dense weights (zero off the selected set)."""
    wd = np.zeros((T, M))
    for t in range(T):
        for j in range(idx.shape[1]):
            e = idx[t, j]
            if 0 <= e < M:
                wd[t, e] += w[t, j]
    return wd


def rms(a):
    return float(np.sqrt(np.mean(np.square(a)))) if a.size else 0.0
