"""CPU oracle for the sparse MoE feed-forward layer: forward pass and gradient.

TEST INFRASTRUCTURE ONLY.  The plain fp64 definition of the layer lives in
``moe_oracle.c`` (one token at a time, OpenMP across tokens); this module
loads it with ctypes and adds the page-fixed parameter accounting.  Only the
tests, the smoke check and the harness's CPU-baseline leg may import it; the
HIP library shares no code with it.

Arrays are numpy on the host: x and the expert/shared weights as float32
(fp32 layers) or uint16 holding bf16 bit patterns (bf16 layers); W_r and the
correction bias as float32.  Nothing here rounds: every value is widened
exactly to fp64 inside the C code.

Parameter accounting follows the "Parameters" table of the GLM-5 shared
expert inspector page: a SwiGLU of width F on hidden size D has a gate and
an up projection of D x F each and a down projection of F x D.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

SOFTMAX, SIGMOID = 0, 1
SWIGLU, GELU = 0, 1
F32, BF16 = 0, 1

GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
             "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE fp64: no fast-math, no FMA
    contraction).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int64), ("M", ctypes.c_int64),
                ("F", ctypes.c_int64), ("F_shared", ctypes.c_int64),
                ("k", ctypes.c_int32), ("scorer", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("alpha", ctypes.c_double),
                ("eps", ctypes.c_double), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        cp = ctypes.POINTER(_Cfg)
        lib.oracle_route.argtypes = [cp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_dispatch.argtypes = [i64, i32, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_expert.argtypes = [cp, vp, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_shared.argtypes = [cp, vp, i64, vp, vp, vp]
        lib.oracle_layer.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                     vp, vp, vp]
        lib.oracle_forward.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp,
                                       vp, vp, vp]
        lib.oracle_backward.argtypes = [cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp, vp, vp, vp, i64]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        for f in ("oracle_route", "oracle_dispatch", "oracle_expert", "oracle_shared",
                  "oracle_layer", "oracle_forward", "oracle_backward"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results are the
    same for any count)."""
    _load().oracle_set_num_threads(int(n))


def make_cfg(cfg) -> _Cfg:
    """Oracle descriptor from any object with the layer fields (T, D, M, F,
    F_shared, k, scorer, act, dtype, renorm, alpha, eps; n_group and
    topk_group when present)."""
    return _Cfg(T=cfg.T, D=cfg.D, M=cfg.M, F=cfg.F, F_shared=cfg.F_shared, k=cfg.k,
                scorer=SOFTMAX if cfg.scorer == "softmax" else SIGMOID,
                act=SWIGLU if cfg.act == "swiglu" else GELU,
                dtype=F32 if cfg.dtype == "f32" else BF16,
                renorm=1 if cfg.renorm else 0, alpha=float(cfg.alpha), eps=float(cfg.eps),
                n_group=int(getattr(cfg, "n_group", 0)),
                topk_group=int(getattr(cfg, "topk_group", 0)))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_storage(c: _Cfg, **arrays):
    want = np.float32 if c.dtype == F32 else np.uint16
    for name, a in arrays.items():
        if a is None:
            continue
        if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"oracle: {name} must be contiguous {np.dtype(want).name}")


def _f32(a):
    if a is None:
        return None
    if a.dtype != np.float32 or not a.flags["C_CONTIGUOUS"]:
        raise TypeError("oracle: router weights and bias must be contiguous float32")
    return a


def _tokens(cfg, tokens):
    if tokens is None:
        return np.arange(cfg.T, dtype=np.int64)
    return np.ascontiguousarray(tokens, dtype=np.int64)


def route(cfg, x, W_r, bias=None, tokens=None, want_logits=False, want_sel=False):
    """Router for the listed tokens (default: all T).  Returns idx[n,k]
    int32, w[n,k] fp64, gap[n] fp64 (k-th minus (k+1)-th selection score)
    and, if asked, logits[n,M] and selection scores sel[n,M] (fp64), in
    that order."""
    c = make_cfg(cfg)
    _check_storage(c, x=x)
    tok = _tokens(cfg, tokens)
    n = tok.shape[0]
    idx = np.zeros((n, cfg.k), np.int32)
    w = np.zeros((n, cfg.k), np.float64)
    gap = np.zeros(n, np.float64)
    logits = np.zeros((n, cfg.M), np.float64) if want_logits else None
    sel = np.zeros((n, cfg.M), np.float64) if want_sel else None
    _load().oracle_route(ctypes.byref(c), _ptr(x), _ptr(_f32(W_r)), _ptr(_f32(bias)), n,
                         _ptr(tok), _ptr(idx), _ptr(w), _ptr(gap), _ptr(logits), _ptr(sel))
    res = [idx, w, gap]
    if want_logits:
        res.append(logits)
    if want_sel:
        res.append(sel)
    return tuple(res)


def dispatch(T: int, k: int, M: int, idx):
    """Counts, offsets and the stable expert-major permutation of the T*k
    flat slots.  Returns a dict of int32 arrays."""
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
    S = T * k
    assert idx.shape[0] == S
    out = {"counts": np.zeros(M, np.int32), "offsets": np.zeros(M + 1, np.int32),
           "sorted_token": np.zeros(S, np.int32), "sorted_slot": np.zeros(S, np.int32),
           "slot_row": np.zeros(S, np.int32)}
    _load().oracle_dispatch(T, k, M, _ptr(idx), _ptr(out["counts"]), _ptr(out["offsets"]),
                            _ptr(out["sorted_token"]), _ptr(out["sorted_slot"]),
                            _ptr(out["slot_row"]))
    return out


def expert(cfg, x, t, e, W1, b1, W2, b2):
    """E_e(x_t) as fp64[D]."""
    c = make_cfg(cfg)
    _check_storage(c, x=x, W1=W1, b1=b1, W2=W2, b2=b2)
    out = np.zeros(cfg.D, np.float64)
    _load().oracle_expert(ctypes.byref(c), _ptr(x), int(t), int(e), _ptr(W1), _ptr(b1),
                          _ptr(W2), _ptr(b2), _ptr(out))
    return out


def shared(cfg, x, t, Wsh_gu, Wsh_dn):
    """E_sh(x_t) as fp64[D]."""
    c = make_cfg(cfg)
    _check_storage(c, x=x, Wsh_gu=Wsh_gu, Wsh_dn=Wsh_dn)
    out = np.zeros(cfg.D, np.float64)
    _load().oracle_shared(ctypes.byref(c), _ptr(x), int(t), _ptr(Wsh_gu), _ptr(Wsh_dn),
                          _ptr(out))
    return out


def layer(cfg, x, idx, w, W1, b1, W2, b2, Wsh_gu=None, Wsh_dn=None, tokens=None,
          want_slots=False, want_shared=False):
    """Layer output for the listed tokens given routing idx[T,k], w[T,k]
    (indexed by token).  Returns y[n,D] fp64, plus per-slot weighted expert
    outputs [n,k,D] and the shared-expert output [n,D] when asked."""
    c = make_cfg(cfg)
    _check_storage(c, x=x, W1=W1, b1=b1, W2=W2, b2=b2, Wsh_gu=Wsh_gu, Wsh_dn=Wsh_dn)
    if cfg.F_shared > 0 and (Wsh_gu is None or Wsh_dn is None):
        raise ValueError("oracle: F_shared > 0 needs both shared weights")
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(cfg.T, cfg.k)
    w = np.ascontiguousarray(w, dtype=np.float64).reshape(cfg.T, cfg.k)
    tok = _tokens(cfg, tokens)
    n = tok.shape[0]
    y = np.zeros((n, cfg.D), np.float64)
    slots = np.zeros((n, cfg.k, cfg.D), np.float64) if want_slots else None
    sh = np.zeros((n, cfg.D), np.float64) if want_shared else None
    _load().oracle_layer(ctypes.byref(c), _ptr(x), _ptr(idx), _ptr(w), _ptr(W1), _ptr(b1),
                         _ptr(W2), _ptr(b2), _ptr(Wsh_gu), _ptr(Wsh_dn), n, _ptr(tok),
                         _ptr(y), _ptr(slots), _ptr(sh))
    res = [y]
    if want_slots:
        res.append(slots)
    if want_shared:
        res.append(sh)
    return res[0] if len(res) == 1 else tuple(res)


def forward(cfg, h, tokens=None):
    """Router then layer for the listed tokens, from a dict of host arrays
    (keys as produced by the input generator).  Returns idx[n,k], w[n,k],
    y[n,D] indexed by list position."""
    c = make_cfg(cfg)
    _check_storage(c, x=h["x"], W1=h["W1"], b1=h.get("b1"), W2=h["W2"], b2=h.get("b2"),
                   Wsh_gu=h.get("Wsh_gu"), Wsh_dn=h.get("Wsh_dn"))
    tok = _tokens(cfg, tokens)
    n = tok.shape[0]
    idx = np.zeros((n, cfg.k), np.int32)
    w = np.zeros((n, cfg.k), np.float64)
    y = np.zeros((n, cfg.D), np.float64)
    _load().oracle_forward(ctypes.byref(c), _ptr(h["x"]), _ptr(_f32(h["W_r"])),
                           _ptr(_f32(h.get("bias"))), _ptr(h["W1"]), _ptr(h.get("b1")),
                           _ptr(h["W2"]), _ptr(h.get("b2")), _ptr(h.get("Wsh_gu")),
                           _ptr(h.get("Wsh_dn")), n, _ptr(tok), _ptr(idx), _ptr(w), _ptr(y))
    return idx, w, y


def backward(cfg, h, dy, experts=None):
    """Gradient of forward() over all T tokens for the output gradient
    dy[T,D] (any float array, used in fp64).  Returns a dict of fp64 arrays:
    dx[T,D], dW_r[M,D], dW1 / dW2 (and db1 / db2 when the layer has biases,
    dWsh_gu / dWsh_dn when it has a shared expert) in their weights' shapes,
    and the load statistics load_count[M] (int64 slots per expert) and
    load_score[M] (sum over tokens of each expert's gate value).

    ``experts`` (a list of expert ids) keeps the expert weight and bias
    gradients of those experts only, stacked in list order (dW1 is then
    [len(experts), G*F, D]); everything else is unchanged."""
    c = make_cfg(cfg)
    _check_storage(c, x=h["x"], W1=h["W1"], b1=h.get("b1"), W2=h["W2"], b2=h.get("b2"),
                   Wsh_gu=h.get("Wsh_gu"), Wsh_dn=h.get("Wsh_dn"))
    T, D, M, F, Fs = cfg.T, cfg.D, cfg.M, cfg.F, cfg.F_shared
    G = 2 if cfg.act == "swiglu" else 1
    dy = np.ascontiguousarray(dy, dtype=np.float64).reshape(T, D)
    slot, Mg = None, M
    if experts is not None:
        slot = np.full(M, -1, np.int32)
        for i, e in enumerate(experts):
            assert 0 <= e < M and slot[e] < 0, "experts must be distinct ids below M"
            slot[e] = i
        Mg = len(experts)
    out = {"dx": np.zeros((T, D)), "dW_r": np.zeros((M, D)),
           "dW1": np.zeros((Mg, G * F, D)), "dW2": np.zeros((Mg, D, F)),
           "load_count": np.zeros(M, np.int64), "load_score": np.zeros(M)}
    if h.get("b1") is not None:
        out["db1"] = np.zeros((Mg, F))
    if h.get("b2") is not None:
        out["db2"] = np.zeros((Mg, D))
    if Fs > 0:
        out["dWsh_gu"] = np.zeros((2 * Fs, D))
        out["dWsh_dn"] = np.zeros((D, Fs))
    _load().oracle_backward(
        ctypes.byref(c), _ptr(h["x"]), _ptr(_f32(h["W_r"])), _ptr(_f32(h.get("bias"))),
        _ptr(h["W1"]), _ptr(h.get("b1")), _ptr(h["W2"]), _ptr(h.get("b2")),
        _ptr(h.get("Wsh_gu")), _ptr(h.get("Wsh_dn")), _ptr(dy), _ptr(out["dx"]),
        _ptr(out["dW_r"]), _ptr(out["dW1"]), _ptr(out.get("db1")), _ptr(out["dW2"]),
        _ptr(out.get("db2")), _ptr(out.get("dWsh_gu")), _ptr(out.get("dWsh_dn")),
        _ptr(out["load_count"]), _ptr(out["load_score"]), _ptr(slot), Mg)
    return out


# ---- parameter accounting ("Parameters" table, GLM-5 shared expert page) ----

def swiglu_params(D: int, F: int) -> int:
    """Gate (D x F) + up (D x F) + down (F x D)."""
    return D * F + D * F + F * D


def gelu_ffn_params(D: int, F: int, biases: bool) -> int:
    """W1 (F x D) + W2 (D x F), plus b1 (F) and b2 (D) when present."""
    return 2 * D * F + ((F + D) if biases else 0)


def routed_expert_params(cfg) -> int:
    if cfg.act == "swiglu":
        return swiglu_params(cfg.D, cfg.F)
    return gelu_ffn_params(cfg.D, cfg.F, cfg.ffn_bias_std > 0)


def layer_params(cfg) -> dict:
    """Total and per-token-active parameter counts of one MoE layer."""
    routed = routed_expert_params(cfg)
    shared_p = swiglu_params(cfg.D, cfg.F_shared) if cfg.F_shared else 0
    router = cfg.M * cfg.D
    bias = cfg.M if cfg.scorer == "sigmoid" else 0
    return {"routed_per_expert": routed, "shared": shared_p, "router": router,
            "correction_bias": bias,
            "total": cfg.M * routed + shared_p + router + bias,
            "active_per_token": cfg.k * routed + shared_p + router + bias}
