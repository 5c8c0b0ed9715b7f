"""The weight-gradient allowances used by the backward parity tests hold for
a numpy emulation of the bf16 path's roundings (saved pre-activations and
the pre-activation gradient in bf16, everything else exact), on shapes with
many pre-activations near the zeros of the activations' derivatives; and a
plain relative bound would not."""
import numpy as np
import pytest
from scipy import special

from tests.gpu_util import ffn_grad_allowances


def _bf16(a):
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _act_grad(act, z, dh):
    F = dh.shape[1]
    if act == "gelu":
        return dh * (special.ndtr(z) + z * np.exp(-0.5 * z * z) / np.sqrt(2 * np.pi))
    a, b = z[:, :F], z[:, F:]
    sg = special.expit(a)
    return np.concatenate([dh * b * sg * (1 + a * (1 - sg)), dh * a * sg], axis=1)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_w1_allowance_covers_bf16_roundings(act):
    rng = np.random.default_rng(4)
    n, D, F = 24, 96, 512
    G = 2 if act == "swiglu" else 1
    X = _bf16(rng.normal(0, 1, (n, D)))
    W1 = _bf16(rng.normal(0, 1 / np.sqrt(D), (G * F, D)))
    W2 = _bf16(rng.normal(0, 1 / np.sqrt(F), (D, F)))
    b1 = _bf16(rng.normal(0, 0.1, F)) if act == "gelu" else None
    dO = rng.normal(0, 1, (n, D)) * rng.uniform(0.1, 1.0, (n, 1))
    z = X @ W1.T + (b1 if b1 is not None else 0.0)
    dh = dO @ W2
    exact = _act_grad(act, z, dh).T @ X
    # the bf16 path: z through fp32 then bf16, dh in fp32, dz rounded to bf16
    zs = _bf16(np.float32(z))
    dz = _bf16(np.float32(_act_grad(act, zs, np.float64(np.float32(dh)))))
    emul = dz.T @ X
    err = np.abs(emul - exact)
    allow = ffn_grad_allowances(act, X, W1, b1, W2, dO)[0]
    rms = np.sqrt(np.mean(exact ** 2))
    assert (err <= allow + 1e-3 * rms).all(), float((err - allow).max() / rms)
    # many pre-activations sit near the derivative's zero, where a relative
    # bound of a few bf16 roundings breaks down
    rel = err / np.maximum(np.abs(exact), 1e-300)
    assert (rel > 4 * 2.0 ** -8).any()


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_w2_allowance_covers_bf16_roundings(act):
    rng = np.random.default_rng(5)
    n, D, F = 16, 128, 256
    G = 2 if act == "swiglu" else 1
    X = _bf16(rng.normal(0, 1, (n, D)))
    W1 = _bf16(rng.normal(0, 1 / np.sqrt(D), (G * F, D)))
    W2 = _bf16(rng.normal(0, 1 / np.sqrt(F), (D, F)))
    dO = rng.normal(0, 1, (n, D))
    z = X @ W1.T
    H = (0.5 * z * (1 + special.erf(z / np.sqrt(2))) if act == "gelu"
         else special.expit(z[:, :F]) * z[:, :F] * z[:, F:])
    exact = dO.T @ H
    emul = _bf16(dO).T @ _bf16(np.float32(H))
    allow = ffn_grad_allowances(act, X, W1, None, W2, dO)[1]
    rms = np.sqrt(np.mean(exact ** 2))
    err = np.abs(emul - exact)
    assert (err <= allow + 1e-3 * rms).all()
    # cancellation across tokens: a bound relative to |dW2| alone fails
    assert (err > 2.0 ** -7 * np.abs(exact) + 1e-3 * rms).any()


@pytest.mark.parametrize("scorer,renorm,alpha", [("softmax", True, 1.0), ("sigmoid", True, 2.5),
                                                 ("sigmoid", False, 1.5),
                                                 ("softmax", False, 0.7)])
def test_tie_weights_helper_matches_the_oracle(scorer, renorm, alpha):
    """The helper that weights a tie-exempt token's alternative expert set
    reproduces the oracle's own weights on the oracle's own selection."""
    import oracle
    import workloads
    from tests.gpu_util import weights_for
    cfg = workloads.shrink(workloads.GLM45_PREFILL, T=40, D=64, F=16, F_shared=0).replace(
        scorer=scorer, renorm=renorm, alpha=alpha, M=24, k=4)
    h = workloads.host_inputs(workloads.generate(cfg, seed=7, device="cpu"))
    idx, w, _, logits = oracle.route(cfg, h["x"], h["W_r"], h["bias"], want_logits=True)
    got = weights_for(cfg, logits, idx)
    assert np.allclose(got, w, rtol=1e-12, atol=1e-15 * alpha)


def test_tie_exempt_check_accepts_the_alternative_and_catches_errors():
    """check_tie_exempt on a planted alternative selection: one token's k-th
    expert swapped for its (k+1)-th, the output computed by the oracle on
    that selection, passes; the same with a 5% error in that token fails."""
    import oracle
    import workloads
    from tests.gpu_util import check_tie_exempt, weights_for
    cfg = workloads.shrink(workloads.GLM45_PREFILL, T=24, D=64, F=32, F_shared=32).replace(
        M=16, k=4)
    h = workloads.host_inputs(workloads.generate(cfg, seed=3, device="cpu"))
    idx_o, w_o, _, logits, sel = oracle.route(cfg, h["x"], h["W_r"], h["bias"],
                                              want_logits=True, want_sel=True)
    t0 = 5
    order = np.lexsort((np.arange(cfg.M), -sel[t0]))   # best first, lower index on ties
    alt = np.sort(np.concatenate([order[:cfg.k - 1], order[cfg.k:cfg.k + 1]]))
    idx_g = idx_o.copy()
    idx_g[t0] = alt
    w_g = weights_for(cfg, logits, idx_g).astype(np.float32)
    y_g = oracle.layer(cfg, h["x"], idx_g, w_g.astype(np.float64), h["W1"], h["b1"], h["W2"],
                       h["b2"], h["Wsh_gu"], h["Wsh_dn"])
    mism = np.zeros(cfg.T, bool)
    mism[t0] = True
    scale = float(np.sqrt(np.mean(y_g ** 2)))
    assert check_tie_exempt(cfg, h, mism, idx_g, w_g, y_g, logits, idx_o, w_o, scale, "t") == 1
    bad = y_g.copy()
    bad[t0, 3] += 0.05 * scale
    with pytest.raises(AssertionError):
        check_tie_exempt(cfg, h, mism, idx_g, w_g, bad, logits, idx_o, w_o, scale, "t")
