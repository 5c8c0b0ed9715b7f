"""moe_forward_no_alloc: the layer on the library's fixed per-GPU scratch,
for callers that cannot allocate.  Called through the C ABI twice in a row
(the second call with a smaller batch, so the scratch holds the first
call's data) and checked bitwise against moe_forward on a caller workspace,
which the other parity tests hold to the oracle.  A layer too large for the
scratch is refused before anything is enqueued."""
import ctypes

import pytest
import torch

import workloads
from sparse_mixture_experts_15_amd import binding as B
from tests.gpu_util import new_layer

pytestmark = pytest.mark.gpu


def _args(t):
    return (t["x"], t["W_r"], t["bias"], t["W1"], t.get("b1"), t["W2"], t.get("b2"),
            t.get("Wsh_gu"), t.get("Wsh_dn"))


def _bits(y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y


@pytest.mark.parametrize("name,T1,T2", [("decode", 64, 24), ("glm45_small", 200, 37)])
def test_no_alloc_matches_forward_twice(name, T1, T2):
    base = (workloads.get("decode") if name == "decode" else
            workloads.shrink(workloads.GLM45_PREFILL, T=200, D=264, F=200, F_shared=136))
    cfg = base.replace(T=T1)
    print(f"no-alloc forward: {cfg.name}, T {T1} then {T2}", flush=True)
    t = workloads.generate(cfg, seed=7, device="cuda")
    aux = torch.cuda.Stream()
    for T in (T1, T2):
        c = cfg.replace(T=T)
        L = new_layer(c)
        d = L.desc
        assert B.moe_workspace_size(d) <= B.NO_ALLOC_SCRATCH_BYTES
        tt = dict(t)
        tt["x"] = t["x"][:T].contiguous()
        y_ref = torch.empty(T, c.D, dtype=torch.bfloat16, device="cuda")
        B.moe_forward(L.handle, d, *_args(tt), y_ref, L.ws, aux_stream=aux)
        y = torch.full((T, c.D), 9.0, dtype=torch.bfloat16, device="cuda")
        B.moe_forward_no_alloc(L.handle, d, *_args(tt), y, aux_stream=aux)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref)), f"T={T}"
        L.close()


def test_no_alloc_refuses_a_layer_beyond_the_scratch():
    cfg = workloads.get("decode").replace(T=1024)
    d = B.make_desc(cfg)
    assert B.moe_workspace_size(d) > B.NO_ALLOC_SCRATCH_BYTES
    t = workloads.generate(cfg.replace(T=1), seed=0, device="cuda")
    x = torch.zeros(cfg.T, cfg.D, dtype=torch.bfloat16, device="cuda")
    y = torch.full((cfg.T, cfg.D), 3.0, dtype=torch.bfloat16, device="cuda")
    h = B.moe_create(0)
    try:
        with pytest.raises(B.MoEError) as ei:
            B.moe_forward_no_alloc(h, d, x, t["W_r"], t["bias"], t["W1"], None, t["W2"], None,
                                   t["Wsh_gu"], t["Wsh_dn"], y)
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert (y.float() == 3.0).all()
    finally:
        B.moe_destroy(h)
