"""The MoELayer wrapper on a side stream: it orders that stream after the
current one (where the inputs were made and where temporaries were freed)
and marks its workspace and output as used by the side streams, so memory
the caching allocator hands out again on the current stream cannot be
overwritten under the layer.  Regression test for an unordered side-stream
call whose workspace was handed memory still being written."""
import pytest
import torch

import workloads
from tests.gpu_util import new_layer

pytestmark = pytest.mark.gpu


def _bits(y):
    return y.view(torch.int16)


def test_forward_on_side_stream_after_frees():
    cfg = workloads.shrink(workloads.GLM45_PREFILL, T=1500, D=256, F=128, F_shared=128)
    t = workloads.generate(cfg, seed=4, device="cuda")
    L = new_layer(cfg)
    args = (t["x"], t["W_r"], t["bias"], t["W1"], None, t["W2"], None, t["Wsh_gu"], t["Wsh_dn"])
    y_ref = L.forward(*args)
    torch.cuda.synchronize()
    side, aux = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        # temporaries made and freed on the current stream just before the call
        tmp = torch.randn(1 << 22, device="cuda") * (rep + 2)
        del tmp
        outs.append(L.forward(*args, stream=side, aux_stream=aux))
        # new work on the current stream right after: reuses freed memory
        junk = torch.full((1 << 22,), float(rep), device="cuda")
        junk.mul_(3.0)
        del junk
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(_bits(y), _bits(y_ref))
