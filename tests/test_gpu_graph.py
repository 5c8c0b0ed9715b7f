"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph) replays to the
eager result bitwise: the call enqueues only kernels and event
dependencies (no host synchronisation, no memset nodes), and the shared
expert's fork onto the second stream and its join are captured as graph
edges.  Each replay follows unrelated eager work and a synchronisation, and
is checked on its own."""
import pytest
import torch

import workloads
from tests.gpu_util import new_layer, tiled_weights

pytestmark = pytest.mark.gpu

S = workloads.shrink

GRAPH = {
    "glm45_shared": S(workloads.GLM45_PREFILL, T=333, D=264, F=200, F_shared=136),
    "decode": S(workloads.GLM45_DECODE, T=64, D=264, F=200, F_shared=200),
    "glam_t1500": S(workloads.GLAM_4K, T=1500, D=128, F=96),
}


def _bits(y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("name", list(GRAPH))
def test_graph_replay_matches_eager(name, tiled):
    cfg = GRAPH[name]
    t = workloads.generate(cfg, seed=2, device="cuda")
    L = new_layer(cfg, weight_layout="tiled" if tiled else "rows")
    if tiled:
        t = tiled_weights(L, t)
    main, aux = torch.cuda.Stream(), torch.cuda.Stream()
    y = torch.empty_like(t["x"])
    y_eager = torch.empty_like(t["x"])
    # the inputs, workspace and outputs were made on the current stream:
    # order both side streams after that work before using them
    torch.cuda.synchronize()
    main.wait_stream(torch.cuda.current_stream())
    aux.wait_stream(torch.cuda.current_stream())

    def fwd(out):
        L.forward(t["x"], t["W_r"], t["bias"], t["W1"], t["b1"], t["W2"], t["b2"],
                  t["Wsh_gu"], t["Wsh_dn"], y=out, stream=main, aux_stream=aux)

    with torch.cuda.stream(main):
        fwd(y_eager)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        fwd(y)
    torch.cuda.synchronize()

    scratch = torch.empty_like(t["x"])
    for rep in range(3):
        # unrelated eager work on the same workspace and streams in between
        with torch.cuda.stream(main):
            fwd(scratch)
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_eager)), f"replay {rep}"
