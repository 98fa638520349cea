"""The forward pass captured in a HIP graph (torch.cuda.CUDAGraph on the
library's launch stream) and replayed: every replay, with eager work and
synchronisations between replays and new token values each time, gives the
same bits as an eager moe_forward on the same inputs."""
import pytest
import torch

import sparse_mixture_experts_gating_amd as moe
import workloads
from gpu_harness import DEV, to_dev

pytestmark = pytest.mark.gpu

GRAPH_SPECS = workloads.SMALL


@pytest.mark.parametrize("spec", GRAPH_SPECS, ids=lambda s: s.name)
def test_graph_replays_match_eager(spec):
    dinp = to_dev(workloads.make_inputs(spec))
    cfg = moe.config_from_spec(spec)
    w = moe.make_weights(dinp)
    routing = moe.alloc_routing(cfg, DEV)
    r = moe.make_routing(routing)
    ws = moe.alloc_workspace(cfg, moe.STAGE_FORWARD, DEV)
    x = dinp["x"].clone()
    y = torch.empty((spec.T, spec.d), dtype=spec.torch_dtype, device=DEV)

    def step():
        moe.moe_forward(cfg, x, w, y, r, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up outside the capture (first-use queries are cached)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    gen = torch.Generator(device="cpu")
    for rep in range(3):
        gen.manual_seed(900 + rep)
        new_x = torch.randn(spec.T, spec.d, generator=gen).to(spec.torch_dtype).to(DEV)
        x.copy_(new_x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y_graph = y.clone()
        y.zero_()
        torch.cuda.synchronize()
        step()  # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(y_graph, y), f"replay {rep}"
    del g
