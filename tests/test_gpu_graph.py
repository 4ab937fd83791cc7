"""The whole share captured in a HIP graph and replayed, against eager calls.

The forward pass enqueues only kernels on the caller's stream (no host
synchronisation, no allocation, no memset), so a serving loop can capture it
once and replay it. Each replay must give the eager call's bits; eager work and
synchronisations run between the replays, and the output buffer is reset to
NaN before each one, so a replay that skipped a write would show.
"""
from __future__ import annotations

import pytest
import torch

import expert_token_routing_amd as M
import workloads as W
from tests.gpu_helpers import DevInputs, device, say

pytestmark = pytest.mark.gpu

CASES = [
    W.CONFIGS["tiny_top1"],
    W.CONFIGS["dsr1_ep8_decode"],
    W.MoEConfig("graph_ragged", T=1100, H=200, I=136, E=12, k=3, e0=4, E_local=5),
    W.MoEConfig("graph_dma", T=1500, H=256, I=384, E=16, k=4, e0=3, E_local=6),
]


@pytest.mark.parametrize("fused", [False, True], ids=["moe_forward", "moe_forward_fused"])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_graph_replays_match_eager(cfg, fused):
    dev = device()
    d = DevInputs(W.make_inputs(cfg), dev)
    fwd = M.moe_forward_fused if fused else M.moe_forward
    nbytes = M.forward_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.E_local)
    ws_eager = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_graph = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y_eager = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    y_graph = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    args = (d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize)

    say(f"graph {cfg.name} fused={fused}: eager reference")
    fwd(*args, y=y_eager, workspace=ws_eager)
    torch.cuda.synchronize()
    ref = y_eager.view(torch.int16).clone()

    say(f"graph {cfg.name} fused={fused}: capture")
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # one eager call on the capturing stream first
        fwd(*args, y=y_graph, workspace=ws_graph)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd(*args, y=y_graph, workspace=ws_graph)
    torch.cuda.synchronize()

    for rep in range(4):
        say(f"graph {cfg.name} fused={fused}: replay {rep}")
        y_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), ref), rep
        # eager work between the replays
        fwd(*args, y=y_eager, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(y_eager.view(torch.int16), ref), rep
