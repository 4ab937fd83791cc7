"""moe_forward_noalloc (the forward in the library's static scratch, for
callers that cannot allocate) against moe_forward with a caller workspace,
through the C-ABI: two calls in a row, the second with a smaller problem, each
bit for bit equal to moe_forward's y."""
import ctypes

import numpy as np
import pytest
import torch

import expert_token_routing_amd as M
import workloads as W
from tests.gpu_helpers import DevInputs, device, say

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _case(cfg):
    dev = device()
    d = DevInputs(W.make_inputs(cfg), dev)
    c = cfg
    L = M.lib()
    stream = P(torch.cuda.current_stream(dev).cuda_stream)
    I = d.w_gate_up.shape[2] // 2
    ws_bytes = L.moe_forward_workspace_size(c.T, c.H, I, c.E, c.k, c.E_local)
    assert ws_bytes <= M.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    y_ref = torch.full((c.T, c.H), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((c.T, c.H), float("nan"), dtype=torch.bfloat16, device=dev)
    say(f"noalloc: moe_forward {cfg.name} T={c.T} H={c.H} I={I} E={c.E} k={c.k} e0={c.e0} E_local={c.E_local}")
    st = L.moe_forward(_ptr(d.x), _ptr(d.w_router), _ptr(d.bias), _ptr(d.w_gate_up), _ptr(d.w_down), c.T, c.H, I, c.E,
                       c.k, c.e0, c.E_local, c.renormalize, _ptr(y_ref), _ptr(ws), ws_bytes, stream)
    assert st == M.MOE_OK, M.status_string(st)
    say(f"noalloc: moe_forward_noalloc {cfg.name}")
    st = L.moe_forward_noalloc(_ptr(d.x), _ptr(d.w_router), _ptr(d.bias), _ptr(d.w_gate_up), _ptr(d.w_down), c.T, c.H,
                               I, c.E, c.k, c.e0, c.E_local, c.renormalize, _ptr(y), stream)
    assert st == M.MOE_OK, M.status_string(st)
    torch.cuda.synchronize()
    a = y.view(torch.int16).cpu().numpy()
    b = y_ref.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b), f"{cfg.name}: {int((a != b).sum())} elements differ from moe_forward"


def test_noalloc_equals_forward_two_calls():
    big = W.MoEConfig("noalloc_big", T=1536, H=1024, I=768, E=16, k=4, e0=4, E_local=8)
    small = W.MoEConfig("noalloc_small", T=200, H=256, I=96, E=8, k=2, e0=2, E_local=4)
    _case(big)
    _case(small)


def test_noalloc_rejects_oversize():
    # the DeepSeek-R1-shaped share at T = 16384 needs about 4 GB: rejected on
    # the host, nothing launched
    L = M.lib()
    T, H, I, E, k, El = 16384, 7168, 2048, 256, 8, 32
    assert L.moe_forward_workspace_size(T, H, I, E, k, El) > M.NOALLOC_SCRATCH_BYTES
    dev = device()
    x = torch.empty((16, 8), dtype=torch.bfloat16, device=dev)  # never read: the call is rejected first
    st = L.moe_forward_noalloc(_ptr(x), _ptr(x), None, _ptr(x), _ptr(x), T, H, I, E, k, 0, El, 1, _ptr(x), None)
    assert st == M.MOE_ERR_WORKSPACE
