"""Expert-parallel shares on one GPU: the float32 partial-output entry points
and a sweep over EP degrees.

Under expert parallelism every rank's [T, H] output is a partial sum of the
layer: tokens whose selected experts are elsewhere contribute zeros, and the
layer is the sum of all ranks' outputs ("Expert Parallelism (EP)", "Why a
Single All-Reduce/Reduce-Scatter Works"). The float32 form keeps each share
unrounded so that the layer is rounded once, after the sum.

Bars: a float32 share rounded to bf16 equals the bf16 share bit for bit (both
round the same float32 sum); the float32 combine is the oracle's combine of
the GPU's own expert outputs to within float32 summation error; the float32
shares of every EP degree add up to the all-local float32 output to within
that same summation error (the expert outputs do not depend on which other
experts are local); and the summed layer meets the 2e-2 bar against the
float64 oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import expert_token_routing_amd as M
import oracle.moe_oracle as O
import workloads as W
from tests.gpu_helpers import OUT_TOL, DevInputs, bf16_bits, bf16_f64, device, rel_max_err, say

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24  # unit roundoff of float32


def _bits16(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16)


def _abs_sum(out_bits: np.ndarray, inv: np.ndarray, w: np.ndarray, T: int, k: int) -> np.ndarray:
    """sum_j |w[t,j]| * |out[inv[t,j]]| per element: the scale of the float32
    summation error (sign bits cleared, then the oracle's combine)."""
    return O.oracle_combine(out_bits & np.uint16(0x7FFF), inv, np.abs(w), T, k)


CASES = [
    W.MoEConfig("f32_ragged", T=300, H=200, I=136, E=12, k=3, e0=4, E_local=5),
    W.MoEConfig("f32_many_experts", T=257, H=136, I=72, E=1024, k=32, e0=512, E_local=96),
    W.MoEConfig("f32_dma", T=640, H=576, I=448, E=16, k=4, e0=3, E_local=6, renormalize=0),
    W.MoEConfig("f32_single_expert", T=129, H=72, I=24, E=7, k=7, e0=6, E_local=1),
    # few tokens, long rows: each token's row is combined in two column blocks
    W.MoEConfig("f32_col_blocks", T=100, H=2048, I=64, E=8, k=2, e0=0, E_local=8),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_f32_combine_is_unrounded_combine(cfg):
    dev = device()
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    say(f"moe_combine_f32 {cfg.name}")
    _, idx, w = M.moe_route(d.x, d.w_router, d.bias, cfg.k, cfg.renormalize)
    _, offsets, _, inv, x_perm = M.moe_dispatch(d.x, idx, cfg.E, cfg.e0, cfg.E_local)
    _, out = M.moe_expert_ffn(x_perm, offsets, d.w_gate_up, d.w_down)
    y16 = M.moe_combine(out, inv, w)
    y32 = M.moe_combine_f32(out, inv, w)
    torch.cuda.synchronize()
    assert torch.equal(_bits16(y32.to(torch.bfloat16)), _bits16(y16))
    rinv = inv.cpu().numpy()
    gw = w.cpu().numpy().astype(np.float64)
    N = int(rinv.max()) + 1 if np.any(rinv >= 0) else 1
    outs = bf16_bits(out[:N])
    ref = O.oracle_combine(outs, rinv, gw, cfg.T, cfg.k)
    bound = cfg.k * EPS32 * _abs_sum(outs, rinv, gw, cfg.T, cfg.k)
    err = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float(np.max(err - bound))
    none = ~(rinv.reshape(cfg.T, cfg.k) >= 0).any(1)
    assert np.all(y32.cpu().numpy()[none] == 0.0)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_f32_forward_rounds_to_bf16_forward(cfg):
    dev = device()
    d = DevInputs(W.make_inputs(cfg), dev)
    say(f"moe_forward_f32 {cfg.name}")
    y16, _ = M.moe_forward(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize)
    y32, _ = M.moe_forward_f32(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize)
    torch.cuda.synchronize()
    assert y32.dtype == torch.float32
    assert torch.equal(_bits16(y32.to(torch.bfloat16)), _bits16(y16))


def test_f32_forward_empty_batch():
    dev = device()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    wr = torch.randn(4, 64, device=dev)
    gu = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=dev)
    dn = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    say("moe_forward_f32 empty batch")
    y, _ = M.moe_forward_f32(x, wr, None, gu, dn, 2, 0)
    assert y.shape == (0, 64) and y.dtype == torch.float32


def test_ep_sweep_f32_shares_sum_to_layer():
    """For EP degrees 1..E, the float32 shares of all ranks (e0 = r * E/ep)
    add up to the all-local float32 output within float32 summation error,
    and the summed layer meets the output bar against the float64 oracle."""
    dev = device()
    cfg = W.MoEConfig("ep_sweep", T=500, H=256, I=192, E=32, k=4, e0=0, E_local=32)
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    say("ep sweep: all-local steps T=500 E=32 k=4")
    logits, idx, w = M.moe_route(d.x, d.w_router, d.bias, cfg.k, cfg.renormalize)
    _, offsets, _, inv, x_perm = M.moe_dispatch(d.x, idx, cfg.E, 0, cfg.E)
    _, out = M.moe_expert_ffn(x_perm, offsets, d.w_gate_up, d.w_down)
    y_all = M.moe_combine_f32(out, inv, w)
    torch.cuda.synchronize()
    rinv = inv.cpu().numpy()
    gw = w.cpu().numpy().astype(np.float64)
    outs = bf16_bits(out[:int(rinv.max()) + 1])
    scale = _abs_sum(outs, rinv, gw, cfg.T, cfg.k)
    y_all64 = y_all.cpu().numpy().astype(np.float64)
    y_ref = O.oracle_forward(inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down, cfg.k, 0, cfg.E,
                             cfg.renormalize, logits=logits.cpu().numpy().astype(np.float64))
    for ep in (1, 2, 4, 8, 16, 32):
        El = cfg.E // ep
        say(f"ep sweep: ep={ep} E_local={El}")
        tot = np.zeros((cfg.T, cfg.H), np.float64)
        for r in range(ep):
            y_r, _ = M.moe_forward_f32(d.x, d.w_router, d.bias, d.w_gate_up[r * El:(r + 1) * El],
                                       d.w_down[r * El:(r + 1) * El], cfg.k, r * El, cfg.renormalize)
            tot += y_r.cpu().numpy().astype(np.float64)
        # each side is a float32 chain over at most k products
        err = np.abs(tot - y_all64)
        assert np.all(err <= 2 * cfg.k * EPS32 * scale), (ep, float(np.max(err - 2 * cfg.k * EPS32 * scale)))
        assert rel_max_err(tot, y_ref) <= OUT_TOL, ep
        # the layer rounded once is within the bar too
        assert rel_max_err(bf16_f64(torch.from_numpy(tot.astype(np.float32)).to(torch.bfloat16)), y_ref) <= OUT_TOL


def test_ep_tp_shares_sum_to_layer():
    """Variable EP + TP ("Expert Parallelism (EP)", "Variable EP (EP+TP for
    MoE)"): rank (r_ep, r_tp) runs its local experts' intermediate slice r_tp
    of tp. Each rank's float32 output meets the output bar against the
    oracle's output for the same shard, and the sum over all ranks meets it
    against the oracle's whole layer. Slices of 24 columns (tp = 16) take the
    k-by-32 GEMM path, the others the panel path."""
    dev = device()
    full = W.MoEConfig("eptp", T=300, H=256, I=384, E=8, k=2, e0=0, E_local=8)
    fi = W.make_inputs(full)
    fd = DevInputs(fi, dev)
    say("ep x tp shares: route T=300 E=8 k=2")
    logits, _, _ = M.moe_route(fd.x, fd.w_router, fd.bias, full.k, full.renormalize)
    gl = logits.cpu().numpy().astype(np.float64)
    y_ref = O.oracle_forward(fi.x, fi.w_router, fi.bias, fi.w_gate_up, fi.w_down, full.k, 0, full.E,
                             full.renormalize, logits=gl)
    for ep, tp in [(1, 2), (2, 4), (4, 3), (2, 16)]:
        El = full.E // ep
        tot = np.zeros((full.T, full.H), np.float64)
        for r_ep in range(ep):
            for r_tp in range(tp):
                c = full.scaled(I=full.I // tp, tp=tp, tp_rank=r_tp, e0=r_ep * El, E_local=El)
                si = W.make_inputs(c)
                sd = DevInputs(si, dev)
                say(f"ep x tp shares: ep={ep} tp={tp} rank ({r_ep}, {r_tp}) I={c.I}")
                y_r, _ = M.moe_forward_f32(sd.x, sd.w_router, sd.bias, sd.w_gate_up, sd.w_down, c.k, c.e0,
                                           c.renormalize)
                yr = y_r.cpu().numpy().astype(np.float64)
                ref_r = O.oracle_forward(si.x, si.w_router, si.bias, si.w_gate_up, si.w_down, c.k, c.e0, El,
                                         c.renormalize, logits=gl)
                assert rel_max_err(yr, ref_r) <= OUT_TOL, (ep, tp, r_ep, r_tp)
                tot += yr
        assert rel_max_err(tot, y_ref) <= OUT_TOL, (ep, tp)
