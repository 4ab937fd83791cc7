"""HIP path against the CPU oracle, through the C-ABI, on one GPU.

Bar (from the problem statement): routing indices, counts, offsets,
permutations and dispatched rows bit-exact given identical router logits;
expert outputs and the combined output within max relative error 2e-2
(bf16 inputs, float32 accumulation). Small sizes are compared element by
element; the full-size workloads on sampled rows that the oracle computes one
by one, plus properties that hold at any size.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import expert_token_routing_amd as M
import oracle.moe_oracle as O
import workloads as W
from tests import oracle_pins as P
from tests.gpu_helpers import (OUT_TOL, W_RTOL, DevInputs, bf16_bits, bf16_f64, device, panel_blocks, rel_max_err,
                               say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu

_INPUT_CACHE: dict = {}


def inputs_for(cfg: W.MoEConfig) -> W.MoEInputs:
    key = cfg
    if key not in _INPUT_CACHE:
        _INPUT_CACHE.clear()
        _INPUT_CACHE[key] = W.make_inputs(cfg)
    return _INPUT_CACHE[key]


def ragged(name, **kw):
    return W.MoEConfig(name, **kw)


# Small problems the oracle finishes in seconds; they span several tiles in
# every kernel and end in ragged tails (T not a multiple of 64/128, H and I
# not multiples of the 64-wide k stage or the 128/256-wide n tiles).
SMALL_CASES = [
    W.CONFIGS["tiny_top1"],
    ragged("ragged_a", T=300, H=200, I=136, E=12, k=3, e0=4, E_local=5),
    ragged("ragged_b", T=517, H=264, I=392, E=40, k=6, e0=0, E_local=40, renormalize=0),
    ragged("ragged_c", T=129, H=72, I=24, E=7, k=7, e0=6, E_local=1),
    ragged("single_token", T=1, H=64, I=64, E=9, k=2, e0=0, E_local=9),
    ragged("many_experts", T=257, H=136, I=72, E=1024, k=32, e0=512, E_local=96),
    # k extents multiples of 32 (the direct-to-LDS GEMM path) with ragged n
    # tails and several row blocks per expert
    ragged("dma_ragged_n", T=300, H=192, I=320, E=12, k=3, e0=4, E_local=5),
    ragged("dma_multi_mtile", T=1500, H=256, I=384, E=4, k=2, e0=0, E_local=4),
    ragged("dma_wide_n", T=640, H=576, I=448, E=16, k=4, e0=3, E_local=6, renormalize=0),
    # few rows per expert (T k / E <= 16): the forward's GEMMs take the
    # grouped GEMV; 7 and 5 k-steps (fewer than its ring of loads), ragged
    # 128-column panels at the end of H, experts of one and two 16-row groups;
    # then a skewed router whose hottest local expert needs several 32-row
    # waves per panel; then H off the 32 grid (gate/up on the fallback GEMM,
    # down on the GEMV with an 8-column tail)
    ragged("gemv_ragged", T=120, H=224, I=160, E=40, k=5, e0=5, E_local=12),
    ragged("gemv_hot", T=120, H=224, I=160, E=40, k=5, e0=5, E_local=12, zipf_s=1.0),
    ragged("gemv_mixed", T=40, H=200, I=96, E=6, k=2, e0=1, E_local=4),
    # the GEMV's wave table at its limit: 1024 local experts, most without rows
    ragged("gemv_1024_experts", T=100, H=64, I=64, E=1024, k=4, e0=0, E_local=1024),
    # k extents that end in half a 64-deep stage (H % 64 == I % 64 == 32)
    ragged("dma_half_stage", T=700, H=160, I=224, E=8, k=2, e0=2, E_local=4),
    # few tokens for a long hidden dimension: the router's k range in 4 parts
    # (19 stages of 64: 5 + 5 + 5 + 4)
    ragged("route_parts", T=500, H=1216, I=96, E=40, k=4, e0=8, E_local=8),
    # more tokens than one dispatch workgroup takes, H off the 32 grid: the
    # forward copies rows with placement fused into the copy
    ragged("copy_placed", T=1100, H=200, I=136, E=12, k=3, e0=4, E_local=5),
]


# --------------------------------------------------------------------------- #
# step-by-step runner                                                          #
# --------------------------------------------------------------------------- #
def run_steps(d: DevInputs):
    cfg = d.cfg
    say(f"moe_route {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    logits, idx, w = M.moe_route(d.x, d.w_router, d.bias, cfg.k, cfg.renormalize)
    torch.cuda.synchronize()
    say(f"moe_dispatch {cfg.name} e0={cfg.e0} E_local={cfg.E_local}")
    counts, offsets, perm_src, inv, x_perm = M.moe_dispatch(d.x, idx, cfg.E, cfg.e0, cfg.E_local)
    torch.cuda.synchronize()
    res = dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, perm_src=perm_src, inv=inv,
               x_perm=x_perm)
    if d.w_gate_up is not None:
        say(f"moe_expert_ffn {cfg.name} I={cfg.I}")
        h, out = M.moe_expert_ffn(x_perm, offsets, d.w_gate_up, d.w_down)
        torch.cuda.synchronize()
        say(f"moe_combine {cfg.name}")
        y = M.moe_combine(out, inv, w)
        torch.cuda.synchronize()
        res.update(h=h, out=out, y=y)
    return res


def check_fused_forward(d: DevInputs, y_ref: torch.Tensor) -> None:
    """moe_forward_fused (single-selection tokens combined in the down GEMM's
    epilogue) gives the separate combine's bits; y starts as NaN, so a row
    that neither the epilogue nor the combine wrote would show."""
    cfg = d.cfg
    say(f"moe_forward_fused {cfg.name}")
    y = torch.full((cfg.T, cfg.H), float("nan"), dtype=torch.bfloat16, device=d.x.device)
    M.moe_forward_fused(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), \
        int((y.view(torch.int16) != y_ref.view(torch.int16)).sum())


def check_route(cfg, inp, logits, idx, w):
    """Logits within float32 accuracy of the float64 definition; selection
    and weights exactly / tightly equal to the oracle's on the same logits."""
    gl = logits.cpu().numpy().astype(np.float64)
    ref = O.oracle_logits(inp.x, inp.w_router, inp.bias)
    xa = np.abs(O.bf16_to_f64(inp.x))
    bound = 1e-5 * (xa @ np.abs(inp.w_router.astype(np.float64)).T) + 1e-6
    assert np.all(np.abs(gl - ref) <= bound), float(np.max(np.abs(gl - ref) / bound))
    gi = idx.cpu().numpy()
    ri = O.oracle_topk(gl, cfg.k)
    assert np.array_equal(gi, ri), np.argwhere(gi != ri)[:5]
    rw = O.oracle_weights(gl, ri, cfg.renormalize)
    gw = w.cpu().numpy().astype(np.float64)
    assert np.allclose(gw, rw, rtol=W_RTOL, atol=1e-7), float(np.max(np.abs(gw - rw)))
    # where the float64 logits leave a clear margin, their selection agrees too
    srt = -np.sort(-ref, axis=1)
    if cfg.k < cfg.E:
        margin = srt[:, cfg.k - 1] - srt[:, cfg.k]
        clear = margin > 1e-3
        r64 = O.oracle_topk(ref, cfg.k)
        assert np.array_equal(np.sort(gi[clear], 1), np.sort(r64[clear], 1))
    return gl, gi, gw


def check_dispatch(cfg, inp, gi, res):
    counts, offsets, perm_src, inv = (res[n].cpu().numpy() for n in ("counts", "offsets", "perm_src", "inv"))
    rc = O.oracle_counts(gi, cfg.E)
    ro = O.oracle_offsets(rc, cfg.e0, cfg.E_local)
    rp, rinv = O.oracle_permutation(gi, cfg.e0, cfg.E_local)
    assert np.array_equal(counts, rc)
    assert int(counts.sum()) == cfg.T * cfg.k
    assert np.array_equal(offsets, ro)
    N = int(ro[-1])
    assert np.array_equal(perm_src[:N], rp)
    assert np.array_equal(inv, rinv)
    # x_perm rows are the token vectors, bit for bit (property check on the GPU)
    src = torch.from_numpy(rp.astype(np.int64) // cfg.k).to(res["x_perm"].device)
    xs = res["x_perm"][:N].view(torch.int16)
    ok = torch.equal(xs, to_dev_bf16(inp.x, xs.device).view(torch.int16)[src])
    assert ok, "x_perm differs from x[perm_src // k]"
    return N, ro, rp, rinv


def sample_rows(offsets, per_expert, rng, blocks=()):
    """Rows to check: the first and last rows of each segment, the edges of
    the row blocks the GEMMs cut it into (`blocks`: (first, end) pairs) and
    of the 16-row fragments beside them, and a random draw per segment."""
    rows = set()
    E_local = len(offsets) - 1
    for a, b in blocks:
        rows.update(r for r in (a, a + 1, a + 15, a + 16, b - 17, b - 16, b - 2, b - 1) if a <= r < b)
    for i in range(E_local):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if b <= a:
            continue
        rows.update((a, b - 1))
        if b - a > per_expert:
            rows.update(rng.choice(np.arange(a, b), size=per_expert, replace=False).tolist())
        else:
            rows.update(range(a, b))
    return np.asarray(sorted(rows), dtype=np.int64)


def gemm_blocks(cfg, ro, capacity):
    """Row blocks of both grouped GEMMs of moe_expert_ffn for the realised
    segments (the union of the two launches' splits)."""
    seg = np.diff(np.asarray(ro)).tolist()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    _, b1 = panel_blocks(seg, cfg.I, True, capacity, cus)
    _, b2 = panel_blocks(seg, cfg.H, False, capacity, cus)
    return sorted(set(b1) | set(b2))


def expert_of_rows(offsets, rows):
    return np.searchsorted(np.asarray(offsets), rows, side="right") - 1


def check_ffn(cfg, inp, res, N, ro, rows=None):
    out = res["out"]
    if rows is None:
        rows = np.arange(N)
    if rows.size == 0:
        return
    ex = expert_of_rows(ro, rows)
    sel_dev = torch.from_numpy(rows).to(out.device)
    got = bf16_f64(out[sel_dev])
    got_h = bf16_f64(res["h"][sel_dev])
    xp = bf16_bits(res["x_perm"][sel_dev])
    ref = np.zeros_like(got)
    ref_h = np.zeros_like(got_h)
    for i in np.unique(ex):
        sel = ex == i
        ref_h[sel] = O.oracle_expert_h(xp[sel], inp.w_gate_up[i])
        ref[sel] = O.oracle_expert_mlp(xp[sel], inp.w_gate_up[i], inp.w_down[i])
    # the gate/up GEMM's h on its own, then the expert outputs
    err_h = rel_max_err(got_h, ref_h)
    assert err_h <= OUT_TOL, ("h", err_h)
    err = rel_max_err(got, ref)
    assert err <= OUT_TOL, err


def check_combine(cfg, res, gw, rinv):
    """y against the oracle's combine of the GPU's own expert outputs."""
    y = bf16_f64(res["y"])
    N = int(np.max(rinv)) + 1 if np.any(rinv >= 0) else 0
    outs = bf16_bits(res["out"][:max(N, 1)])
    ref = O.oracle_combine(outs, rinv, gw, cfg.T, cfg.k)
    assert rel_max_err(y, ref) <= OUT_TOL
    none = ~(rinv.reshape(cfg.T, cfg.k) >= 0).any(1)
    assert np.all(y[none] == 0.0)


# --------------------------------------------------------------------------- #
# tests                                                                        #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("T,H,E", [(192, 136, 70), (192, 1216, 70), (100, 7168, 256), (1000, 1216, 70),
                                   (2500, 1216, 70)])
def test_mfma_router_split_is_exact(T, H, E):
    """One-hot tokens make each logit a single product x*w = w, so the three
    bf16 parts must add back to the float32 router weight exactly (and every
    other k part of a split sum adds zeros). The k-split cases cover both
    cuts: in registers for a few token tiles (T <= 2048; 64-token tiles up to
    T = 512, 256-token tiles at T = 1000), through the plane pass beyond
    (T = 2500: 10 tiles of 256 tokens, 4 parts)."""
    dev = device()
    rng = np.random.default_rng(5)
    xf = np.zeros((T, H), np.float32)
    hsel = rng.integers(0, H, size=T)
    xf[np.arange(T), hsel] = 1.0
    x = W.bf16_bits_from_f32(xf)
    wr = (rng.standard_normal((E, H)) * np.exp(rng.uniform(-20, 20, (E, H)))).astype(np.float32)
    say(f"moe_route split exactness T={T} H={H} E={E}")
    logits, idx, w = M.moe_route(to_dev_bf16(x, dev), to_dev(wr, dev), None, 3, True)
    gl = logits.cpu().numpy()
    assert np.array_equal(gl, wr[:, hsel].T), np.argwhere(gl != wr[:, hsel].T)[:4]


@pytest.mark.parametrize("cfg", SMALL_CASES, ids=lambda c: c.name)
def test_small_case_all_steps(cfg):
    """Every step, every element, on problems the oracle finishes at once."""
    dev = device()
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    res = run_steps(d)
    gl, gi, gw = check_route(cfg, inp, res["logits"], res["idx"], res["w"])
    N, ro, rp, rinv = check_dispatch(cfg, inp, gi, res)
    check_ffn(cfg, inp, res, N, ro)
    check_combine(cfg, res, gw, rinv)
    # end to end against the oracle (routing on the GPU's float32 logits)
    y_ref = O.oracle_forward(inp.x, inp.w_router, inp.bias, inp.w_gate_up, inp.w_down, cfg.k, cfg.e0,
                             cfg.E_local, cfg.renormalize, logits=gl)
    assert rel_max_err(bf16_f64(res["y"]), y_ref) <= OUT_TOL
    # the whole-share entry point gives the same bits as the four steps
    say(f"moe_forward {cfg.name}")
    y, _ = M.moe_forward(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), res["y"].view(torch.int16))
    check_fused_forward(d, res["y"])


def test_identity_experts_return_tokens_unchanged():
    """Tiny top-1 workload with identity experts (combine applied to the
    dispatched rows): every token comes back bit for bit in its place."""
    dev = device()
    cfg = W.CONFIGS["tiny_top1"]
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    say("identity round trip tiny_top1")
    _, idx, w = M.moe_route(d.x, d.w_router, None, 1, True)
    assert torch.all(w == 1.0)
    counts, offsets, perm_src, inv, x_perm = M.moe_dispatch(d.x, idx, cfg.E, 0, cfg.E)
    y = M.moe_combine(x_perm, inv, w)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), d.x.view(torch.int16))
    assert int(counts.sum()) == cfg.T


@pytest.mark.parametrize("fixture", ["walkthrough_top1_4tok.json", "imbalance_top1_8tok.json"])
def test_pages_dispatch_examples(fixture):
    """The pages' top-1 walk-through and imbalance example through the GPU
    router (unit router rows, one-hot tokens) and dispatch, for every share."""
    dev = device()
    g = P.load_golden(fixture)
    want = [r[0] for r in g["topk_idx"]]
    T, E, H = len(want), g["E"], 64
    xf = np.zeros((T, H), np.float32)
    for t in range(T):
        xf[t, want[t]] = 1.0
        xf[t, 8:16] = np.arange(8) * 0.25 + t
    x = to_dev_bf16(W.bf16_bits_from_f32(xf), dev)
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), np.arange(E)] = 1.0
    say(f"pages example {fixture}")
    _, idx, w = M.moe_route(x, to_dev(wr, dev), None, 1, True)
    assert idx.cpu().numpy().tolist() == g["topk_idx"]
    for s in g["shares"]:
        counts, offsets, perm_src, inv, x_perm = M.moe_dispatch(x, idx, E, s["e0"], s["E_local"])
        torch.cuda.synchronize()
        assert counts.cpu().tolist() == g["counts"]
        assert offsets.cpu().tolist() == s["offsets"]
        n = s["offsets"][-1]
        assert perm_src[:n].cpu().tolist() == s["perm_src"]
        assert inv.cpu().tolist() == s["inv"]
        y = M.moe_combine(x_perm, inv, w)
        yb = bf16_f64(y)
        for t in range(T):
            local = s["e0"] <= want[t] < s["e0"] + s["E_local"]
            assert np.array_equal(yb[t], xf[t] if local else np.zeros(H))


@pytest.mark.parametrize("E,k,renorm,T", [(4, 4, 1, 128), (100, 7, 0, 128), (256, 8, 1, 128), (1000, 32, 1, 128),
                                          (1024, 1, 0, 128), (32, 4, 0, 2100), (64, 16, 1, 2048), (128, 5, 0, 2100),
                                          (256, 16, 0, 2048), (256, 8, 1, 2099), (128, 8, 1, -2100)])
def test_topk_ties_and_edges(E, k, renorm, T):
    """Selection with many exactly equal logits (ties go to the lowest expert
    id), signed zeros, experts pushed to -inf by the bias, E not a multiple of
    64 and the largest E and k. Logits are set exactly: token t's x is the
    one-hot vector at position t % H, so logit[t, e] = w_router[e, t % H] +
    bias[e]. E = 32, 64, 128, 256 with k <= 16 and T >= 2048 take the kernel
    with one 16-lane row per token (T = 2099: the last wave holds three
    tokens). A negative T means |T| tokens with the bias one float past a
    16-byte boundary (element loads instead of vector loads)."""
    dev = device()
    H = 128
    bias_off = T < 0
    T = abs(T)
    rng = np.random.default_rng(E * 100 + k + 7 * T + bias_off)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    wr = vals[rng.integers(0, len(vals), size=(E, H))]
    bias = np.zeros(E, np.float32)
    bias[rng.choice(E, size=E // 4, replace=False)] = -np.inf
    hot = np.arange(T) % H
    xf = np.zeros((T, H), np.float32)
    xf[np.arange(T), hot] = 1.0
    say(f"topk ties E={E} k={k} renorm={renorm}")
    bias_d = to_dev(np.concatenate([np.zeros(1, np.float32), bias]), dev)[1:] if bias_off else to_dev(bias, dev)
    logits, idx, w = M.moe_route(to_dev_bf16(W.bf16_bits_from_f32(xf), dev), to_dev(wr, dev), bias_d, k,
                                 bool(renorm))
    lg = logits.cpu().numpy()
    want_l = wr[:, hot].T.astype(np.float64) + bias[None, :]
    assert np.array_equal(lg, want_l.astype(np.float32))
    want_idx = O.oracle_topk(lg, k)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    want_w = O.oracle_weights(lg, want_idx, renorm)
    assert np.allclose(w.cpu().numpy(), want_w, rtol=1e-5, atol=1e-7)


def test_pages_top2_and_top4_shares():
    """Top-2 (0.7, 0.3) and top-4 ([0.3, 0.25, 0.25, 0.2], tie 7/15) examples:
    GPU router picks and weights, and each rank share keeps its own terms."""
    dev = device()
    for fixture, E, El in [("top2_weighted_sum.json", 4, 2), ("top4_partial_sums.json", 32, 4)]:
        g = P.load_golden(fixture)
        k, sel, wts = g["k"], g["selected"], g["weights"]
        H = 64
        # logits ln(p) on the selected experts, -20 elsewhere, realised as
        # x = one-hot(0) * 1 and router column 0 = desired logits
        lg = np.full(E, -20.0, np.float32)
        lg[sel] = np.log(np.asarray(wts, np.float32))
        xf = np.zeros((1, H), np.float32)
        xf[0, 0] = 1.0
        wr = np.zeros((E, H), np.float32)
        wr[:, 0] = lg
        say(f"pages example {fixture}")
        _, idx, w = M.moe_route(to_dev_bf16(W.bf16_bits_from_f32(xf), dev), to_dev(wr, dev), None, k, True)
        assert idx.cpu().numpy().tolist() == [sel]
        assert np.allclose(w.cpu().numpy()[0], wts, rtol=1e-6, atol=1e-7)
        # every share's inverse index holds exactly its own selected slots
        for r in range(E // El):
            _, _, _, inv, _ = M.moe_dispatch(to_dev_bf16(W.bf16_bits_from_f32(xf), dev), idx, E, r * El, El)
            loc = [j for j, e in enumerate(sel) if r * El <= e < (r + 1) * El]
            assert [j for j, v in enumerate(inv.cpu().tolist()) if v >= 0] == loc


def test_sum_of_rank_shares_equals_all_local():
    """Running every rank's share (e0 = r*E_local) and adding the outputs gives
    the all-local output (the pages' single all-reduce / reduce-scatter)."""
    dev = device()
    cfg = W.MoEConfig("shares", T=333, H=128, I=96, E=16, k=4, e0=0, E_local=16)
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    say("sum of shares T=333 E=16 k=4")
    y_all, _ = M.moe_forward(d.x, d.w_router, None, d.w_gate_up, d.w_down, cfg.k, 0)
    for El in (2, 4, 8):
        tot = torch.zeros_like(y_all, dtype=torch.float32)
        for r in range(cfg.E // El):
            y_r, _ = M.moe_forward(d.x, d.w_router, None, d.w_gate_up[r * El:(r + 1) * El].contiguous(),
                                   d.w_down[r * El:(r + 1) * El].contiguous(), cfg.k, r * El)
            tot += y_r.float()
        torch.cuda.synchronize()
        assert rel_max_err(tot.cpu().numpy(), bf16_f64(y_all)) <= OUT_TOL


def test_deterministic_and_row_independent():
    """Two runs give identical bits; permuting the tokens permutes the output
    rows bit for bit (no cross-token mixing, no atomics on the float path)."""
    dev = device()
    cfg = W.MoEConfig("perm", T=700, H=256, I=192, E=24, k=5, e0=8, E_local=8)
    inp = W.make_inputs(cfg)
    d = DevInputs(inp, dev)
    say("determinism / permutation T=700")
    y1, _ = M.moe_forward(d.x, d.w_router, None, d.w_gate_up, d.w_down, cfg.k, cfg.e0)
    y2, _ = M.moe_forward(d.x, d.w_router, None, d.w_gate_up, d.w_down, cfg.k, cfg.e0)
    p = torch.from_numpy(np.random.default_rng(3).permutation(cfg.T)).to(dev)
    yp, _ = M.moe_forward(d.x[p].contiguous(), d.w_router, None, d.w_gate_up, d.w_down, cfg.k, cfg.e0)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(yp.view(torch.int16), y1[p].view(torch.int16))


@pytest.mark.parametrize("T,E,k,e0,E_local", [(700, 40, 4, 8, 8), (1100, 24, 5, 4, 12), (2048, 8, 2, 0, 8),
                                               (2049, 16, 3, 2, 9)])
def test_forward_tables_match_oracle(T, E, k, e0, E_local):
    """The dispatch tables moe_forward builds in its workspace (one workgroup
    in one or two rounds of 1024 tokens up to T = 2048, three kernels above)
    equal the oracle's stable permutation on the forward's own top-k ids."""
    dev = device()
    cfg = W.MoEConfig(f"tables{T}", T=T, H=64, I=64, E=E, k=k, e0=e0, E_local=E_local)
    d = DevInputs(W.make_inputs(cfg), dev)
    ws = torch.empty(M.forward_workspace_size(T, cfg.H, cfg.I, E, k, E_local), dtype=torch.uint8, device=dev)
    say(f"moe_forward tables T={T} E={E} k={k} e0={e0} E_local={E_local}")
    M.moe_forward(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, k, e0, cfg.renormalize, workspace=ws)
    torch.cuda.synchronize()
    lay = M.forward_workspace_layout(T, cfg.H, cfg.I, E, k, E_local)
    host = ws.cpu().numpy()

    def i32(name, n):
        return host[lay[name]:lay[name] + 4 * n].view(np.int32)

    idx = i32("topk_idx", T * k).reshape(T, k)
    rc = O.oracle_counts(idx, E)
    ro = O.oracle_offsets(rc, e0, E_local)
    rp, rinv = O.oracle_permutation(idx, e0, E_local)
    assert np.array_equal(i32("counts", E), rc)
    assert np.array_equal(i32("offsets", E_local + 1), ro)
    N = int(ro[-1])
    assert np.array_equal(i32("perm_src", N), rp)
    assert np.array_equal(i32("inv", T * k), rinv)


def test_empty_batch_is_noop():
    dev = device()
    cfg = W.MoEConfig("empty", T=0, H=64, I=64, E=4, k=2, e0=0, E_local=4)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    wr = torch.randn(4, 64, device=dev)
    gu = torch.zeros((4, 64, 128), dtype=torch.bfloat16, device=dev)
    dn = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    say("empty batch")
    y, _ = M.moe_forward(x, wr, None, gu, dn, cfg.k, 0)
    assert y.shape == (0, 64)


# --------------------------------------------------------------------------- #
# the named workloads at their full sizes                                       #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("name", ["small_top2", "gptoss20b_ep8_share", "gptoss20b_ep2_tp4_share", "dsr1_ep8_share",
                                  "dsr1_ep8_decode", "gptoss20b_ep8_decode", "dsr1_ep8_share_zipf"])
def test_named_workload_full_size(name):
    cfg = W.CONFIGS[name]
    dev = device()
    inp = inputs_for(cfg)
    d = DevInputs(inp, dev)
    res = run_steps(d)
    gl, gi, gw = check_route(cfg, inp, res["logits"], res["idx"], res["w"])
    N, ro, rp, rinv = check_dispatch(cfg, inp, gi, res)
    rng = np.random.default_rng(7)
    rows = np.arange(N) if N <= 4096 else sample_rows(ro, 12, rng, gemm_blocks(cfg, ro, res["x_perm"].shape[0]))
    check_ffn(cfg, inp, res, N, ro, rows)
    check_combine(cfg, res, gw, rinv)
    say(f"moe_forward {name}")
    y, _ = M.moe_forward(d.x, d.w_router, d.bias, d.w_gate_up, d.w_down, cfg.k, cfg.e0, cfg.renormalize)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), res["y"].view(torch.int16))
    check_fused_forward(d, res["y"])
    # sampled tokens end to end against the oracle's definition
    toks = rng.choice(cfg.T, size=min(cfg.T, 48), replace=False)
    yref = np.zeros((toks.size, cfg.H))
    xs = O.bf16_to_f64(inp.x[toks])
    for n, t in enumerate(toks):
        for j in range(cfg.k):
            e = int(gi[t, j])
            if cfg.e0 <= e < cfg.e0 + cfg.E_local:
                i = e - cfg.e0
                yref[n] += gw[t, j] * O.oracle_expert_mlp(xs[n:n + 1], inp.w_gate_up[i], inp.w_down[i])[0]
    assert rel_max_err(bf16_f64(y[torch.from_numpy(toks).to(dev)]), yref) <= OUT_TOL
    if cfg.zipf_s > 0:
        local = res["counts"].cpu().numpy()[cfg.e0:cfg.e0 + cfg.E_local]
        mean = cfg.T * cfg.k / cfg.E
        assert local.max() >= 20 * mean, local.max()
        assert (local == 0).any()
