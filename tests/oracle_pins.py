"""Checks that tie the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages print (worked examples under ``tests/golden``), with a closed
form, or with a brute-force computation written here in plain Python. The
functions look the oracle up at call time, so ``test_oracle_mutants`` can
plant a plausible mistake in the oracle and check that some pin fails.
"""
from __future__ import annotations

import json
import math
import pathlib

import numpy as np

import oracle.moe_oracle as O

GOLDEN = pathlib.Path(__file__).parent / "golden"


def load_golden(name: str) -> dict:
    with open(GOLDEN / name) as f:
        return json.load(f)


# --------------------------------------------------------------------------- #
# helpers written independently of the oracle                                  #
# --------------------------------------------------------------------------- #
def py_silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def py_topk(row, k):
    """Largest first, lower expert id first among equal values (brute force)."""
    return sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]


def bits_of_f32(a) -> np.ndarray:
    """bfloat16 bits of float32 values that are exactly representable in bf16."""
    b = np.asarray(a, dtype=np.float32).view(np.uint32)
    assert np.all((b & np.uint32(0xFFFF)) == 0), "value not exact in bfloat16"
    return (b >> np.uint32(16)).astype(np.uint16)


def routing_logits_from_probs(T, E, picks, probs, floor=-60.0):
    """Logits whose softmax over the picked experts reproduces ``probs``."""
    ell = np.full((T, E), floor, dtype=np.float64)
    for t in range(T):
        for e, p in zip(picks[t], probs[t]):
            ell[t, e] = math.log(p)
    return ell


def identity_experts(E_local, H, scales):
    """gate = c_i * Id, up = Id, down = Id (I = H): expert i maps x to
    silu(c_i x) * x elementwise."""
    w_gu = np.zeros((E_local, H, 2 * H), dtype=np.float64)
    w_d = np.zeros((E_local, H, H), dtype=np.float64)
    for i in range(E_local):
        for h in range(H):
            w_gu[i, h, h] = scales[i]
            w_gu[i, h, H + h] = 1.0
            w_d[i, h, h] = 1.0
    return w_gu, w_d


def _dispatch_checks(g, idx):
    counts = O.oracle_counts(idx, g["E"])
    assert counts.tolist() == g["counts"], (counts, g["counts"])
    for s in g["shares"]:
        offsets = O.oracle_offsets(counts, s["e0"], s["E_local"])
        perm_src, inv = O.oracle_permutation(idx, s["e0"], s["E_local"])
        assert offsets.tolist() == s["offsets"], (s["name"], offsets, s["offsets"])
        assert perm_src.tolist() == s["perm_src"], (s["name"], perm_src, s["perm_src"])
        assert inv.tolist() == s["inv"], (s["name"], inv, s["inv"])
        if "rows" in s:
            assert int(offsets[-1]) == s["rows"]


# --------------------------------------------------------------------------- #
# pins from the pages' worked examples                                         #
# --------------------------------------------------------------------------- #
def pin_walkthrough_top1():
    """Four tokens, four experts, top-1, weight one: routing realised through
    the router (unit-vector router rows, one-hot tokens), dispatch tables as
    the example states, and identity experts give every token back unchanged
    in its original order."""
    g = load_golden("walkthrough_top1_4tok.json")
    T, E, k, H = len(g["tokens"]), g["E"], g["k"], 8
    want = [r[0] for r in g["topk_idx"]]
    xf = np.zeros((T, H), np.float32)
    for t in range(T):
        xf[t, want[t]] = 1.0
        xf[t, 4:] = [0.5 * (t + 1), -0.25 * (t + 1), 0.125 * (t + 2), -2.0 * (t + 1)]
    x = bits_of_f32(xf)
    wr = np.zeros((E, H), np.float32)
    for e in range(E):
        wr[e, e] = 1.0
    ell, idx, w = O.oracle_route(x, wr, None, k, 1)
    assert idx.tolist() == g["topk_idx"], idx
    assert np.array_equal(w, np.asarray(g["topk_w"])), w
    _dispatch_checks(g, idx)
    # identity experts: combine(dispatch(x)) is x, bit for bit, in token order
    for s in g["shares"]:
        counts, offsets, perm_src, inv, x_perm = O.oracle_dispatch(x, idx, E, s["e0"], s["E_local"])
        assert x_perm.dtype == np.uint16
        assert np.array_equal(x_perm, x[np.asarray(s["perm_src"], np.int64)])
        y = O.oracle_combine(x_perm, inv, w, T, k)
        for t in range(T):
            local = s["e0"] <= want[t] < s["e0"] + s["E_local"]
            expect = xf[t].astype(np.float64) if local else np.zeros(H)
            assert np.array_equal(y[t], expect), (s["name"], t, y[t], expect)


def pin_imbalance_top1():
    """Eight tokens, E2 takes six: the permutation is not an involution, so
    this tells the permutation from its inverse; the two ranks' row counts
    are 2 and 6."""
    g = load_golden("imbalance_top1_8tok.json")
    idx = np.asarray(g["topk_idx"], np.int32)
    _dispatch_checks(g, idx)
    x = np.arange(len(g["tokens"]) * 4, dtype=np.uint16).reshape(-1, 4) + np.uint16(0x3F00)
    for s in g["shares"]:
        _, _, perm_src, inv, x_perm = O.oracle_dispatch(x, idx, g["E"], s["e0"], s["E_local"])
        for n, src in enumerate(s["perm_src"]):
            assert np.array_equal(x_perm[n], x[src]), (s["name"], n)


def pin_top2_weighted_sum():
    """y(A2) = 0.7 u0 + 0.3 u2, and each rank keeps only its own term."""
    g = load_golden("top2_weighted_sum.json")
    E, k, H = g["E"], g["k"], 4
    ell = routing_logits_from_probs(1, E, [g["selected"]], [g["weights"]])
    ell[0, 1], ell[0, 3] = -40.0, -45.0
    idx = O.oracle_topk(ell, k)
    assert idx.tolist() == [g["selected"]], idx
    w = O.oracle_weights(ell, idx, 1)
    assert np.allclose(w[0], g["weights"], rtol=0, atol=1e-15), w
    scales = [0.5, -1.0, 2.0, 3.0]
    xrow = [0.75, -1.5, 0.25, 2.0]
    x = np.asarray([xrow], np.float64)
    w_gu, w_d = identity_experts(E, H, scales)

    def u(e):
        return [py_silu(scales[e] * v) * v for v in xrow]

    full = O.oracle_forward(x, np.eye(E, H), None, w_gu, w_d, k, 0, E, 1, logits=ell)
    expect = [0.7 * a + 0.3 * b for a, b in zip(u(0), u(2))]
    assert np.allclose(full[0], expect, rtol=1e-13, atol=1e-15), (full, expect)
    for s in g["shares"]:
        e0, El = s["e0"], s["E_local"]
        y = O.oracle_forward(x, np.eye(E, H), None, w_gu[e0:e0 + El], w_d[e0:e0 + El], k, e0, El, 1,
                             logits=ell)
        expect = np.zeros(H)
        for e, wt in s["terms"]:
            expect += wt * np.asarray(u(e))
        assert np.allclose(y[0], expect, rtol=1e-13, atol=1e-15), (s["name"], y, expect)


def pin_top4_partial_sums():
    """Experts [2, 7, 15, 28] with [0.3, 0.25, 0.25, 0.2]: the exact 7/15 tie
    goes to the lower id first, and over the 8 ranks of 4 experts each, each
    owning rank contributes exactly its one weighted term."""
    g = load_golden("top4_partial_sums.json")
    E, k, El, H = g["E"], g["k"], g["E_local"], 3
    ell = routing_logits_from_probs(1, E, [g["selected"]], [g["weights"]])
    idx = O.oracle_topk(ell, k)
    assert idx.tolist() == [g["selected"]], idx
    w = O.oracle_weights(ell, idx, 1)
    assert np.allclose(w[0], g["weights"], rtol=0, atol=1e-15), w
    xrow = [1.25, -0.5, 3.0]
    x = np.asarray([xrow])
    scales = [0.1 * (e + 1) * (-1) ** e for e in range(E)]
    w_gu, w_d = identity_experts(E, H, scales)
    total = np.zeros(H)
    for r in range(E // El):
        e0 = r * El
        y = O.oracle_forward(x, np.eye(E, H), None, w_gu[e0:e0 + El], w_d[e0:e0 + El], k, e0, El, 1,
                             logits=ell)
        expect = np.zeros(H)
        for e, wt in g["rank_terms"][str(r)]:
            expect += wt * np.asarray([py_silu(scales[e] * v) * v for v in xrow])
        assert np.allclose(y[0], expect, rtol=1e-13, atol=1e-15), (r, y, expect)
        total += y[0]
    full = O.oracle_forward(x, np.eye(E, H), None, w_gu, w_d, k, 0, E, 1, logits=ell)
    assert np.allclose(total, full[0], rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------- #
# closed forms, invariants and brute force                                     #
# --------------------------------------------------------------------------- #
def pin_logits_bruteforce():
    """Affinities against math.fsum over the products (non-square shapes,
    non-zero bias)."""
    rng = np.random.default_rng(11)
    T, H, E = 5, 7, 3
    xf = rng.standard_normal((T, H)).astype(np.float32)
    x = bits_of_f32((xf.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32))
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(float)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    ell = O.oracle_logits(x, wr, b)
    assert ell.shape == (T, E)
    for t in range(T):
        for e in range(E):
            ref = math.fsum([xv[t, h] * float(wr[e, h]) for h in range(H)] + [float(b[e])])
            assert abs(ell[t, e] - ref) <= 1e-12 * max(1.0, abs(ref)), (t, e, ell[t, e], ref)


def pin_topk_bruteforce():
    """Top-k against a plain Python sort, with exact ties forced by duplicate
    router rows (identical dot products) and by repeated logit values."""
    rng = np.random.default_rng(12)
    T, H, E = 40, 16, 12
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H))
    wr[5] = wr[2]
    wr[9] = wr[2]
    wr[11] = wr[0]
    ell = O.oracle_logits(x, wr)
    ell[::3] = np.round(ell[::3])          # many exact ties
    for k in (1, 2, 3, 5, E):
        idx = O.oracle_topk(ell, k)
        for t in range(T):
            assert idx[t].tolist() == py_topk(ell[t].tolist(), k), (k, t)


def pin_softmax_closed_form():
    """Logits ln[1, 2, 3, 4]: probabilities 0.1..0.4; top-2 is experts 3, 2
    with weights 4/7, 3/7 renormalised and 0.4, 0.3 without; top-1
    renormalised weighs exactly 1."""
    ell = np.log(np.asarray([[1.0, 2.0, 3.0, 4.0], [4.0, 3.0, 2.0, 1.0]]))
    idx = O.oracle_topk(ell, 2)
    assert idx.tolist() == [[3, 2], [0, 1]]
    w = O.oracle_weights(ell, idx, 1)
    assert np.allclose(w, [[4 / 7, 3 / 7]] * 2, rtol=0, atol=1e-15), w
    w = O.oracle_weights(ell, idx, 0)
    assert np.allclose(w, [[0.4, 0.3]] * 2, rtol=0, atol=1e-15), w
    rng = np.random.default_rng(13)
    ell = rng.standard_normal((50, 9)) * 4
    idx1 = O.oracle_topk(ell, 1)
    assert np.all(O.oracle_weights(ell, idx1, 1) == 1.0)
    for k in (2, 4, 9):
        w = O.oracle_weights(ell, O.oracle_topk(ell, k), 1)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
        assert np.all(np.diff(w, axis=1) <= 0)    # slots in descending weight
    wall = O.oracle_weights(ell, O.oracle_topk(ell, 9), 0)
    assert np.allclose(wall.sum(1), 1.0, rtol=0, atol=1e-15)


def pin_ffn_closed_form():
    """gate = c_i Id, up = Id, down = Id: expert i returns silu(c_i x) * x,
    with a different c_i per expert (catches gate/up swaps and experts
    applied to the wrong segment)."""
    rng = np.random.default_rng(14)
    H, El = 6, 3
    scales = [0.5, -2.0, 1.5]
    w_gu, w_d = identity_experts(El, H, scales)
    counts = [3, 0, 4]
    offsets = np.cumsum([0] + counts)
    xp = rng.standard_normal((offsets[-1], H))
    out = O.oracle_expert_ffn(xp, offsets, w_gu, w_d)
    for i in range(El):
        for n in range(offsets[i], offsets[i + 1]):
            want = [py_silu(scales[i] * v) * v for v in xp[n]]
            assert np.allclose(out[n], want, rtol=1e-14, atol=1e-15), (i, n)


def pin_ffn_hand_example():
    """H = 2, I = 1 worked by hand: x = [1, 2], gate column [1, 0] gives g = 1,
    up column [0, 1] gives u = 2, h = silu(1) * 2, down row [3, -1]."""
    x = np.asarray([[1.0, 2.0]])
    w_gu = np.asarray([[1.0, 0.0], [0.0, 1.0]])      # [H=2, 2I=2]: col 0 gate, col 1 up
    w_d = np.asarray([[3.0, -1.0]])                  # [I=1, H=2]
    out = O.oracle_expert_mlp(x, w_gu, w_d)
    h = 2.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(out[0], [3.0 * h, -h], rtol=1e-15, atol=0), out


def pin_expert_h_hand_example():
    """H = 3, I = 2 worked by hand (gate and up blocks of different shapes
    than the down matrix, so a transposed operand cannot pass):
    x = [1, -2, 0.5];
    gate columns [1, 0, 2] and [0, 0, 0] give g = [2, 0];
    up columns [0, 1, 0] and [1, 1, 1] give u = [-2, -0.5];
    h = [silu(2) * -2, silu(0) * -0.5] = [-4 / (1 + e^-2), 0].
    A second row x = [0, 1, 0] gives g = [0, 0], u = [1, 1], h = [0, 0]."""
    x = np.asarray([[1.0, -2.0, 0.5], [0.0, 1.0, 0.0]])
    w_gu = np.asarray([[1.0, 0.0, 0.0, 1.0],
                       [0.0, 0.0, 1.0, 1.0],
                       [2.0, 0.0, 0.0, 1.0]])          # [H=3, 2I=4]: cols 0-1 gate, 2-3 up
    h = O.oracle_expert_h(x, w_gu)
    assert h.shape == (2, 2), h.shape
    want0 = -4.0 / (1.0 + math.exp(-2.0))
    assert math.isclose(h[0, 0], want0, rel_tol=1e-15), h
    assert h[0, 1] == 0.0 and h[1, 0] == 0.0 and h[1, 1] == 0.0, h
    # with gate = up, h = silu(g) * g: g = 2 gives 4 / (1 + e^-2)
    w_same = np.concatenate([w_gu[:, :2], w_gu[:, :2]], axis=1)
    assert math.isclose(O.oracle_expert_h(x[:1], w_same)[0, 0], -want0, rel_tol=1e-15)


def _random_share_problem(seed, T, H, I, E, k, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)) * scale
    wr = rng.standard_normal((E, H))
    w_gu = rng.standard_normal((E, H, 2 * I)) / math.sqrt(H)
    w_d = rng.standard_normal((E, I, H)) / math.sqrt(I)
    return x, wr, w_gu, w_d


def pin_dispatch_invariants():
    """Sum of counts = T*k; ids per token distinct; perm_src and inv are
    inverse to each other; segments hold only their expert's rows, in
    ascending (token, slot) order; offsets are the running count."""
    rng = np.random.default_rng(15)
    for (T, E, k, e0, El) in [(37, 8, 3, 2, 4), (64, 16, 4, 0, 16), (1, 5, 5, 4, 1), (0, 4, 2, 0, 4)]:
        ell = rng.standard_normal((T, E))
        idx = O.oracle_topk(ell, k)
        counts = O.oracle_counts(idx, E)
        assert int(counts.sum()) == T * k
        for t in range(T):
            assert len(set(idx[t].tolist())) == k
        offsets = O.oracle_offsets(counts, e0, El)
        perm_src, inv = O.oracle_permutation(idx, e0, El)
        assert int(offsets[-1]) == perm_src.shape[0] == int(counts[e0:e0 + El].sum())
        assert np.all(np.diff(offsets) >= 0)
        flat = idx.ravel()
        for n, s in enumerate(perm_src):
            assert inv[s] == n
        for s in range(T * k):
            local = e0 <= flat[s] < e0 + El
            assert (inv[s] >= 0) == local
            if local:
                assert perm_src[inv[s]] == s
        for i in range(El):
            seg = perm_src[offsets[i]:offsets[i + 1]]
            assert np.all(flat[seg] == e0 + i)
            assert np.all(np.diff(seg) > 0)


def pin_identity_roundtrip():
    """Identity experts on the tiny top-1 workload shape: combine(dispatch(x))
    returns x bit for bit with all experts local; with top-k the result is
    x * (sum of the local weights)."""
    rng = np.random.default_rng(16)
    T, H, E = 64, 128, 4
    x = (rng.integers(0x3C00, 0x4100, size=(T, H))).astype(np.uint16)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ell = rng.standard_normal((T, E))
    for k, e0, El in [(1, 0, 4), (2, 0, 4), (3, 1, 2)]:
        idx = O.oracle_topk(ell, k)
        w = O.oracle_weights(ell, idx, 1)
        _, _, _, inv, x_perm = O.oracle_dispatch(x, idx, E, e0, El)
        y = O.oracle_combine(x_perm, inv, w, T, k)
        wl = np.where((idx >= e0) & (idx < e0 + El), w, 0.0).sum(1)
        if k == 1 and El == E:
            assert np.array_equal(y, xv)
        else:
            assert np.allclose(y, xv * wl[:, None], rtol=1e-15, atol=0)


def pin_sum_of_shares():
    """Adding the outputs of all rank shares e0 = r*E_local gives the output
    with every expert local."""
    x, wr, w_gu, w_d = _random_share_problem(17, T=23, H=8, I=6, E=8, k=3)
    full = O.oracle_forward(x, wr, None, w_gu, w_d, 3, 0, 8, 1)
    for El in (1, 2, 4):
        tot = np.zeros_like(full)
        for r in range(8 // El):
            e0 = r * El
            tot += O.oracle_forward(x, wr, None, w_gu[e0:e0 + El], w_d[e0:e0 + El], 3, e0, El, 1)
        assert np.allclose(tot, full, rtol=1e-12, atol=1e-14)


def pin_sum_of_ep_tp_shares():
    """Variable EP + TP: rank (r_ep, r_tp) holds experts [r_ep E_L, (r_ep+1) E_L)
    with intermediate slice r_tp of tp (gate and up columns and down rows of
    that slice, as the workload generator cuts them). Summing every rank's
    output gives the layer with whole experts, all local ("Expert Parallelism
    (EP)", "Variable EP (EP+TP for MoE)": one collective sums the TP partial
    products and the EP expert contributions)."""
    import workloads as W
    full = W.MoEConfig("eptp_full", T=21, H=16, I=24, E=8, k=3, e0=0, E_local=8, x_scale=1.0)
    fi = W.make_inputs(full)
    y_full = O.oracle_forward(fi.x, fi.w_router, None, fi.w_gate_up, fi.w_down, 3, 0, 8, 1)
    for ep, tp in [(1, 2), (2, 3), (4, 4), (8, 1)]:
        El = 8 // ep
        tot = np.zeros_like(y_full)
        for r_ep in range(ep):
            for r_tp in range(tp):
                c = full.scaled(I=24 // tp, tp=tp, tp_rank=r_tp, e0=r_ep * El, E_local=El)
                si = W.make_inputs(c)
                assert si.w_gate_up.shape == (El, 16, 2 * (24 // tp))
                tot += O.oracle_forward(si.x, si.w_router, None, si.w_gate_up, si.w_down, 3, c.e0, El, 1)
        assert np.allclose(tot, y_full, rtol=1e-12, atol=1e-14), (ep, tp, float(np.max(np.abs(tot - y_full))))


def pin_dense_equals_grouped():
    """The dispatch / grouped path equals the dense masked evaluation of every
    local expert on every token."""
    for seed, (T, H, I, E, k, e0, El) in enumerate([(19, 8, 5, 6, 2, 0, 6), (16, 4, 4, 8, 3, 2, 4),
                                                   (5, 6, 3, 4, 1, 1, 2)]):
        x, wr, w_gu, w_d = _random_share_problem(100 + seed, T, H, I, E, k)
        r = O.oracle_forward(x, wr, None, w_gu[e0:e0 + El], w_d[e0:e0 + El], k, e0, El, 1,
                             return_all=True)
        yd = O.oracle_dense_forward(x, r["topk_idx"], r["topk_w"], w_gu[e0:e0 + El], w_d[e0:e0 + El],
                                    e0, El)
        assert np.allclose(r["y"], yd, rtol=1e-12, atol=1e-14)


def pin_row_independence():
    """Experts act on each token on its own: permuting the tokens permutes
    the output rows."""
    x, wr, w_gu, w_d = _random_share_problem(18, T=30, H=8, I=4, E=6, k=2)
    y = O.oracle_forward(x, wr, None, w_gu, w_d, 2, 0, 6, 1)
    p = np.random.default_rng(19).permutation(30)
    yp = O.oracle_forward(x[p], wr, None, w_gu, w_d, 2, 0, 6, 1)
    assert np.allclose(yp, y[p], rtol=1e-13, atol=1e-15)


def pin_bf16_decode():
    """Known bfloat16 bit patterns decode to their values."""
    bits = np.asarray([0x3F80, 0xC000, 0x3F00, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0080], np.uint16)
    want = [1.0, -2.0, 0.5, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -126]
    got = O.bf16_to_f64(bits)
    assert got.tolist() == want, got
    assert math.copysign(1.0, got[5]) == -1.0


ALL_PINS = [
    pin_walkthrough_top1, pin_imbalance_top1, pin_top2_weighted_sum, pin_top4_partial_sums,
    pin_logits_bruteforce, pin_topk_bruteforce, pin_softmax_closed_form, pin_ffn_closed_form,
    pin_ffn_hand_example, pin_expert_h_hand_example, pin_dispatch_invariants, pin_identity_roundtrip, pin_sum_of_shares, pin_sum_of_ep_tp_shares,
    pin_dense_equals_grouped, pin_row_independence, pin_bf16_decode,
]
