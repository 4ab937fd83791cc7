"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them."""
import numpy as np
import pytest

import oracle.moe_oracle as O
from tests import oracle_pins as P

_orig = {name: getattr(O, name) for name in dir(O) if name.startswith("oracle_")}


def _logits_no_bias(x, w_router, bias=None):
    return O._f64(x) @ O._f64(w_router).T


def _logits_bias_sub(x, w_router, bias=None):
    ell = O._f64(x) @ O._f64(w_router).T
    return ell - (0 if bias is None else O._f64(bias)[None, :])


def _topk_ties_high(logits, k):
    ell = np.asarray(logits, np.float64)
    order = np.argsort(ell, axis=1, kind="stable")[:, ::-1]
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def _topk_smallest(logits, k):
    return np.argsort(np.asarray(logits), axis=1, kind="stable")[:, :k].astype(np.int32)


def _weights_never_renorm(logits, idx, renormalize):
    return _orig["oracle_weights"](logits, idx, 0)


def _weights_always_renorm(logits, idx, renormalize):
    return _orig["oracle_weights"](logits, idx, 1)


def _weights_no_max_shift_wrong_axis(logits, idx, renormalize):
    ell = np.asarray(logits, np.float64)
    z = np.exp(ell - ell.max(axis=0, keepdims=True))
    z = z / z.sum(axis=0, keepdims=True)
    sel = np.take_along_axis(z, np.asarray(idx, np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True) if renormalize else sel


def _perm_swapped(idx, e0, E_local):
    p, inv = _orig["oracle_permutation"](idx, e0, E_local)
    n = p.shape[0]
    inv2 = np.full_like(inv, -1)
    # return the inverse table in place of the permutation and vice versa
    return inv[inv >= 0][:n].astype(np.int32), np.where(inv >= 0, inv, -1).astype(np.int32)[::-1].copy()


def _perm_unstable(idx, e0, E_local):
    flat = np.asarray(idx).ravel()
    segs = [np.nonzero(flat == e0 + i)[0][::-1] for i in range(E_local)]
    p = np.concatenate(segs).astype(np.int32) if segs else np.zeros(0, np.int32)
    inv = np.full(flat.shape[0], -1, np.int32)
    inv[p] = np.arange(p.shape[0], dtype=np.int32)
    return p, inv


def _offsets_global_index(counts, e0, E_local):
    off = np.zeros(E_local + 1, np.int64)
    for i in range(E_local):
        off[i + 1] = off[i] + int(counts[i])
    return off.astype(np.int32)


def _counts_local_only(idx, E):
    c = _orig["oracle_counts"](idx, E)
    c[E // 2:] = 0
    return c


def _mlp_gate_up_swapped(xrows, w_gate_up, w_down):
    W = O._f64(w_gate_up)
    I = W.shape[1] // 2
    return _orig["oracle_expert_mlp"](xrows, np.concatenate([W[:, I:], W[:, :I]], axis=1), w_down)


def _mlp_interleaved(xrows, w_gate_up, w_down):
    W = O._f64(w_gate_up)
    return _orig["oracle_expert_mlp"](xrows, np.concatenate([W[:, 0::2], W[:, 1::2]], axis=1), w_down)


def _h_gate_up_swapped(xrows, w_gate_up):
    W = O._f64(w_gate_up)
    I = W.shape[1] // 2
    return _orig["oracle_expert_h"](xrows, np.concatenate([W[:, I:], W[:, :I]], axis=1))


def _h_no_up(xrows, w_gate_up):
    W = O._f64(w_gate_up)
    I = W.shape[1] // 2
    return O.oracle_silu(O._f64(xrows) @ W[:, :I])


def _h_silu_of_product(xrows, w_gate_up):
    W = O._f64(w_gate_up)
    I = W.shape[1] // 2
    X = O._f64(xrows)
    return O.oracle_silu((X @ W[:, :I]) * (X @ W[:, I:]))


def _silu_sigmoid(z):
    z = np.asarray(z, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _silu_sign(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(z))


def _ffn_expert_shift(x_perm, offsets, w_gate_up, w_down):
    El = np.asarray(offsets).shape[0] - 1
    order = [(i + 1) % El for i in range(El)]
    return _orig["oracle_expert_ffn"](x_perm, offsets, np.asarray(w_gate_up)[order],
                                      np.asarray(w_down)[order])


def _combine_no_weights(expert_out, inv, topk_w, T, k):
    return _orig["oracle_combine"](expert_out, inv, np.ones_like(np.asarray(topk_w, np.float64)), T, k)


def _combine_slot_reversed(expert_out, inv, topk_w, T, k):
    w = np.asarray(topk_w, np.float64).reshape(T, k)[:, ::-1]
    return _orig["oracle_combine"](expert_out, inv, np.ascontiguousarray(w), T, k)


def _gather_wrong_div(x, perm_src, k):
    return np.asarray(x)[np.asarray(perm_src, np.int64) % max(1, np.asarray(x).shape[0])]


def _decode_truncating(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return np.abs(b.view(np.float32).astype(np.float64))


MUTANTS = {
    "logits: bias dropped": ("oracle_logits", _logits_no_bias),
    "logits: bias sign": ("oracle_logits", _logits_bias_sub),
    "topk: ties to higher id": ("oracle_topk", _topk_ties_high),
    "topk: smallest logits": ("oracle_topk", _topk_smallest),
    "weights: never renormalised": ("oracle_weights", _weights_never_renorm),
    "weights: always renormalised": ("oracle_weights", _weights_always_renorm),
    "weights: softmax over tokens": ("oracle_weights", _weights_no_max_shift_wrong_axis),
    "dispatch: perm/inverse swapped": ("oracle_permutation", _perm_swapped),
    "dispatch: unstable segment order": ("oracle_permutation", _perm_unstable),
    "dispatch: offsets from global ids": ("oracle_offsets", _offsets_global_index),
    "dispatch: remote counts dropped": ("oracle_counts", _counts_local_only),
    "dispatch: gather with modulo": ("oracle_gather", _gather_wrong_div),
    "mlp: gate and up swapped": ("oracle_expert_mlp", _mlp_gate_up_swapped),
    "mlp: interleaved gate/up": ("oracle_expert_mlp", _mlp_interleaved),
    "h: gate and up swapped": ("oracle_expert_h", _h_gate_up_swapped),
    "h: up projection dropped": ("oracle_expert_h", _h_no_up),
    "h: silu of the product": ("oracle_expert_h", _h_silu_of_product),
    "mlp: sigmoid instead of silu": ("oracle_silu", _silu_sigmoid),
    "mlp: silu sign": ("oracle_silu", _silu_sign),
    "ffn: experts shifted": ("oracle_expert_ffn", _ffn_expert_shift),
    "combine: weights ignored": ("oracle_combine", _combine_no_weights),
    "combine: slot weights reversed": ("oracle_combine", _combine_slot_reversed),
    "decode: sign lost": ("bf16_to_f64", _decode_truncating),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception as exc:      # AssertionError, or a shape error from the mistake
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"no pin caught the mutant '{name}'"
