"""CPU oracle for one expert-parallel rank's share of an MoE layer.

TEST INFRASTRUCTURE ONLY. Nothing in the GPU library imports, calls or links
this module; only the test suite, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the GPU path: it reads raw input
arrays (bfloat16 as uint16 bit patterns, float32 router weights) and decodes
them itself.

Everything is float64 numpy, written as the plain definition of what the layer
computes, step by step, in the order the pages describe it:

1. router logits and top-k selection with combine weights
   ("Expert Parallelism (EP)", AWS Neuron vLLM design doc, sections
   "Router Weights" and "Collective Patterns / Prefill": every rank scores all
   experts from the replicated router, then keeps its local ones);
2. dispatch: local (token, slot) pairs grouped by expert
   ("EP: Partition Experts and Route Tokens", section "Send tokens to experts
   and return their results": token vectors are grouped by selected expert;
   rows of one expert are stacked for one matmul);
3. each local expert's MLP on its rows (gate_up [H, 2I] and down [I, H] per
   expert, "Expert Weight Distribution", weight-shape table);
4. combine: the weighted sum of a token's expert outputs back in the original
   token order ("EP: Partition Experts and Route Tokens", section "Return
   multiple expert results to the same token": y(A2) = 0.7 u0 + 0.3 u2),
   with zeros for tokens that picked no local expert ("Why a Single
   All-Reduce/Reduce-Scatter Works").

Readings taken where the pages are silent (each one is pinned by a test):
* scores: softmax over all E router logits; with ``renormalize`` the k
  selected probabilities are rescaled to sum to one (both worked examples'
  weights sum to one);
* selection is made on the logits; ties go to the lower expert id, and slots
  are ordered by descending logit;
* expert MLP: h = silu(x Wg) * (x Wu) with gate = first I columns of gate_up,
  up = last I; silu(z) = z / (1 + exp(-z)); no biases;
* within an expert's segment rows are in ascending (token, slot) order;
* a rank share uses the global top-k weights (not renormalised over the local
  subset), so summing the shares of all ranks gives the full layer.

Parity pinning: every function here is checked by ``tests/test_oracle_pins.py``
against the pages' worked examples, closed forms and brute force.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "oracle_logits", "oracle_topk", "oracle_weights", "oracle_route",
    "oracle_counts", "oracle_offsets", "oracle_permutation", "oracle_gather",
    "oracle_dispatch", "oracle_silu", "oracle_expert_h", "oracle_expert_mlp", "oracle_expert_ffn",
    "oracle_combine", "oracle_forward", "oracle_dense_forward",
]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64: a bfloat16 is
    the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


# --------------------------------------------------------------------------- #
# 1. Router                                                                    #
# --------------------------------------------------------------------------- #
def oracle_logits(x, w_router, bias=None) -> np.ndarray:
    """Affinities of every token for every expert: l[t, e] = sum_h x[t,h] W_r[e,h] + b[e].

    "Expert Parallelism (EP)", section "Collective Patterns / Prefill", step 1:
    [T, H] @ [H, E] gives [T, E] affinities for all experts."""
    ell = _f64(x) @ _f64(w_router).T
    if bias is not None:
        ell = ell + _f64(bias)[None, :]
    return ell


def oracle_topk(logits, k: int) -> np.ndarray:
    """The k experts with the largest logits per token, as int32 [T, k].

    Order: logit descending, expert id ascending among equal logits; a stable
    sort of the negated logits yields exactly that order."""
    ell = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-ell, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def oracle_weights(logits, idx, renormalize: int) -> np.ndarray:
    """Combine weights of the selected experts, float64 [T, k].

    p[t, e] = exp(l[t,e] - m_t) / sum_e' exp(l[t,e'] - m_t) (softmax over all
    E); with ``renormalize`` the k selected p are divided by their sum so that
    they add up to one, as in both worked examples ([0.3, 0.25, 0.25, 0.2] in
    "Why a Single All-Reduce/Reduce-Scatter Works"; 0.7 / 0.3 in "Return
    multiple expert results to the same token")."""
    ell = np.asarray(logits, dtype=np.float64)
    idx = np.asarray(idx)
    m = ell.max(axis=1, keepdims=True)
    z = np.exp(ell - m)
    sel = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    den = sel.sum(axis=1, keepdims=True) if renormalize else z.sum(axis=1, keepdims=True)
    return sel / den


def oracle_route(x, w_router, bias, k: int, renormalize: int, logits=None):
    """Router step: (logits, topk_idx, topk_w). If ``logits`` is given (for
    example the GPU's float32 logits), selection and weights are taken from
    those values instead of the float64 ones."""
    ell = oracle_logits(x, w_router, bias) if logits is None else np.asarray(logits, np.float64)
    idx = oracle_topk(ell, k)
    w = oracle_weights(ell, idx, renormalize)
    return ell, idx, w


# --------------------------------------------------------------------------- #
# 2. Dispatch                                                                  #
# --------------------------------------------------------------------------- #
def oracle_counts(idx, E: int) -> np.ndarray:
    """Number of (token, slot) selections of every expert, local or remote."""
    idx = np.asarray(idx).ravel()
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(idx == e))
    return counts.astype(np.int32)


def oracle_offsets(counts, e0: int, E_local: int) -> np.ndarray:
    """Start row of each local expert's segment: offsets[0] = 0,
    offsets[i+1] = offsets[i] + counts[e0 + i]. The rank owns the contiguous
    experts [e0, e0 + E_local) ("Expert Parallelism (EP)", "Limitations",
    static contiguous assignment)."""
    offsets = np.zeros(E_local + 1, dtype=np.int64)
    for i in range(E_local):
        offsets[i + 1] = offsets[i] + int(counts[e0 + i])
    return offsets.astype(np.int32)


def oracle_permutation(idx, e0: int, E_local: int):
    """Group the local (token, slot) pairs by expert.

    Returns perm_src[n] = t*k + j for dispatched row n, and inv[t*k + j] = n
    for local pairs, -1 for pairs whose expert is on another rank. Rows of
    expert e0+i come before those of e0+i+1; inside one expert they keep the
    (token, slot) order of the input."""
    idx = np.asarray(idx)
    flat = idx.ravel()
    segments = [np.nonzero(flat == e0 + i)[0] for i in range(E_local)]
    perm_src = (np.concatenate(segments) if segments else np.zeros(0, np.int64)).astype(np.int32)
    inv = np.full(flat.shape[0], -1, dtype=np.int32)
    inv[perm_src] = np.arange(perm_src.shape[0], dtype=np.int32)
    return perm_src, inv


def oracle_gather(x, perm_src, k: int) -> np.ndarray:
    """x_perm[n] = x[perm_src[n] // k]: the token vector of each dispatched row
    (token vectors move, router scores do not). Works on raw bits, so the
    result can be compared byte for byte."""
    src_tok = np.asarray(perm_src, dtype=np.int64) // k
    return np.asarray(x)[src_tok]


def oracle_dispatch(x, idx, E: int, e0: int, E_local: int):
    """counts, offsets, perm_src, inv, x_perm (x_perm in x's dtype)."""
    k = np.asarray(idx).shape[1]
    counts = oracle_counts(idx, E)
    offsets = oracle_offsets(counts, e0, E_local)
    perm_src, inv = oracle_permutation(idx, e0, E_local)
    x_perm = oracle_gather(x, perm_src, k)
    return counts, offsets, perm_src, inv, x_perm


# --------------------------------------------------------------------------- #
# 3. Expert MLPs                                                               #
# --------------------------------------------------------------------------- #
def oracle_silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def oracle_expert_h(xrows, w_gate_up) -> np.ndarray:
    """The hidden rows of one expert's SwiGLU MLP on stacked rows [M, H]:
    g = X Wg, u = X Wu, h = silu(g) * u, float64 [M, I], where Wg / Wu are
    the first / last I columns of gate_up [H, 2I]."""
    X = _f64(xrows)
    Wgu = _f64(w_gate_up)
    I = Wgu.shape[1] // 2
    g = X @ Wgu[:, :I]
    u = X @ Wgu[:, I:]
    return oracle_silu(g) * u


def oracle_expert_mlp(xrows, w_gate_up, w_down) -> np.ndarray:
    """One expert's SwiGLU MLP on stacked rows [M, H]: out = h Wd with h of
    oracle_expert_h and down [I, H]."""
    return oracle_expert_h(xrows, w_gate_up) @ _f64(w_down)


def oracle_expert_ffn(x_perm, offsets, w_gate_up, w_down) -> np.ndarray:
    """Expert outputs of every dispatched row: the rows of local expert i,
    [offsets[i], offsets[i+1]), go through expert i's MLP. float64 [N, H]."""
    offsets = np.asarray(offsets)
    E_local = offsets.shape[0] - 1
    N = int(offsets[-1])
    H = np.asarray(w_down).shape[2]
    out = np.zeros((N, H), dtype=np.float64)
    for i in range(E_local):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if b > a:
            out[a:b] = oracle_expert_mlp(np.asarray(x_perm)[a:b], w_gate_up[i], w_down[i])
    return out


# --------------------------------------------------------------------------- #
# 4. Combine                                                                   #
# --------------------------------------------------------------------------- #
def oracle_combine(expert_out, inv, topk_w, T: int, k: int) -> np.ndarray:
    """y[t] = sum over slots j with a local expert of w[t,j] * out[inv[t*k+j]];
    a token with no local expert gets zeros. float64 [T, H]."""
    out = _f64(expert_out)
    inv = np.asarray(inv).reshape(T, k)
    w = np.asarray(topk_w, dtype=np.float64).reshape(T, k)
    H = out.shape[1] if out.ndim == 2 else 0
    y = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        rows = inv[:, j]
        m = rows >= 0
        y[m] += w[m, j][:, None] * out[rows[m]]
    return y


# --------------------------------------------------------------------------- #
# Whole share                                                                  #
# --------------------------------------------------------------------------- #
def oracle_forward(x, w_router, bias, w_gate_up, w_down, k: int, e0: int, E_local: int,
                   renormalize: int = 1, logits=None, return_all: bool = False):
    """One rank's share of the MoE layer, route -> dispatch -> experts -> combine."""
    E = np.asarray(w_router).shape[0]
    T = np.asarray(x).shape[0]
    ell, idx, w = oracle_route(x, w_router, bias, k, renormalize, logits=logits)
    counts, offsets, perm_src, inv, x_perm = oracle_dispatch(x, idx, E, e0, E_local)
    out = oracle_expert_ffn(x_perm, offsets, w_gate_up, w_down)
    y = oracle_combine(out, inv, w, T, k)
    if return_all:
        return dict(logits=ell, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets,
                    perm_src=perm_src, inv=inv, x_perm=x_perm, expert_out=out, y=y)
    return y


def oracle_dense_forward(x, topk_idx, topk_w, w_gate_up, w_down, e0: int, E_local: int) -> np.ndarray:
    """The same share computed densely, without dispatch: every local expert
    runs on every token and its output is masked by the token's gate value
    for that expert (zero when not selected). This is the masking form of
    expert parallelism, written independently of the grouped path."""
    X = _f64(x)
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float64)
    T = X.shape[0]
    H = X.shape[1]
    y = np.zeros((T, H), dtype=np.float64)
    for i in range(E_local):
        gate = np.where(idx == e0 + i, w, 0.0).sum(axis=1)      # [T]
        y += gate[:, None] * oracle_expert_mlp(X, w_gate_up[i], w_down[i])
    return y
