"""Seeded synthetic inputs for one expert-parallel rank's share of an MoE layer.

This module is the only code that both the CPU oracle and the GPU library's
callers (tests, benchmark) use. It draws random numbers and stores them; it
computes nothing of the method itself (no routing, no softmax, no matmul).

Shapes and distributions follow the workloads the expert-parallelism pages
talk about:

* "Expert Parallelism (EP)" (AWS Neuron vLLM design doc), sections
  "Expert Weight Distribution" and "Router Weights": per-expert ``gate_up``
  is ``[H, 2I]`` and ``down`` is ``[I, H]``, stacked with the expert index
  first; the router weight ``[E, H]`` is replicated and scores all experts;
  rank r owns the contiguous experts ``[r*E_L, (r+1)*E_L)`` ("Limitations").
* The configurations are a tiny top-1 case mirroring the walk-through of
  "EP: Partition Experts and Route Tokens" (section "Send tokens to experts
  and return their results"), a small top-2 layer, a GPT-OSS-20B-shaped EP=8
  rank share (32 experts, 4 local, top-4), the same layer's EP=2 x TP=4 rank
  share (16 local experts, a quarter of the intermediate dimension: "Expert
  Parallelism (EP)", "Variable EP (EP+TP for MoE)" and the table of "How EP
  Differs from TP for MoE"), a DeepSeek-R1-shaped EP=8 rank share (256
  experts, 32 local, top-8), its decode-step size (256 tokens) and a skewed
  variant.
* Tensor-parallel shards (``tp > 1``): the experts are drawn at their full
  intermediate size ``I * tp`` and rank ``tp_rank`` keeps intermediate
  columns ``[tp_rank * I, (tp_rank + 1) * I)`` of both the gate half and the
  up half of ``gate_up`` (stored gate slice first, then up slice, so the
  shard has the ``[H, 2I]`` layout of a whole expert of size I) and the same
  rows of ``down``.

Generation recipe: numpy PCG64 with one substream per tensor and per expert,
``default_rng([seed, tensor_id, expert])``, float32 standard normal draws,
scaled by ``1/sqrt(fan_in)`` and rounded to bfloat16 (round to nearest even).
Router weights stay float32 ~ N(0, 1). Only the local experts' weights are
materialised, and any rank's share is reproducible on its own because the
expert index (not its local slot) names the substream.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# Tensor ids that name the random substreams.
_TID_X = 1
_TID_ROUTER = 2
_TID_GATE_UP = 3
_TID_DOWN = 4
_TID_PERM = 5


@dataclass(frozen=True)
class MoEConfig:
    """Problem statement of one rank's share: T tokens, hidden H, expert
    intermediate I, E experts in total, top-k, local experts [e0, e0+E_local)."""

    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    e0: int
    E_local: int
    renormalize: int = 1
    zipf_s: float = 0.0        # > 0: router bias that skews expert popularity
    zipf_kappa: float = 1.0
    x_scale: float | None = None   # None: 1/sqrt(H)
    seed: int = 0
    tp: int = 1                # > 1: the experts' intermediate dimension is I * tp; this share
    tp_rank: int = 0           # holds slice tp_rank of it (I columns of gate, of up, I rows of down)
    note: str = ""

    @property
    def capacity(self) -> int:
        """Rows a dispatch buffer needs in the worst case: every token can
        select each local expert at most once."""
        return self.T * min(self.k, self.E_local)

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS: dict[str, MoEConfig] = {
    "tiny_top1": MoEConfig("tiny_top1", T=64, H=128, I=256, E=4, k=1, e0=0, E_local=4,
                           note="walk-through sized top-1, all experts local, combine weight 1"),
    "small_top2": MoEConfig("small_top2", T=2048, H=1024, I=2816, E=8, k=2, e0=0, E_local=8,
                            note="top-2, all experts local, renormalised softmax weights"),
    "gptoss20b_ep8_share": MoEConfig("gptoss20b_ep8_share", T=8192, H=2880, I=3072, E=32, k=4,
                                     e0=0, E_local=4,
                                     note="GPT-OSS-20B-shaped layer, rank 0 of EP=8"),
    "gptoss20b_ep2_tp4_share": MoEConfig("gptoss20b_ep2_tp4_share", T=8192, H=2880, I=768, E=32, k=4,
                                         e0=0, E_local=16, tp=4, tp_rank=0,
                                         note="GPT-OSS-20B-shaped layer, rank 0 of EP=2 x TP=4: 16 local "
                                              "experts, intermediate slice 0 of 4"),
    "dsr1_ep8_share": MoEConfig("dsr1_ep8_share", T=16384, H=7168, I=2048, E=256, k=8,
                                e0=0, E_local=32,
                                note="DeepSeek-R1-shaped layer, rank 0 of EP=8"),
    "dsr1_ep8_decode": MoEConfig("dsr1_ep8_decode", T=256, H=7168, I=2048, E=256, k=8, e0=0, E_local=32,
                                 note="DeepSeek-R1-shaped layer, rank 0 of EP=8, one decode step of 256 "
                                      "tokens (about 8 rows per local expert)"),
    "gptoss20b_ep8_decode": MoEConfig("gptoss20b_ep8_decode", T=256, H=2880, I=3072, E=32, k=4, e0=0, E_local=4,
                                      note="GPT-OSS-20B-shaped layer, rank 0 of EP=8, one decode step of 256 "
                                           "tokens (about 32 rows per local expert)"),
    "dsr1_ep8_share_zipf": MoEConfig("dsr1_ep8_share_zipf", T=16384, H=7168, I=2048, E=256, k=8,
                                     e0=0, E_local=32, zipf_s=1.2, zipf_kappa=1.0,
                                     note="DeepSeek-R1 shapes, Zipf(1.2)-skewed expert popularity"),
}
CONFIG_ORDER = list(CONFIGS)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw
    16-bit patterns. Inputs are finite by construction."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(seed: int, tid: int, sub: int, shape, scale: float) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, sub])
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(scale)
    return bf16_bits_from_f32(a)


@dataclass
class MoEInputs:
    """One workload's tensors, all host numpy arrays.

    bf16 tensors are stored as their raw uint16 bit patterns.
    x          [T, H]              bf16 bits
    w_router   [E, H]              float32
    bias       [E] float32 or None
    w_gate_up  [E_local, H, 2I]    bf16 bits (columns [0, I) gate, [I, 2I) up)
    w_down     [E_local, I, H]     bf16 bits
    """

    cfg: MoEConfig
    x: np.ndarray
    w_router: np.ndarray
    bias: np.ndarray | None
    w_gate_up: np.ndarray
    w_down: np.ndarray
    meta: dict = field(default_factory=dict)


def zipf_router_bias(cfg: MoEConfig) -> np.ndarray:
    """Router bias that makes expert popularity follow a Zipf(s) rank law.

    Expert e gets popularity rank pi(e) in 1..E from a seeded permutation in
    which the rank's first local expert e0 is placed at rank 1 (the hottest
    expert is local), and bias[e] = kappa * ln(pi(e)^-s). A constant shift
    of all logits changes neither the top-k nor the softmax, so the Zipf
    normaliser is left out."""
    rng = np.random.default_rng([cfg.seed, _TID_PERM, 0])
    ranks = rng.permutation(cfg.E) + 1            # ranks[e] = pi(e)
    j = int(np.nonzero(ranks == 1)[0][0])
    ranks[j], ranks[cfg.e0] = ranks[cfg.e0], ranks[j]
    bias = -cfg.zipf_kappa * cfg.zipf_s * np.log(ranks.astype(np.float64))
    return bias.astype(np.float32)


def make_inputs(cfg: MoEConfig, threads: int | None = None, weights: bool = True) -> MoEInputs:
    """Draw every input of ``cfg``. ``weights=False`` skips the expert weights
    (routing-only consumers)."""
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    xs = cfg.x_scale if cfg.x_scale is not None else 1.0 / math.sqrt(H)
    x = _normal_bf16(cfg.seed, _TID_X, 0, (T, H), xs)
    wr = np.random.default_rng([cfg.seed, _TID_ROUTER, 0]).standard_normal((E, H), dtype=np.float32)
    bias = zipf_router_bias(cfg) if cfg.zipf_s > 0 else None
    if not weights:
        return MoEInputs(cfg, x, wr, bias, np.zeros((0,), np.uint16), np.zeros((0,), np.uint16))
    experts = list(range(cfg.e0, cfg.e0 + cfg.E_local))
    nthreads = threads or min(16, len(os.sched_getaffinity(0)))

    def both(e):
        return make_expert_weights(cfg, e)

    w_gu = np.empty((cfg.E_local, H, 2 * I), np.uint16)
    w_d = np.empty((cfg.E_local, I, H), np.uint16)
    with ThreadPoolExecutor(max(1, nthreads)) as ex:
        for i, (a, b) in enumerate(ex.map(both, experts)):
            w_gu[i] = a
            w_d[i] = b
    return MoEInputs(cfg, x, wr, bias, w_gu, w_d)


def make_expert_weights(cfg: MoEConfig, e: int) -> tuple[np.ndarray, np.ndarray]:
    """gate_up [H, 2I] and down [I, H] of global expert ``e`` as this share
    holds them (same values as ``make_inputs`` gives for that expert): the
    whole expert, or its tensor-parallel slice ``tp_rank`` of ``tp``."""
    H, I, tp, r = cfg.H, cfg.I, cfg.tp, cfg.tp_rank
    if tp < 1 or not 0 <= r < tp:
        raise ValueError(f"bad tensor-parallel shard {r} of {tp}")
    If = I * tp
    gu = _normal_bf16(cfg.seed, _TID_GATE_UP, e, (H, 2 * If), 1.0 / math.sqrt(H))
    dn = _normal_bf16(cfg.seed, _TID_DOWN, e, (If, H), 1.0 / math.sqrt(If))
    if tp == 1:
        return gu, dn
    cols = np.r_[r * I:(r + 1) * I, If + r * I:If + (r + 1) * I]
    return np.ascontiguousarray(gu[:, cols]), np.ascontiguousarray(dn[r * I:(r + 1) * I])
