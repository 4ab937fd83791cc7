"""Helpers of the GPU tests: moving the seeded numpy inputs to the GPU and the
GPU's outputs back, and the comparison metrics."""
from __future__ import annotations

import sys

import numpy as np
import torch

import expert_token_routing_amd as M
import workloads as W


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def to_dev(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DevInputs:
    def __init__(self, inp: W.MoEInputs, dev):
        self.inp = inp
        self.cfg = inp.cfg
        self.x = to_dev_bf16(inp.x, dev)
        self.w_router = to_dev(inp.w_router, dev)
        self.bias = None if inp.bias is None else to_dev(inp.bias, dev)
        self.w_gate_up = to_dev_bf16(inp.w_gate_up, dev) if inp.w_gate_up.size else None
        self.w_down = to_dev_bf16(inp.w_down, dev) if inp.w_down.size else None


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the compared tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


# Row caps the panel GEMM picks from (largest first) and its column-tile width.
PANEL_ROW_CAPS = (288, 256, 224, 192, 160, 128)
PANEL_BN = 256


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def panel_blocks(seg_rows, n_out: int, gate_up: bool, capacity: int, cus: int):
    """The row blocks the panel GEMM cuts the segments into, as the kernel
    chooses them: for each row cap, the tile count (row blocks x column
    tiles) and the tallest block; the cap minimising ceil(tiles / grid) x
    (tallest + 256) wins, the larger on ties; a segment of m rows becomes
    ceil(m / cap) blocks of equal height rounded up to 16 (the last one
    shorter). Returns (cap, [(first row, end row)] over the whole row range).
    n_out: the GEMM's output columns (I for gate/up, whose column tiles hold
    128 outputs, H for down, 256); capacity: rows of the launch's buffers."""
    ntn = _cdiv(n_out, PANEL_BN // 2 if gate_up else PANEL_BN)
    seg = [int(m) for m in seg_rows]
    bound = (_cdiv(capacity, PANEL_ROW_CAPS[-1]) + len(seg)) * ntn
    grid = max(8, min(cus // 8 * 8, _cdiv(bound, 8) * 8))
    best = None
    for cap in PANEL_ROW_CAPS:
        tiles = sum(_cdiv(m, cap) for m in seg if m > 0) * ntn
        tallest = max([(_cdiv(m, _cdiv(m, cap)) + 15) // 16 * 16 for m in seg if m > 0], default=0)
        est = _cdiv(tiles, grid) * (tallest + PANEL_BN)
        if best is None or est < best[0]:
            best = (est, cap)
    cap = best[1]
    blocks, start = [], 0
    for m in seg:
        if m > 0:
            nrt = _cdiv(m, cap)
            height = (_cdiv(m, nrt) + 15) // 16 * 16
            for i in range(nrt):
                r0 = i * height
                if r0 < m:
                    blocks.append((start + r0, start + min(m, r0 + height)))
        start += m
    return cap, blocks


# Tolerance on expert outputs and the combined output: bf16 inputs and
# weights, float32 accumulation, bf16 storage of h, the expert outputs and y.
OUT_TOL = 2e-2
# Router weights relative to the float64 weights from the same float32 logits.
W_RTOL = 1e-5
