"""The grouped GEMV (experts with at most 32 rows) against the tile kernel.

moe_expert_ffn picks the GEMV when its capacity averages at most 32 rows per
local expert (for a gate/up GEMM whose local experts have 512 panels of 64
outputs or more: at most 16), so the same rows run through both kernels by
passing them once in a buffer of exactly their size and once padded to more
than 64 rows per expert (rows past offsets[E_local] are never read). Every output element is
one MFMA chain over k in the same order in both kernels, so h and the expert
outputs must agree bit for bit. Inputs are drawn on the GPU; this compares
two paths of the library, the oracle comparisons of the same kernels are in
test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import expert_token_routing_amd as M
from tests.gpu_helpers import device, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,I,counts", [
    (224, 160, [0, 1, 5, 16, 17, 3, 40, 16]),   # 7 / 5 k-steps, ragged 64-column panels, both kernels
    (256, 96, [16, 16, 16, 16]),                # exactly 16 rows everywhere (one row group)
    (256, 96, [32, 31, 17, 16, 0, 0]),          # two row groups, full and ragged
    (256, 96, [100, 3, 0, 5, 7, 1, 0, 2]),      # a hot expert: four 32-row waves per panel
    (64, 64, [2, 0, 16]),                       # 2 k-steps, one panel
    (32, 32, [16, 3, 0, 1]),                    # one k-step: every later ring slot reloads it
    (1024, 512, [9, 12, 1, 30, 0, 16, 7, 11]),  # several ring turns
    (7168, 2048, [14, 9, 0, 16, 1, 33, 8, 12]), # the DeepSeek-R1 expert shape (one-wave workgroups)
    (7168, 2048, [14, 9, 0, 16, 1, 33, 8, 12, 5, 20, 3, 7, 11, 2, 30, 4]),  # 512+ panels: four-wave workgroups
    # 17..32 expected rows per expert: both GEMMs on the GEMV while the gate/up
    # panels are fewer than 512 (rows 16 / 17 / 31 / 32 / 33 at the group
    # edges, ragged 64-column gate/up and 128-column down panels)
    (224, 160, [16, 17, 31, 32, 33, 20, 25, 18]),
    (256, 96, [32, 32, 32, 32]),                # exactly 32 rows everywhere (two full groups)
    (2880, 3072, [40, 24, 31, 33]),             # GPT-OSS-20B expert shape, few panels, 32 expected rows
    # 17..32 expected rows with 512 gate/up panels: gate/up on tiles, down on the GEMV
    (1024, 2048, [20, 17, 31, 0, 33, 16, 25, 18, 22, 19, 32, 1, 21, 24, 30, 27]),
], ids=["ragged", "full16", "two_groups", "hot", "tiny", "one_step", "mid", "dsr1", "dsr1_16", "edges17_33", "full32",
        "gptoss", "down_only"])
def test_grouped_gemv_matches_tiles(H, I, counts):
    dev = device()
    E_local = len(counts)
    N = int(sum(counts))
    cap_big = 64 * E_local + 1
    assert N <= 32 * E_local
    g = torch.Generator(device=dev).manual_seed(11)
    x = (torch.randn((cap_big, H), generator=g, device=dev) / H ** 0.5).to(torch.bfloat16)
    wgu = (torch.randn((E_local, H, 2 * I), generator=g, device=dev) / H ** 0.5).to(torch.bfloat16)
    wd = (torch.randn((E_local, I, H), generator=g, device=dev) / I ** 0.5).to(torch.bfloat16)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
    say(f"grouped GEMV H={H} I={I} counts={counts}")
    h1, o1 = M.moe_expert_ffn(x[:max(N, 1)].contiguous(), offsets, wgu, wd)
    say(f"tiles H={H} I={I} capacity={cap_big}")
    h2, o2 = M.moe_expert_ffn(x, offsets, wgu, wd)
    torch.cuda.synchronize()
    hb1, hb2 = h1[:N].view(torch.int16), h2[:N].view(torch.int16)
    ob1, ob2 = o1[:N].view(torch.int16), o2[:N].view(torch.int16)
    assert torch.equal(hb1, hb2), int((hb1 != hb2).sum())
    assert torch.equal(ob1, ob2), int((ob1 != ob2).sum())
    assert torch.isfinite(o1[:N].float()).all()
