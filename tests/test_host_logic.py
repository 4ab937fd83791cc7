"""Host-side logic of the tests themselves (CPU only): the replica of the
panel GEMM's row-block split that the full-size parity tests use to place
their sampled rows on block edges."""
from tests.gpu_helpers import PANEL_ROW_CAPS, panel_blocks


def test_panel_blocks_partition_every_segment():
    for seg, n_out, gate_up in (([600, 0, 17, 289, 1000], 2048, True), ([5000, 1, 288, 576], 7168, False),
                                ([16] * 40, 2880, True), ([0, 0], 512, False)):
        cap, blocks = panel_blocks(seg, n_out, gate_up, capacity=sum(seg), cus=256)
        assert cap in PANEL_ROW_CAPS
        start = 0
        for m in seg:
            mine = [(a, b) for a, b in blocks if start <= a < start + m]
            assert len(mine) == -(-m // cap)
            cur = start
            for j, (a, b) in enumerate(mine):
                assert a == cur and b > a and b - a <= cap
                if j < len(mine) - 1:
                    assert (b - a) % 16 == 0
                cur = b
            assert cur == start + m
            start += m


def test_panel_blocks_hand_example():
    """One expert of 600 rows, gate/up with I = 2048 (16 column tiles),
    buffers of 600 rows: the launch bound (ceil(600/128) + 1) x 16 = 96
    tiles gives a grid of 96; every cap then fits in one round, and the
    estimate (tallest block + 256) is lowest for 128-row caps (5 blocks of
    at most 128 rows: 384 against 416 for 192 and 464 for 288)."""
    cap, blocks = panel_blocks([600], 2048, True, capacity=600, cus=256)
    assert cap == 128
    assert blocks == [(0, 128), (128, 256), (256, 384), (384, 512), (512, 600)]
