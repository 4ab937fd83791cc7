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


def test_sgpr_hazard_scan():
    """The build's scan of the generated code: a direct-to-LDS load reading
    an SGPR that a vector instruction wrote fewer than 5 wait states earlier
    is reported; scalar writes, enough nops or a label in between are not."""
    from expert_token_routing_amd.build_lib import vmem_sgpr_hazards
    load = "buffer_load_dwordx4 v195, s[8:11], s1 offen lds"
    bad = f"v_readlane_b32 s1, v253, 2\n\ts_nop 0\n\t{load}\n"
    assert [h[2] for h in vmem_sgpr_hazards(bad)] == ["v_readlane_b32 s1, v253, 2"]
    desc = f"v_readfirstlane_b32 s9, v4\n\ts_add_i32 m0, s0, 0x2000\n\t{load}\n"
    assert len(vmem_sgpr_hazards(desc)) == 1
    assert vmem_sgpr_hazards(f"v_readlane_b32 s1, v253, 2\n\ts_nop 4\n\t{load}\n") == []
    assert vmem_sgpr_hazards(f"v_readlane_b32 s7, v253, 2\n\t{load}\n") == []       # not read by the load
    assert vmem_sgpr_hazards(f"s_mov_b32 s1, s84\n\t{load}\n") == []                # scalar write
    assert vmem_sgpr_hazards(f"v_readlane_b32 s1, v253, 2\n.LBB0_1:\n\t{load}\n") == []
    five = "\n\t".join(["v_readlane_b32 s1, v253, 2"] + ["s_add_i32 s2, s2, 1"] * 5 + [load])
    assert vmem_sgpr_hazards(five) == []
    four = "\n\t".join(["v_readlane_b32 s1, v253, 2"] + ["s_add_i32 s2, s2, 1"] * 4 + [load])
    assert len(vmem_sgpr_hazards(four)) == 1
