"""The oracle against the hand-worked routing example (tests/golden): every
layout output in the normal (alignment 1 and 4), low-latency and rank-major
modes, the dispatched rows, and the exact combine of the identity expert."""
import numpy as np
import pytest

from golden_example import (EX, H, K, MODES, R, T, TOPK, W, E, bf16_bits, check_layout,
                            expected_out, expected_rows, x_values)
from oracle import oracle as orc


@pytest.mark.parametrize("section", sorted(MODES))
def test_oracle_matches_worked_example(section):
    mode, align = MODES[section]
    p = orc.Problem(R, T, H, E, K, align=align, mode=mode)
    lay = orc.layout(p, TOPK)
    assert lay.err == 0
    check_layout(lambda f: getattr(lay, f), section)
    # dispatch: every filled row holds its source token's row
    x = bf16_bits(x_values())
    cap = E * R * T if mode == 1 else lay.total_rows
    err, recv, _ = orc.dispatch(p, x, TOPK, lay.send_pos, cap)
    assert err == 0
    for r, st in expected_rows(section).items():
        if st >= 0:
            assert np.array_equal(recv[r], x.reshape(R * T, H)[st]), (section, r)
    # combine of the identity expert
    err, out = orc.combine(p, recv, W, lay.send_pos)
    assert err == 0
    assert np.array_equal(out, expected_out(section)), section


def test_fixture_is_self_consistent():
    # closed forms the hand derivation must satisfy
    assert int(np.sum(EX["num_tokens_per_expert"])) == int(np.sum(TOPK >= 0))
    rpm = np.cumsum(np.array(EX["num_tokens_per_rank"]), axis=0)
    assert np.array_equal(rpm, np.array(EX["rank_prefix_matrix"]))
    assert EX["normal_align1"]["row_base"][-1] == int(np.sum(TOPK >= 0))
    assert EX["rank_major"]["row_base"][-1] == int(np.sum(EX["is_token_in_rank"]))


@pytest.mark.parametrize("mode", [0, 1], ids=["normal", "low_latency"])
@pytest.mark.parametrize("quant", [1, 2], ids=["fp32_scale", "ue8m0"])
def test_oracle_matches_hand_quantised_group(quant, mode):
    from golden_example import FP8, fp8_input_and_codes
    x, codes = fp8_input_and_codes()
    pr = FP8["problem"]
    p = orc.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=mode, quant=quant)
    topk = np.zeros((1, 1, 1), np.int32)
    lay = orc.layout(p, topk)
    cap = 1
    assert lay.send_pos.reshape(-1)[0] == 0
    err, recv, scales = orc.dispatch(p, x, topk, lay.send_pos, cap)
    assert err == 0
    assert np.array_equal(recv[0], codes)
    if quant == 1:
        assert scales.reshape(-1)[0] == np.float32(FP8["fp32_scale"])
    else:
        assert int(scales.reshape(-1)[0]) == FP8["ue8m0_byte"]


def test_oracle_matches_hand_worked_messages():
    from golden_example import MSG, check_messages, check_unpacked, message_inputs
    x, topk, wt, codes = message_inputs()
    pr = MSG["problem"]
    p = orc.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=2, quant=1,
                    region_bytes=pr["region_bytes"], epoch=pr["epoch"])
    om = orc.messages(p, x, topk, wt, 512, 64)
    assert om.err == 0
    check_messages(om.table, om.arena_base, om.desc, om.num_desc, om.send_arena, codes)
    # delivery and the receiver
    err, recv = orc.messages_execute(p, om, int(om.arena_base[1][-1]))
    assert err == 0
    lay = orc.layout(p, topk)
    un = orc.messages_unpack(p, recv, om.table, lay.num_tokens_per_expert)
    assert un.err == 0
    check_unpacked(un.recv, un.scales, un.recv_count, un.recv_src_idx, codes)


@pytest.mark.parametrize("section", ["normal", "low_latency", "rank_major"])
def test_oracle_matches_duplicate_ids_example(section):
    from golden_example import DUP, DUP_MODES, check_dup_layout, dup_expected_out, dup_inputs
    topk, wt, xb, x = dup_inputs()
    pr = DUP["problem"]
    p = orc.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=DUP_MODES[section])
    lay = orc.layout(p, topk)
    assert lay.err == 0
    rows = check_dup_layout(lambda f: getattr(lay, f), section)
    cap = pr["E"] * pr["R"] * pr["T"] if section == "low_latency" else lay.total_rows
    err, recv, _ = orc.dispatch(p, xb, topk, lay.send_pos, cap)
    assert err == 0
    for r, st in rows.items():
        assert np.array_equal(recv[r], xb.reshape(-1, pr["H"])[st])
    err, out = orc.combine(p, recv, wt, lay.send_pos)
    assert err == 0
    assert np.array_equal(out, dup_expected_out(section, x))


def test_oracle_matches_low_latency_overflow_example():
    from golden_example import DUP
    o = DUP["overflow"]
    pr = o["problem"]
    p = orc.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=1)
    lay = orc.layout(p, np.array(o["topk_idx"], np.int32))
    assert lay.err == o["err"]
    assert np.array_equal(lay.send_pos, np.array(o["send_pos"]))
