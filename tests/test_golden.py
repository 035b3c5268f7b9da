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
