"""The HIP path, through the C ABI, against the hand-worked routing example
(tests/golden): every layout output in the normal (alignment 1 and 4),
low-latency and rank-major modes, from ep_get_layout and from the fused
call; the dispatched rows; and the combine of the identity expert, which is
exact here, so it must match bit for bit."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep
from golden_example import (H, K, MODES, R, T, TOPK, W, E, bf16_bits, check_layout,
                            expected_out, expected_rows, x_values)
from gpu_util import DEV, h, say

pytestmark = pytest.mark.gpu


def run(section, fused):
    mode, align = MODES[section]
    p = ep.Problem(R, T, H, E, K, align=align, mode=mode)
    cap = ep.max_recv_rows(p)
    lay = ep.Layout(p, recv_capacity=cap)
    lay.recv_src_idx.fill_(-7)  # rows nobody writes stay visible
    ws = ep.workspace(p)
    tk = torch.from_numpy(TOPK).to(DEV)
    x = bf16_bits(x_values())
    xg = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    wt = torch.from_numpy(W).to(DEV)
    recv = ep.Recv(p, cap)
    if fused:
        ep.dispatch_fused(p, tk, lay, xg, recv, ws)
    else:
        ep.get_layout(p, tk, lay, ws)
        kw = dict(topk_idx=tk, topk_weights=wt) if mode == ep.MODE_RANK_MAJOR else {}
        ep.dispatch(p, lay, xg, recv=recv, ws=ws, **kw)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    return p, lay, recv, x, wt


# the fused call serves the normal and low-latency modes
CASES = [(s, False) for s in sorted(MODES)] + [(s, True) for s in sorted(MODES)
                                                if MODES[s][0] != ep.MODE_RANK_MAJOR]


@pytest.mark.parametrize("section,fused", CASES,
                         ids=[f"{s}-{'fused' if f else 'separate'}" for s, f in CASES])
def test_hip_matches_worked_example(section, fused):
    mode, _ = MODES[section]
    say("golden", section, "fused" if fused else "separate")
    p, lay, recv, x, wt = run(section, fused)
    check_layout(lambda f: h(getattr(lay, f)), section)
    rows = h(recv.x.view(torch.int16)).view(np.uint16)
    for r, st in expected_rows(section).items():
        if st >= 0:
            assert np.array_equal(rows[r], x.reshape(R * T, H)[st]), (section, r)
    out = torch.empty((R, T, H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, lay, recv.x, None if mode == ep.MODE_RANK_MAJOR else wt, out)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    assert np.array_equal(h(out.view(torch.int16)).view(np.uint16), expected_out(section))
