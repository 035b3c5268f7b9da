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


@pytest.mark.parametrize("mode", [ep.MODE_NORMAL, ep.MODE_LOW_LATENCY], ids=["normal", "low_latency"])
@pytest.mark.parametrize("quant", [ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0], ids=["fp32_scale", "ue8m0"])
def test_hip_matches_hand_quantised_group(quant, mode):
    from golden_example import FP8, fp8_input_and_codes
    say("golden fp8", quant, mode)
    x, codes = fp8_input_and_codes()
    pr = FP8["problem"]
    p = ep.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=mode, quant=quant)
    cap = ep.max_recv_rows(p)
    lay = ep.Layout(p, recv_capacity=cap)
    ws = ep.workspace(p)
    tk = torch.zeros((1, 1, 1), dtype=torch.int32, device=DEV)
    ep.get_layout(p, tk, lay, ws)
    recv = ep.Recv(p, cap)
    xg = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    ep.dispatch(p, lay, xg, recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    assert int(h(lay.send_pos).reshape(-1)[0]) == 0
    assert np.array_equal(h(recv.x)[0], codes)
    sc = h(recv.scales).reshape(-1)[0]
    if quant == ep.QUANT_FP8_F32:
        assert sc == np.float32(FP8["fp32_scale"])
    else:
        assert int(sc) == FP8["ue8m0_byte"]


def test_hip_matches_hand_worked_messages():
    """Packer and descriptors through the C ABI against the hand derivation,
    then the loopback delivery (each region arrives at its receive offset
    byte for byte) and the receiver's low-latency layout."""
    from golden_example import MSG, check_messages, check_unpacked, message_inputs
    say("golden messages")
    x, topk, wt, codes = message_inputs()
    pr = MSG["problem"]
    p = ep.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=ep.MODE_MESSAGES,
                   quant=ep.QUANT_FP8_F32, region_bytes=pr["region_bytes"], epoch=pr["epoch"])
    lay = ep.Layout(p)
    ws = ep.workspace(p)
    tk = torch.from_numpy(topk).to(DEV)
    ep.get_layout(p, tk, lay, ws)
    msgs = ep.Messages(p, 512, 64)
    msgs.send_arena.fill_(0xAB)  # bytes outside the regions are not the packer's
    xg = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    ep.dispatch(p, lay, xg, msgs=msgs, topk_idx=tk, topk_weights=torch.from_numpy(wt).to(DEV),
                ws=ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    nd = int(h(msgs.num_descriptors)[0])
    arena = h(msgs.send_arena)
    check_messages(h(msgs.table), h(msgs.arena_base), h(msgs.descriptors)[:nd], nd, arena, codes)
    recv = torch.full((512,), 0xCD, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_execute(p, msgs, recv, err)
    torch.cuda.synchronize()
    assert int(h(err)[0]) == 0
    got = h(recv)
    for row in np.array(MSG["table"]).reshape(-1, 8):
        if row[2] > 0:
            assert np.array_equal(got[row[1]:row[1] + row[2]], arena[row[0]:row[0] + row[2]])
    # the receiver
    recv_cap = int(MSG["arena_base"][1][-1])
    out, cnt, src = ep.unpack_buffers(p)
    ep.messages_unpack(p, msgs, recv[:recv_cap], lay.num_tokens_per_expert, out, cnt, src, err)
    torch.cuda.synchronize()
    assert int(h(err)[0]) == 0
    check_unpacked(h(out.x), h(out.scales), h(cnt), h(src), codes)


@pytest.mark.parametrize("section", ["normal", "low_latency", "rank_major"])
def test_hip_matches_duplicate_ids_example(section):
    from golden_example import DUP, DUP_MODES, check_dup_layout, dup_expected_out, dup_inputs
    say("golden duplicates", section)
    topk, wt, xb, x = dup_inputs()
    pr = DUP["problem"]
    mode = DUP_MODES[section]
    p = ep.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=mode)
    cap = ep.max_recv_rows(p)
    lay = ep.Layout(p, recv_capacity=cap)
    ws = ep.workspace(p)
    tk = torch.from_numpy(topk).to(DEV)
    ep.get_layout(p, tk, lay, ws)
    recv = ep.Recv(p, cap)
    xg = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    wtg = torch.from_numpy(wt).to(DEV)
    kw = dict(topk_idx=tk, topk_weights=wtg) if mode == ep.MODE_RANK_MAJOR else {}
    ep.dispatch(p, lay, xg, recv=recv, ws=ws, **kw)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    rows = check_dup_layout(lambda f: h(getattr(lay, f)), section)
    got = h(recv.x.view(torch.int16)).view(np.uint16)
    for r, st in rows.items():
        assert np.array_equal(got[r], xb.reshape(-1, pr["H"])[st])
    out = torch.empty((pr["R"], pr["T"], pr["H"]), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, lay, recv.x, None if mode == ep.MODE_RANK_MAJOR else wtg, out)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    assert np.array_equal(h(out.view(torch.int16)).view(np.uint16), dup_expected_out(section, x))


def test_hip_matches_low_latency_overflow_example():
    from golden_example import DUP
    o = DUP["overflow"]
    pr = o["problem"]
    say("golden overflow")
    p = ep.Problem(pr["R"], pr["T"], pr["H"], pr["E"], pr["K"], mode=ep.MODE_LOW_LATENCY)
    lay = ep.Layout(p)
    ws = ep.workspace(p)
    ep.get_layout(p, torch.tensor(o["topk_idx"], dtype=torch.int32, device=DEV), lay, ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == o["err"]
    assert np.array_equal(h(lay.send_pos), np.array(o["send_pos"]))
