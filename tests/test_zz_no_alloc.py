"""ep_dispatch_fused_noalloc (the library's fixed scratch array in place of
the caller's workspace) against ep_dispatch_fused through the C ABI, bit for
bit: two calls in a row on one stream, the second with a smaller problem
(the array keeps the first call's contents), every layout output, receive
row and scale compared; then the same pair again in the other order on a
second stream; the call captured into a HIP graph and replayed with fresh
inputs; a problem needing more scratch than the array is refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import DEV, LAYOUT_FIELDS, assert_layout_equal, h, say

pytestmark = pytest.mark.gpu

N, L, QF, QU = ep.MODE_NORMAL, ep.MODE_LOW_LATENCY, ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0
# name, R, T, H, E, K, mode, quant, align, masked, duplicates -- both past the
# one-launch layout (6,144 entries), so the chunked layout and the fused
# dispatch kernel use the scratch memory
BIG = ("ll_decode_shape", 8, 128, 7168, 256, 8, L, QF, 1, 0.0, 0.0)
SMALL = ("normal_ue8m0_smaller", 4, 300, 1024, 32, 8, N, QU, 4, 0.1, 0.2)


def make(case):
    name, R, T, H, E, K, mode, quant, align, mfrac, dfrac = case
    w = inputs.small(f"noalloc_{name}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=41)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=6)
    x = inputs.gen_x(w)
    p = ep.Problem(R, T, H, E, K, align=align, mode=mode, quant=quant)
    assert 0 < ep.workspace_bytes(p) <= ep.NOALLOC_SCRATCH_BYTES
    assert R * T * K > 6144
    po = orc.Problem(R, T, H, E, K, align=align, mode=mode, quant=quant)
    return p, po, topk, x


def outputs(p):
    cap = ep.max_recv_rows(p)
    lay = ep.Layout(p)
    recv = ep.Recv(p, cap)
    recv.x.view(torch.uint8).fill_(0x33)
    recv.scales.view(torch.uint8).fill_(0x33)
    lay.recv_src_idx.fill_(-7)
    return lay, recv


def check(case, stream):
    p, po, topk, x = make(case)
    say("noalloc", case[0])
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    with torch.cuda.stream(stream):
        ln, rn = outputs(p)
        ep.dispatch_fused_noalloc(p, tk, ln, xg, rn)
        lf, rf = outputs(p)
        ep.dispatch_fused(p, tk, lf, xg, rf, ep.workspace(p))
    torch.cuda.synchronize()
    for f in LAYOUT_FIELDS + ["err", "recv_src_idx"]:
        assert torch.equal(getattr(ln, f), getattr(lf, f)), f
    assert torch.equal(rn.x, rf.x)
    assert torch.equal(rn.scales, rf.scales)
    assert_layout_equal(ln, orc.layout(po, topk), p.mode)


def test_noalloc_matches_fused_call_twice():
    s = torch.cuda.current_stream()
    check(BIG, s)
    check(SMALL, s)  # smaller problem: the array holds the first call's data


def test_noalloc_on_a_second_stream():
    s = torch.cuda.Stream()
    check(SMALL, s)
    check(BIG, s)


def test_noalloc_replays_in_a_graph():
    """The entry point captured once into a HIP graph (the callers it is
    for) and replayed with fresh routing and tokens copied into its inputs,
    every output poisoned first: each replay equals an eager
    ep_dispatch_fused of the same inputs, bit for bit."""
    name, R, T, H, E, K, mode, quant, align, _, _ = BIG
    p, po, topk, x = make(BIG)
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    lg, rg = outputs(p)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call = ep.prepare(ep.dispatch_fused_noalloc, p, tk, lg, xg, rg)
        call()  # first call on the device (the array's address is looked up) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        w = inputs.small(f"noalloc_graph_{rep}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant,
                         seed=300 + rep)
        topk_r = inputs.gen_topk(w)
        if rep % 2 == 1:
            topk_r = inputs.masked_topk(w, topk_r, 0.2, 0.0, seed=rep)
        tk.copy_(torch.from_numpy(topk_r))
        xg.copy_(torch.from_numpy(inputs.gen_x(w)).view(torch.bfloat16))
        rg.x.view(torch.uint8).fill_(0x33)
        rg.scales.view(torch.uint8).fill_(0x33)
        lg.recv_src_idx.fill_(-7)
        lg.send_pos.fill_(-7)
        torch.cuda.synchronize()
        say("noalloc graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        lf, rf = outputs(p)
        ep.dispatch_fused(p, tk, lf, xg, rf, ep.workspace(p))
        torch.cuda.synchronize()
        for f in LAYOUT_FIELDS + ["err", "recv_src_idx"]:
            assert torch.equal(getattr(lg, f), getattr(lf, f)), (rep, f)
        assert torch.equal(rg.x, rf.x)
        assert torch.equal(rg.scales, rf.scales)
        assert_layout_equal(lg, orc.layout(po, topk_r), p.mode)


def test_noalloc_refuses_problems_past_the_array():
    # 64 ranks x 8192 tokens: per-(token, rank) stream ranks alone need 128 MiB
    p = ep.Problem(64, 8192, 128, 256, 8, mode=N)
    assert ep.workspace_bytes(p) > ep.NOALLOC_SCRATCH_BYTES
    st = ep.lib().ep_dispatch_fused_noalloc(ctypes.byref(p.c()), None, None, None, None, None)
    assert st == ep.ERR_SCRATCH
    assert "scratch" in ep.status_string(st)
