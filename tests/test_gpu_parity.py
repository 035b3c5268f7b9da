"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for layout, indices, rows, FP8 codes,
scales, message bytes and descriptors; bf16 combine within 1e-2 relative
error per element (plus a rounding floor, see gpu_util.combine_close).

Small sweeps span several chunks and ragged tails, masked (-1) and
duplicate expert ids, expert alignment, K = 1 .. 16, R = 1 .. 64, hidden
sizes with a partial last row piece, and empty input.  The five workloads
run at full size; where the oracle cannot hold the whole output, sampled
tokens are compared, plus properties that hold at any size.
"""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import (DEV, abs_weighted_sum, assert_layout_equal, bf16_to_f32, combine_close,
                      gpu_layout, h, problems, say)

pytestmark = pytest.mark.gpu

N, LL, MSG = ep.MODE_NORMAL, ep.MODE_LOW_LATENCY, ep.MODE_MESSAGES
QN, QF, QU = ep.QUANT_NONE, ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0

# name, R, T, H, E, K, align, mode, quant, masked, duplicates, region bytes
SMALL = [
    ("r1", 1, 5, 128, 4, 2, 1, N, QN, 0.0, 0.0, 0),
    ("tiny", 2, 8, 128, 8, 2, 1, N, QN, 0.0, 0.0, 0),
    ("ragged", 3, 1000, 256, 12, 3, 4, N, QN, 0.1, 0.1, 0),
    ("k1", 4, 2500, 128, 8, 1, 1, N, QN, 0.05, 0.0, 0),
    ("multi_launch", 4, 1300, 128, 16, 4, 2, N, QN, 0.05, 0.05, 0),  # > 16384 entries
    ("multi_launch_ll", 4, 1100, 128, 8, 4, 1, LL, QF, 0.05, 0.0, 0),
    ("k16", 2, 100, 256, 64, 16, 2, N, QN, 0.1, 0.2, 0),
    ("r64", 64, 40, 128, 256, 8, 1, N, QN, 0.0, 0.0, 0),
    ("e_eq_r", 8, 300, 128, 8, 4, 1, N, QN, 0.0, 0.5, 0),
    ("h_tail", 2, 16, 7176, 8, 2, 1, N, QN, 0.0, 0.0, 0),
    ("h_16k_lds", 2, 9, 16384, 8, 3, 1, N, QN, 0.1, 0.0, 0),  # widest LDS-staged copy
    ("h_32k_regs", 2, 7, 32768, 8, 3, 2, N, QN, 0.1, 0.1, 0),  # register-resident copy
    ("ll_h_16392", 2, 5, 16392, 4, 2, 1, LL, QN, 0.0, 0.3, 0),
    ("ll", 4, 130, 256, 16, 4, 1, LL, QN, 0.1, 0.0, 0),
    ("ll_dup", 2, 20, 128, 4, 4, 1, LL, QN, 0.0, 0.9, 0),
    ("fp8n", 4, 333, 384, 16, 4, 1, N, QF, 0.05, 0.0, 0),
    ("fp8ll", 4, 90, 256, 16, 4, 1, LL, QF, 0.05, 0.0, 0),
    ("ue8n", 4, 200, 512, 16, 4, 3, N, QU, 0.05, 0.05, 0),
    ("ue8ll", 2, 64, 128, 8, 2, 1, LL, QU, 0.0, 0.0, 0),
    ("fp8_htail", 2, 16, 8320, 8, 2, 1, LL, QF, 0.0, 0.0, 0),
    ("empty", 2, 0, 128, 8, 2, 1, N, QN, 0.0, 0.0, 0),
    # grouped-GEMM tile alignments: chunked and one-launch layouts, the scale
    # transpose with padding rows
    ("align128", 4, 600, 256, 32, 4, 128, N, QN, 0.05, 0.0, 0),
    ("align128_ue8", 4, 300, 512, 16, 8, 128, N, QU, 0.05, 0.05, 0),
    ("align64_direct", 2, 50, 128, 8, 4, 64, N, QF, 0.1, 0.0, 0),
    # the documented limits: 256 ranks, 2048 experts, top-64, hidden 32768
    ("max_r", 256, 3, 128, 256, 8, 1, N, QN, 0.1, 0.1, 0),
    ("max_r_chunked", 256, 5, 128, 512, 8, 2, N, QN, 0.05, 0.0, 0),
    ("max_e_k", 4, 9, 128, 2048, 64, 2, N, QN, 0.05, 0.1, 0),
    ("max_k_ll", 2, 16, 128, 64, 64, 1, LL, QN, 0.0, 0.0, 0),
    ("max_r_ll", 256, 2, 128, 256, 4, 1, LL, QF, 0.0, 0.0, 0),
    ("max_h_fp8", 2, 5, 32768, 8, 2, 1, N, QF, 0.0, 0.0, 0),
    ("fp8_h4096_one_wave", 4, 37, 4096, 16, 4, 2, N, QU, 0.1, 0.1, 0),
    ("fp8_h2048", 3, 21, 2048, 12, 3, 1, N, QF, 0.05, 0.0, 0),
    ("max_h_ue8_ll", 2, 3, 32768, 4, 2, 1, LL, QU, 0.0, 0.0, 0),
    ("msg", 4, 50, 256, 16, 4, 1, MSG, QF, 0.1, 0.1, 512),
    ("msg_ue8", 3, 40, 128, 6, 3, 1, MSG, QU, 0.0, 0.0, 256),
    ("msg_bf16", 4, 30, 136, 8, 3, 1, MSG, QN, 0.1, 0.0, 128),
    ("msg_r64", 64, 12, 256, 128, 8, 1, MSG, QF, 0.0, 0.0, 4096),
    ("msg_max_r", 256, 2, 128, 256, 4, 1, MSG, QF, 0.0, 0.0, 4096),
]
IDS = [c[0] for c in SMALL]


def small_case(c, seed=7):
    name, R, T, H, E, K, align, mode, quant, mfrac, dfrac, rb = c
    w = inputs.small(name, R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=300 + seed,
                     region_bytes=rb or (2 << 20), epoch=9)
    topk = inputs.gen_topk(w) if T > 0 else np.zeros((R, 0, K), np.int32)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac)
    return w, align, topk


# Chunk counts that give the layout scan three and six chunks per thread
# (register-held rows, part of the registers unused) and ten (the
# element-by-element loop), with 1,504, 3,008 and 5,008 chunks; layout only.
LONG_SCAN = [
    ("scan_rows_3", 8, 12000, 128, 64, 8, 4, N, QN, 0.05, 0.05, 0),
    ("scan_rows_6", 16, 12000, 128, 64, 8, 1, N, QN, 0.0, 0.1, 0),
    ("scan_rows_10", 16, 20000, 128, 64, 8, 2, N, QN, 0.05, 0.0, 0),
]


@pytest.mark.parametrize("case", LONG_SCAN, ids=[c[0] for c in LONG_SCAN])
def test_layout_long_scan_rows(case):
    w, align, topk = small_case(case)
    say("layout", case)
    p, po = problems(w, align)
    gl, _ = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert_layout_equal(gl, ol, w.mode)


@pytest.mark.parametrize("case", SMALL, ids=IDS)
def test_layout_small(case):
    w, align, topk = small_case(case)
    say("layout", case)
    p, po = problems(w, align)
    gl, _ = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert_layout_equal(gl, ol, w.mode)


def test_layout_is_deterministic():
    w, align, topk = small_case(SMALL[2])
    p, _ = problems(w, align)
    a, _ = gpu_layout(p, topk)
    b, _ = gpu_layout(p, topk)
    for f in ["send_pos", "send_head", "rank_prefix_matrix", "expert_start"]:
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    total = int(a.row_base[-1].item())  # rows past the filled range are not written
    assert torch.equal(a.recv_src_idx[:total], b.recv_src_idx[:total])


def _recv_capacity(w, ol):
    return ol.total_rows if w.mode == N else w.E * w.R * w.T


def _scale_index(w, row, cap):
    G, RT = w.G, w.R * w.T
    g = np.arange(G)
    if w.mode == LL:
        return (row // RT * G + g) * RT + row % RT
    return g * cap + row


@pytest.mark.parametrize("case", [c for c in SMALL if c[7] != MSG], ids=[c[0] for c in SMALL if c[7] != MSG])
def test_dispatch_small(case):
    w, align, topk = small_case(case)
    say("dispatch", case)
    p, po = problems(w, align)
    x = inputs.gen_x(w) if w.T > 0 else np.zeros((w.R, 0, w.H), np.uint16)
    gl, ws = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    cap = _recv_capacity(w, ol)
    recv = ep.Recv(p, cap)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    ep.dispatch(p, gl, xg, recv=recv, ws=ws)
    torch.cuda.synchronize()
    err, orecv, osc = orc.dispatch(po, x, topk, ol.send_pos, cap)
    assert err == 0 and int(h(gl.err)[0]) == ol.err
    rows = ol.send_pos[ol.send_pos >= 0]
    grecv = h(recv.x.view(torch.uint16) if w.quant == QN else recv.x)
    assert np.array_equal(grecv[rows], orecv[rows])
    if w.quant != QN:
        gsc = h(recv.scales)
        for r in rows:
            si = _scale_index(w, int(r), cap)
            assert np.array_equal(gsc[si], osc[si]), r


@pytest.mark.parametrize("case", [c for c in SMALL if c[7] != MSG], ids=[c[0] for c in SMALL if c[7] != MSG])
def test_combine_small(case):
    w, align, topk = small_case(case)
    say("combine", case)
    p, po = problems(w, align)
    gl, ws = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    cap = max(_recv_capacity(w, ol), 1)
    y = inputs.gen_y(w, cap)
    wt = inputs.gen_weights(w) if w.T > 0 else np.zeros((w.R, 0, w.K), np.float32)
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, torch.from_numpy(y).view(torch.bfloat16).to(DEV),
               torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    err, oout = orc.combine(po, y, wt, ol.send_pos)
    assert err == 0
    g = h(out.view(torch.uint16)).reshape(-1, w.H)
    if g.size:
        absw = abs_weighted_sum(bf16_to_f32(y), wt, ol.send_pos)
        rel = combine_close(g, oout.reshape(-1, w.H), absw)
        say("max rel err", rel)


def _messages_compare(w, p, po, gl, topk, x, wt, ws):
    counts = h(gl.num_tokens_per_rank)
    send_cap, desc_cap = ep.messages_capacity(p, counts)
    msgs = ep.Messages(p, send_cap, desc_cap)
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), msgs=msgs,
                topk_idx=torch.from_numpy(topk).to(DEV), topk_weights=torch.from_numpy(wt).to(DEV),
                ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
    assert om.err == 0
    table = h(msgs.table)
    assert np.array_equal(table, om.table)
    assert np.array_equal(h(msgs.arena_base), om.arena_base)
    nd = int(h(msgs.num_descriptors)[0])
    assert nd == om.num_desc
    assert np.array_equal(h(msgs.descriptors)[:nd], om.desc)
    arena = msgs.send_arena
    for off, reg in table.reshape(-1, 8)[:, [0, 2]]:
        if reg > 0:
            g = h(arena[off:off + reg])
            assert np.array_equal(g, om.send_arena[off:off + reg]), (off, reg)
    return om


@pytest.mark.parametrize("case", [c for c in SMALL if c[7] == MSG], ids=[c[0] for c in SMALL if c[7] == MSG])
def test_messages_small(case):
    w, align, topk = small_case(case)
    say("messages", case)
    p, po = problems(w, align)
    x = inputs.gen_x(w)
    wt = inputs.gen_weights(w)
    gl, ws = gpu_layout(p, topk)
    _messages_compare(w, p, po, gl, topk, x, wt, ws)


# ----------------------------------------------------------------- errors
def test_out_of_range_ids_are_flagged_and_skipped():
    w = inputs.small("oor", R=2, T=40, H=128, E=8, K=2, seed=5)
    topk = inputs.gen_topk(w)
    topk[0, 3, 1] = 8
    topk[1, 7, 0] = -5
    p, po = problems(w)
    gl, _ = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert ol.err & orc.ERR_TOPK_RANGE
    assert_layout_equal(gl, ol, w.mode)


def test_capacity_errors_and_canaries():
    w = inputs.small("cap", R=2, T=64, H=256, E=8, K=2, seed=6)
    topk = inputs.gen_topk(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    total = ol.total_rows
    # recv_src_idx with too few rows: error bit, no write past the capacity
    lay = ep.Layout(p, recv_capacity=total - 5)
    guard = torch.full((total + 64,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    lay.recv_src_idx = guard[: total - 5]
    ws = ep.workspace(p)
    ep.get_layout(p, torch.from_numpy(topk).to(DEV), lay, ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) & ep.DEVERR_CAPACITY
    assert (h(guard)[total - 5:] == 0x5A5A5A5A).all()
    # dispatch into too few rows: error bit, rows past the capacity untouched
    lay2 = ep.Layout(p)
    ep.get_layout(p, torch.from_numpy(topk).to(DEV), lay2, ws)
    cap = total - 7
    big = torch.full((total + 8, w.H), 1.5, dtype=torch.bfloat16, device=DEV)
    recv = ep.Recv(p, 1)
    recv.x = big[:cap]
    recv.capacity = cap
    x = inputs.gen_x(w)
    ep.dispatch(p, lay2, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(lay2.err)[0]) & ep.DEVERR_CAPACITY
    assert (big[cap:].float() == 1.5).all().item()
    # the rows that fit are right
    sp = ol.send_pos.reshape(-1)
    src = np.repeat(np.arange(w.R * w.T), w.K)
    ok = (sp >= 0) & (sp < cap)
    g = h(big[:cap].view(torch.uint16))
    assert np.array_equal(g[sp[ok]], x.reshape(-1, w.H)[src[ok]])


def test_low_latency_overflow_flagged():
    w, align, topk = small_case([c for c in SMALL if c[0] == "ll_dup"][0])
    p, po = problems(w, align)
    gl, _ = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert ol.err & orc.ERR_LL_OVERFLOW
    assert int(h(gl.err)[0]) == ol.err


# ----------------------------------------------------------------- workloads
WL = inputs.ORDER


@pytest.mark.parametrize("name", WL)
def test_workload_layout(name):
    w = inputs.WORKLOADS[name]
    say("workload layout", name)
    topk = inputs.gen_topk(w)
    p, po = problems(w)
    gl, _ = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert_layout_equal(gl, ol, w.mode)


def test_workload_tiny_end_to_end():
    w = inputs.WORKLOADS["tiny"]
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    recv = ep.Recv(p, ol.total_rows)
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, recv.x, torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    _, orecv, _ = orc.dispatch(po, x, topk, ol.send_pos, ol.total_rows)
    assert np.array_equal(h(recv.x.view(torch.uint16)), orecv)
    _, oout = orc.combine(po, orecv, wt, ol.send_pos)
    absw = abs_weighted_sum(bf16_to_f32(orecv), wt, ol.send_pos)
    combine_close(h(out.view(torch.uint16)).reshape(-1, w.H), oout.reshape(-1, w.H), absw)


def test_workload_normal_prefill():
    """R8 T4096 H7168 E256 top-8 Zipf(1.2), bf16 contiguous: every receive
    row checked; combine of the identity expert checked on sampled tokens
    against the oracle and on all tokens against x * sum(w)."""
    w = inputs.WORKLOADS["normal_prefill"]
    say("normal_prefill: inputs")
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    gl, ws = gpu_layout(p, topk)
    assert_layout_equal(gl, ol, w.mode)
    total = ol.total_rows
    recv = ep.Recv(p, total)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    say("normal_prefill: dispatch")
    ep.dispatch(p, gl, xg, recv=recv, ws=ws)
    torch.cuda.synchronize()
    xf = x.reshape(-1, w.H)
    src = ol.recv_src_idx
    step = 16384
    for a in range(0, total, step):
        b = min(total, a + step)
        g = h(recv.x[a:b].view(torch.uint16))
        assert np.array_equal(g, xf[src[a:b]]), a
    say("normal_prefill: combine")
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    wg = torch.from_numpy(wt).to(DEV)
    ep.combine(p, gl, recv.x, wg, out)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    go = h(out.view(torch.uint16)).reshape(-1, w.H)
    # sampled tokens against the oracle (identity expert: y rows = x rows)
    toks = np.random.default_rng(1).choice(w.N, 2048, replace=False)
    rows = ol.send_pos.reshape(-1, w.K)[toks]
    uniq = np.unique(rows[rows >= 0])
    y_c = xf[src[uniq]]
    remap = -np.ones(total, np.int64)
    remap[uniq] = np.arange(uniq.size)
    sp_c = np.where(ol.send_pos >= 0, remap[np.maximum(ol.send_pos, 0)], -1).astype(np.int32)
    _, oo = orc.combine(po, y_c, wt, sp_c, toks)
    absw = abs_weighted_sum(bf16_to_f32(y_c), wt, sp_c, toks)
    rel = combine_close(go[toks], oo, absw)
    say("normal_prefill: sampled max rel err", rel)
    # all tokens: out ~ x * sum_k w_k (identity expert, every entry valid)
    xs = bf16_to_f32(xf).astype(np.float64)
    ws_ = wt.reshape(-1, w.K).astype(np.float64).sum(axis=1)[:, None]
    ref = xs * ws_
    gf = bf16_to_f32(go).astype(np.float64)
    assert (np.abs(gf - ref) <= 1e-2 * np.abs(ref) + 2.0 ** -16 * np.abs(xs) * ws_).all()


def test_workload_ll_decode():
    """R8 T128 H7168 E256 top-8, low-latency packed layout, FP8 with fp32
    scales: every filled row and scale; combine of random expert outputs."""
    w = inputs.WORKLOADS["ll_decode"]
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    gl, ws = gpu_layout(p, topk)
    assert_layout_equal(gl, ol, w.mode)
    cap = w.E * w.R * w.T
    recv = ep.Recv(p, cap)
    say("ll_decode: dispatch")
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    err, oc, osc = orc.dispatch(po, x, topk, ol.send_pos, cap)
    rows = np.sort(ol.send_pos[ol.send_pos >= 0])
    gr = h(recv.x[torch.from_numpy(rows).to(DEV)])
    assert np.array_equal(gr, oc[rows])
    gsc = h(recv.scales)
    si = np.concatenate([_scale_index(w, int(r), cap) for r in rows])
    assert np.array_equal(gsc[si], osc[si])
    say("ll_decode: combine")
    yc = inputs.gen_y(w, rows.size)
    y = torch.zeros((cap, w.H), dtype=torch.bfloat16, device=DEV)
    y[torch.from_numpy(rows).to(DEV)] = torch.from_numpy(yc).view(torch.bfloat16).to(DEV)
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, y, torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    remap = -np.ones(cap, np.int64)
    remap[rows] = np.arange(rows.size)
    sp_c = np.where(ol.send_pos >= 0, remap[np.maximum(ol.send_pos, 0)], -1).astype(np.int32)
    _, oo = orc.combine(po, yc, wt, sp_c)
    absw = abs_weighted_sum(bf16_to_f32(yc), wt, sp_c)
    rel = combine_close(h(out.view(torch.uint16)).reshape(-1, w.H), oo.reshape(-1, w.H), absw)
    say("ll_decode: max rel err", rel)


def test_workload_fp8_train():
    """R16 T8192 H4096 E128 top-8 Zipf(1.0), outlier channels, FP8 with
    UE8M0 scales, column-major: sampled tokens' codes and scales in all
    their rows; combine of random expert outputs on sampled tokens."""
    w = inputs.WORKLOADS["fp8_train"]
    say("fp8_train: inputs")
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    gl, ws = gpu_layout(p, topk)
    assert_layout_equal(gl, ol, w.mode)
    cap = ol.total_rows
    recv = ep.Recv(p, cap)
    say("fp8_train: dispatch")
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    toks = np.sort(np.random.default_rng(2).choice(w.N, 1024, replace=False))
    # oracle codes of the sampled tokens: a one-rank problem with one row per token
    sub = orc.Problem(1, toks.size, w.H, 1, 1, quant=w.quant)
    xs = x.reshape(-1, w.H)[toks]
    _, sc_codes, sc_scales = orc.dispatch(sub, xs, np.zeros((1, toks.size, 1), np.int32),
                                          np.arange(toks.size, dtype=np.int32), toks.size)
    sp = ol.send_pos.reshape(-1, w.K)[toks]
    gsc = recv.scales
    for k in range(w.K):
        rows = sp[:, k]
        gr = h(recv.x[torch.from_numpy(rows.astype(np.int64)).to(DEV)])
        assert np.array_equal(gr, sc_codes), k
        for g in range(w.G):
            idx = torch.from_numpy(g * cap + rows.astype(np.int64)).to(DEV)
            assert np.array_equal(h(gsc[idx]), sc_scales[g * toks.size:(g + 1) * toks.size]), (k, g)
    say("fp8_train: combine")
    del recv
    torch.cuda.empty_cache()
    rows = np.unique(sp[sp >= 0])
    yc = inputs.gen_y(w, rows.size)
    y = torch.zeros((cap, w.H), dtype=torch.bfloat16, device=DEV)
    y[torch.from_numpy(rows.astype(np.int64)).to(DEV)] = torch.from_numpy(yc).view(torch.bfloat16).to(DEV)
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, y, torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    remap = -np.ones(cap, np.int64)
    remap[rows] = np.arange(rows.size)
    sp_c = np.where(ol.send_pos >= 0, remap[np.maximum(ol.send_pos, 0)], -1).astype(np.int32)
    _, oo = orc.combine(po, yc, wt, sp_c, toks)
    absw = abs_weighted_sum(bf16_to_f32(yc), wt, sp_c, toks)
    go = h(out.view(torch.uint16)).reshape(-1, w.H)[toks]
    rel = combine_close(go, oo, absw)
    say("fp8_train: sampled max rel err", rel)


def test_workload_messages():
    """R64 T256 H7168 E256 top-8: every message region byte, the message
    table, arena bases and every descriptor."""
    w = inputs.WORKLOADS["messages"]
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert_layout_equal(gl, ol, w.mode)
    say("messages: pack")
    om = _messages_compare(w, p, po, gl, topk, x, wt, ws)
    say("messages: descriptors", om.num_desc)


def test_combine_without_expert_rows_flags_every_entry():
    """y with zero rows: nothing is read, every routed entry is flagged, and
    the output is zero."""
    w = inputs.small("norows", R=2, T=9, H=256, E=8, K=3, seed=8)
    topk = inputs.gen_topk(w)
    p, _ = problems(w)
    gl, _ = gpu_layout(p, topk)
    out = torch.full((w.R, w.T, w.H), 3.0, dtype=torch.bfloat16, device=DEV)
    y = torch.empty((0, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, y, torch.from_numpy(inputs.gen_weights(w)).to(DEV), out)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) & ep.DEVERR_CAPACITY
    assert (out.float() == 0).all().item()


@pytest.mark.parametrize("quant", [QF, QU])
def test_fp8_normal_capacity_and_scale_canaries(quant):
    """FP8 normal dispatch into too few rows: error bit, codes and scales of
    the rows that fit are right, nothing is written past either buffer."""
    w = inputs.small("fp8cap", R=2, T=48, H=256, E=8, K=3, quant=quant, seed=12)
    topk = inputs.gen_topk(w)
    x = inputs.gen_x(w)
    p, po = problems(w, align=2)
    ol = orc.layout(po, topk)
    gl, ws = gpu_layout(p, topk)
    cap = ol.total_rows - 9
    recv = ep.Recv(p, cap)
    big_x = torch.full((cap + 4, w.H), 0xA5, dtype=torch.uint8, device=DEV)
    recv.x = big_x[:cap]
    dt = torch.float32 if quant == QF else torch.uint8
    big_s = torch.full((w.G * cap + 64,), 7, dtype=dt, device=DEV)
    recv.scales = big_s[: w.G * cap]
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) & ep.DEVERR_CAPACITY
    assert (h(big_x[cap:]) == 0xA5).all()
    assert (h(big_s[w.G * cap:]) == 7).all()
    _, oc, osc = orc.dispatch(po, x, topk, ol.send_pos, ol.total_rows)
    rows = ol.send_pos[(ol.send_pos >= 0) & (ol.send_pos < cap)]
    assert np.array_equal(h(recv.x)[rows], oc[rows])
    gsc = h(big_s)
    for r in rows:
        g = np.arange(w.G)
        assert np.array_equal(gsc[g * cap + r], osc[g * ol.total_rows + r]), r
