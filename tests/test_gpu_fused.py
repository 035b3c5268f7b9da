"""GPU parity of ep_dispatch_fused (layout and dispatch in one call, the
layout's last step taken by the dispatch kernel) through the C ABI: every
layout output and every dispatched row and scale equal those of separate
ep_get_layout + ep_dispatch calls bit for bit, and the oracle's."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import DEV, LAYOUT_FIELDS, assert_layout_equal, h, say, sweep_cases

pytestmark = pytest.mark.gpu

N, L, QF, QU = ep.MODE_NORMAL, ep.MODE_LOW_LATENCY, ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0
CASES = [
    # name, R, T, H, E, K, mode, quant, align, masked, duplicates
    ("small_direct", 2, 17, 256, 8, 3, N, 0, 1, 0.1, 0.0),
    ("normal_bf16", 4, 700, 128, 32, 6, N, 0, 1, 0.0, 0.0),
    ("normal_align", 4, 500, 256, 16, 4, N, QF, 4, 0.2, 0.0),
    ("normal_ue8m0", 8, 300, 384, 64, 8, N, QU, 2, 0.05, 0.1),
    ("ll_fp8", 8, 128, 512, 64, 8, L, QF, 1, 0.0, 0.0),
    ("ll_bf16_dups", 4, 200, 128, 8, 8, L, 0, 1, 0.1, 0.4),
    ("experts_over_tokens", 2, 110, 128, 2048, 64, N, 0, 1, 0.0, 0.0),
    ("ll_experts_over_tokens", 2, 100, 128, 1024, 40, L, QF, 1, 0.0, 0.0),
    # every FP8 row split the normal-mode launcher picks, fused: one
    # wavefront of one pair per lane (hidden 1024), four wavefronts of one
    # pair (2048), one wavefront of four pairs (4096: the training shape's
    # kernel), twelve wavefronts of two pairs (20480); both scale forms,
    # alignment, masked and duplicate ids
    ("fp8_h1024_one_wave_ue8", 4, 600, 1024, 32, 8, N, QU, 4, 0.1, 0.2),
    ("fp8_h1024_one_wave_f32", 4, 600, 1024, 32, 8, N, QF, 2, 0.05, 0.0),
    ("fp8_h2048_four_waves_f32", 4, 300, 2048, 32, 8, N, QF, 8, 0.1, 0.2),
    ("fp8_h2048_four_waves_ue8", 4, 300, 2048, 32, 8, N, QU, 1, 0.0, 0.0),
    ("fp8_h4096_four_pairs_ue8", 4, 300, 4096, 32, 8, N, QU, 8, 0.1, 0.2),
    ("fp8_h4096_four_pairs_f32", 4, 300, 4096, 32, 8, N, QF, 2, 0.05, 0.1),
    ("fp8_h20480_two_pairs_f32", 2, 400, 20480, 16, 8, N, QF, 4, 0.1, 0.1),
    ("fp8_h20480_two_pairs_ue8", 2, 400, 20480, 16, 8, N, QU, 1, 0.0, 0.2),
    ("ll_fp8_h4096_ue8", 4, 200, 4096, 32, 8, L, QU, 1, 0.1, 0.0),
]


def buffers(p, w, total):
    lay = ep.Layout(p)
    recv = ep.Recv(p, total)
    recv.x.view(torch.uint8).fill_(0x33)
    if recv.scales is not None:
        recv.scales.view(torch.uint8).fill_(0x33)
    return lay, recv


def draw(i):
    """A random case: both modes, every payload format, alignment, masked and
    duplicate ids, and token counts on both sides of the one-launch layout's
    limit (6,144 entries)."""
    g = np.random.default_rng(5300 + i)
    mode = int(g.choice([N, L]))
    R = int(g.choice([1, 2, 3, 4, 8, 16] if mode == N else [1, 2, 4, 8]))
    E = R * int(g.integers(1, 17 if mode == N else 9))
    K = int(g.integers(1, min(E, 10) + 1))
    T = int(g.choice([1, 40, 300, 1000, 2100] if mode == N else [1, 40, 200, 500]))
    quant = int(g.choice([0, QF, QU]))
    H = int(8 * g.integers(1, 120)) if quant == 0 else int(128 * g.integers(1, 6))
    align = int(g.choice([1, 1, 2, 8])) if mode == N else 1
    return (f"fuzz{i}", R, T, H, E, K, mode, quant, align, float(g.choice([0.0, 0.1, 0.3])),
            float(g.choice([0.0, 0.3])) if K > 1 else 0.0)


FUZZ = [draw(i) for i in range(sweep_cases(20))]


@pytest.mark.parametrize("c", CASES + FUZZ, ids=[c[0] for c in CASES + FUZZ])
def test_fused_equals_separate_calls_and_oracle(c):
    name, R, T, H, E, K, mode, quant, align, mfrac, dfrac = c
    say("fused", c)
    w = inputs.small(f"fused_{name}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=97)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=4)
    x = inputs.gen_x(w)
    p = ep.Problem(R, T, H, E, K, align=align, mode=mode, quant=quant)
    po = orc.Problem(R, T, H, E, K, align=align, mode=mode, quant=quant)
    ol = orc.layout(po, topk)
    cap = ep.max_recv_rows(p)
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    # fused
    lf, rf = buffers(p, w, cap)
    wsf = ep.workspace(p)
    ep.dispatch_fused(p, tk, lf, xg, rf, wsf)
    # separate
    ls, rs = buffers(p, w, cap)
    wss = ep.workspace(p)
    ep.get_layout(p, tk, ls, wss)
    ep.dispatch(p, ls, xg, recv=rs, ws=wss)
    torch.cuda.synchronize()
    for f in LAYOUT_FIELDS + ["err"]:
        a, b = getattr(lf, f), getattr(ls, f)
        if a is not None:
            assert torch.equal(a, b), f
    assert_layout_equal(lf, ol, mode)
    if mode == N:
        assert torch.equal(lf.recv_src_idx[: ol.total_rows], ls.recv_src_idx[: ol.total_rows])
    sp = ol.send_pos[ol.send_pos >= 0]
    rows = torch.from_numpy(np.unique(sp).astype(np.int64)).to(DEV)
    assert torch.equal(rf.x[rows], rs.x[rows])
    _, orecv, osc = orc.dispatch(po, x, topk, ol.send_pos, cap)
    g = h(rf.x.view(torch.uint16) if quant == 0 else rf.x)
    rn = rows.cpu().numpy()
    assert np.array_equal(g[rn], orecv[rn])
    if quant:
        assert torch.equal(rf.scales, rs.scales)
        G, RT = H // 128, R * T
        gi = np.arange(G)
        si = ((rn[:, None] // RT * G + gi) * RT + rn[:, None] % RT if mode == L
              else gi[None, :] * cap + rn[:, None]).reshape(-1)
        assert np.array_equal(h(rf.scales)[si], osc[si])


@pytest.mark.parametrize("name", ["ll_decode", "normal_prefill"])
def test_fused_workload(name):
    """The low-latency decode and prefill shapes: every layout output against
    the oracle and every dispatched row against the separate calls."""
    w = inputs.WORKLOADS[name]
    say("fused workload", name)
    topk, x = inputs.gen_topk(w), inputs.gen_x(w)
    p = ep.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    po = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    ol = orc.layout(po, topk)
    cap = ol.total_rows
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    lf = ep.Layout(p, recv_capacity=cap)
    rf = ep.Recv(p, cap)
    ep.dispatch_fused(p, tk, lf, xg, rf, ep.workspace(p))
    torch.cuda.synchronize()
    assert_layout_equal(lf, ol, w.mode)
    ls = ep.Layout(p, recv_capacity=cap)
    rs = ep.Recv(p, cap)
    wss = ep.workspace(p)
    ep.get_layout(p, tk, ls, wss)
    ep.dispatch(p, ls, xg, recv=rs, ws=wss)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.unique(ol.send_pos[ol.send_pos >= 0]).astype(np.int64)).to(DEV)
    step = 1 << 14
    for a in range(0, rows.numel(), step):
        r = rows[a:a + step]
        assert torch.equal(rf.x[r], rs.x[r]), a
    if w.quant:
        G, RT = w.G, w.R * w.T
        gi = torch.arange(G, device=DEV)
        si = ((rows // RT)[:, None] * G + gi[None, :]) * RT + (rows % RT)[:, None]
        assert torch.equal(rf.scales[si.reshape(-1)], rs.scales[si.reshape(-1)])


def test_fused_workload_fp8_train():
    """The FP8 training shape (16 x 8192 tokens, hidden 4096, 128 experts,
    top-8 Zipf(1.0), outlier channels, UE8M0 scales) through the fused call,
    in the launch configuration the bench times (one wavefront of four pairs
    per lane): every layout output against the oracle; every code row and
    the whole column-major scale array against the separate calls; 1,024
    sampled tokens' codes and scales in all their rows against the oracle."""
    w = inputs.WORKLOADS["fp8_train"]
    say("fused workload fp8_train: inputs")
    topk, x = inputs.gen_topk(w), inputs.gen_x(w)
    p = ep.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    po = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    ol = orc.layout(po, topk)
    cap = ol.total_rows
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    lf = ep.Layout(p, recv_capacity=cap)
    rf = ep.Recv(p, cap)
    rf.scales.fill_(0x5A)
    say("fused workload fp8_train: fused call")
    ep.dispatch_fused(p, tk, lf, xg, rf, ep.workspace(p))
    torch.cuda.synchronize()
    assert_layout_equal(lf, ol, w.mode)
    say("fused workload fp8_train: separate calls")
    ls = ep.Layout(p, recv_capacity=cap)
    rs = ep.Recv(p, cap)
    rs.scales.fill_(0x5A)
    wss = ep.workspace(p)
    ep.get_layout(p, tk, ls, wss)
    ep.dispatch(p, ls, xg, recv=rs, ws=wss)
    torch.cuda.synchronize()
    assert int(h(ls.err)[0]) == 0
    step = 1 << 14
    for a in range(0, cap, step):
        assert torch.equal(rf.x[a:a + step], rs.x[a:a + step]), a
    assert torch.equal(rf.scales, rs.scales)
    say("fused workload fp8_train: sampled tokens against the oracle")
    toks = np.sort(np.random.default_rng(5).choice(w.N, 1024, replace=False))
    sub = orc.Problem(1, toks.size, w.H, 1, 1, quant=w.quant)
    _, codes, scales = orc.dispatch(sub, x.reshape(-1, w.H)[toks], np.zeros((1, toks.size, 1), np.int32),
                                    np.arange(toks.size, dtype=np.int32), toks.size)
    sp = ol.send_pos.reshape(-1, w.K)[toks]
    for k in range(w.K):
        rows = sp[:, k].astype(np.int64)
        assert np.array_equal(h(rf.x[torch.from_numpy(rows).to(DEV)]), codes), k
        for g in range(w.G):
            got = h(rf.scales[torch.from_numpy(g * cap + rows).to(DEV)])
            assert np.array_equal(got, scales[g * toks.size:(g + 1) * toks.size]), (k, g)
