"""Randomised GPU parity sweep: many small problems drawn from one seed,
spanning ranks, tokens (including empty), hidden sizes, experts, top-k,
alignment, masked and duplicate ids, all three modes and all payload
formats, and message region sizes that force descriptor splits.  Every
output is compared with the oracle to the same bar as the fixed cases."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import (DEV, abs_weighted_sum, assert_layout_equal, bf16_to_f32, combine_close,
                      gpu_layout, h, problems, say, sweep_cases)

pytestmark = pytest.mark.gpu


def draw(i):
    g = np.random.default_rng(4242 + i)
    R = int(g.choice([1, 2, 3, 4, 5, 8, 13, 16, 32]))
    L = int(g.integers(1, 9))
    E = R * L
    K = int(g.integers(1, min(E, 12) + 1))
    T = int(g.choice([0, 1, 3, 17, 64, 129, 300]))
    mode = int(g.choice([0, 0, 1, 2]))
    if mode == 1:  # low-latency buffers hold E*R*T rows: keep them small
        R = min(R, 8)
        L = min(L, 8)
        E = R * L
        K = min(K, E)
        T = min(T, 64)
    quant = int(g.choice([0, 1, 2]))
    if quant == 0:
        H = int(8 * g.integers(1, 160))
    else:
        H = int(128 * g.integers(1, 9))
    align = int(g.choice([1, 1, 2, 4])) if mode == 0 else 1
    mfrac = float(g.choice([0.0, 0.1, 0.4]))
    dfrac = float(g.choice([0.0, 0.0, 0.3])) if K > 1 else 0.0
    rb = int(g.choice([64, 256, 4096, 2 << 20]))
    return dict(R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, align=align, mfrac=mfrac,
                dfrac=dfrac, rb=rb)


CASES = [draw(i) for i in range(sweep_cases(48))]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_fuzz(i):
    c = CASES[i]
    say("fuzz", i, c)
    w = inputs.small(f"fuzz{i}", R=c["R"], T=c["T"], H=c["H"], E=c["E"], K=c["K"],
                     mode=c["mode"], quant=c["quant"], seed=900 + i, region_bytes=c["rb"],
                     epoch=3 + i)
    R, T, H, E, K = w.R, w.T, w.H, w.E, w.K
    if T > 0:
        topk = inputs.masked_topk(w, inputs.gen_topk(w), c["mfrac"], c["dfrac"], seed=i)
        x = inputs.gen_x(w)
        wt = inputs.gen_weights(w)
    else:
        topk = np.zeros((R, 0, K), np.int32)
        x = np.zeros((R, 0, H), np.uint16)
        wt = np.zeros((R, 0, K), np.float32)
    p, po = problems(w, c["align"])
    gl, ws = gpu_layout(p, topk)
    ol = orc.layout(po, topk)
    assert_layout_equal(gl, ol, w.mode)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    if w.mode == ep.MODE_MESSAGES:
        counts = h(gl.num_tokens_per_rank)
        send_cap, desc_cap = ep.messages_capacity(p, counts)
        msgs = ep.Messages(p, send_cap, desc_cap)
        ep.dispatch(p, gl, xg, msgs=msgs, topk_idx=torch.from_numpy(topk).to(DEV),
                    topk_weights=torch.from_numpy(wt).to(DEV), ws=ws)
        torch.cuda.synchronize()
        om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
        assert int(h(gl.err)[0]) == 0 and om.err == 0
        table = h(msgs.table)
        assert np.array_equal(table, om.table)
        assert np.array_equal(h(msgs.arena_base), om.arena_base)
        nd = int(h(msgs.num_descriptors)[0])
        assert nd == om.num_desc
        assert np.array_equal(h(msgs.descriptors)[:nd], om.desc)
        arena = h(msgs.send_arena)
        for off, reg in table.reshape(-1, 8)[:, [0, 2]]:
            if reg > 0:
                assert np.array_equal(arena[off:off + reg], om.send_arena[off:off + reg])
        return
    cap = ol.total_rows if w.mode == ep.MODE_NORMAL else E * R * T
    recv = ep.Recv(p, cap)
    ep.dispatch(p, gl, xg, recv=recv, ws=ws)
    torch.cuda.synchronize()
    _, orecv, osc = orc.dispatch(po, x, topk, ol.send_pos, cap)
    assert int(h(gl.err)[0]) == ol.err
    rows = ol.send_pos[ol.send_pos >= 0]
    grecv = h(recv.x.view(torch.uint16) if w.quant == 0 else recv.x)
    assert np.array_equal(grecv[rows], orecv[rows])
    if w.quant != 0 and rows.size:
        G, RT = w.G, R * T
        gsc = h(recv.scales)
        g = np.arange(G)
        for r in rows:
            si = ((r // RT * G + g) * RT + r % RT) if w.mode == ep.MODE_LOW_LATENCY else g * cap + r
            assert np.array_equal(gsc[si], osc[si]), r
    # combine of random expert outputs in the receive layout
    y = inputs.gen_y(w, max(cap, 1), seed_offset=i)
    out = torch.empty((R, T, H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, torch.from_numpy(y).view(torch.bfloat16).to(DEV),
               torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    _, oout = orc.combine(po, y, wt, ol.send_pos)
    go = h(out.view(torch.uint16)).reshape(-1, H)
    if go.size:
        combine_close(go, oout.reshape(-1, H), abs_weighted_sum(bf16_to_f32(y), wt, ol.send_pos))
