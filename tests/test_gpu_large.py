"""Buffers past 32-bit offsets, through the C ABI against the oracle: receive
buffers past 2^31 sixteen-byte vectors (over 32 GiB), where a row index
(int32) times the row's vectors overflows 32 bits, and message arenas past
4 GiB.

- normal mode, bf16, hidden 7168, top-32 of 256 experts, 8 ranks x 9400
  tokens: 2,406,400 receive rows, 34.5 GB; the separate layout, dispatch
  and combine calls, the combine's kernel the prefill shape uses;
- low-latency FP8 (fp32 scales) through the fused call, 8 ranks x 2400
  tokens, 256 experts: 4,915,200 slots, 35.2 GB of codes; the combine then
  reads a 70.5 GB bf16 expert output in the same layout;
- message mode with bf16 payloads, 8 ranks x 8192 tokens: send and receive
  arenas of 5.1 GB (byte offsets past 32 bits) through packer, delivery
  and receiver.

Every layout output is compared whole; receive rows, codes and scales and
the combined outputs on sampled tokens, among them the tokens whose rows
lie furthest into the buffers (past 2^31 vectors)."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import (DEV, abs_weighted_sum, assert_layout_equal, bf16_to_f32, combine_close,
                      gpu_layout, h, problems, say)

pytestmark = pytest.mark.gpu

VEC = 16
LIMIT = 1 << 31  # vectors


def need_memory(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of free device memory, has {free / 2**30:.0f}")


def sample_tokens(send_pos, K, n_far=96, n_rand=96, seed=0):
    """Tokens whose largest row is largest, plus random ones (sorted)."""
    sp = send_pos.reshape(-1, K)
    far = np.argsort(sp.max(axis=1), kind="stable")[-n_far:]
    rest = np.setdiff1d(np.arange(sp.shape[0]), far)
    rnd = np.random.default_rng(seed).choice(rest, n_rand, replace=False)
    return np.sort(np.concatenate([far, rnd]))


def rows_of(tensor, rows):
    """Rows (or elements) of a device tensor; bf16 as its uint16 patterns."""
    t = tensor[torch.from_numpy(np.asarray(rows, np.int64)).to(DEV)]
    if t.dtype == torch.bfloat16:
        return h(t.view(torch.int16)).view(np.uint16)
    return h(t)


def check_combine(w, p, po, gl, send_pos, y, yc, rows, wt, toks):
    """Combine on the GPU; the oracle's on the sampled tokens, from `yc`
    (the sampled rows' expert outputs, in the order of `rows`) and the
    oracle's `send_pos`."""
    out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
    ep.combine(p, gl, y, torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    sp = send_pos
    cap = int(y.shape[0])
    remap = -np.ones(cap, np.int64)
    remap[rows] = np.arange(rows.size)
    sp_c = np.where(sp >= 0, remap[np.maximum(sp, 0)], -1).astype(np.int32)
    err, oo = orc.combine(po, yc, wt, sp_c, toks)
    assert err == 0
    absw = abs_weighted_sum(bf16_to_f32(yc), wt, sp_c, toks)
    go = h(out.view(torch.uint16)).reshape(-1, w.H)[toks]
    say("sampled max rel err", combine_close(go, oo, absw))


def test_normal_bf16_rows_past_2_31_vectors():
    w = inputs.small("large_normal", R=8, T=9400, H=7168, E=256, K=32, seed=23)
    V = w.H * 2 // VEC
    need_memory(48 << 30)
    say("large normal: inputs")
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    cap = ol.total_rows
    assert (cap - 1) * V >= LIMIT
    say("large normal: layout", cap, "rows")
    gl, ws = gpu_layout(p, topk, recv_cap=cap)
    assert_layout_equal(gl, ol, w.mode)
    recv = ep.Recv(p, cap)
    recv.x.view(torch.int16)[-1].fill_(0x3333)
    say("large normal: dispatch")
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    toks = sample_tokens(ol.send_pos, w.K)
    sp = ol.send_pos.reshape(-1, w.K)[toks]
    assert int(sp.max()) * V >= LIMIT
    xs = x.reshape(-1, w.H)[toks]
    for k in range(w.K):
        assert np.array_equal(rows_of(recv.x, sp[:, k]), xs), k
    # the last row of the buffer is the last token routed to the last expert
    last = int(ol.recv_src_idx[cap - 1])
    assert np.array_equal(rows_of(recv.x, [cap - 1])[0],
                          x.reshape(-1, w.H)[last])
    say("large normal: combine (identity expert: the receive rows)")
    rows = np.unique(sp[sp >= 0])
    yc = x.reshape(-1, w.H)[ol.recv_src_idx[rows]]  # a receive row is its token's x
    check_combine(w, p, po, gl, ol.send_pos, recv.x, yc, rows, wt, toks)
    del recv, gl, ws
    torch.cuda.empty_cache()


def test_low_latency_fp8_fused_slots_past_2_31_vectors():
    w = inputs.small("large_ll", R=8, T=2400, H=7168, E=256, K=8, mode=ep.MODE_LOW_LATENCY,
                     quant=ep.QUANT_FP8_F32, seed=29)
    RT, G = w.R * w.T, w.G
    need_memory(80 << 30)
    say("large ll: inputs")
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    cap = ep.max_recv_rows(p)
    assert cap == w.E * RT and (cap - 1) * (w.H // VEC) >= LIMIT
    lay = ep.Layout(p)
    recv = ep.Recv(p, cap)
    say("large ll: fused layout + dispatch", cap, "slots")
    tk = torch.from_numpy(topk).to(DEV)
    ep.dispatch_fused(p, tk, lay, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv,
                      ep.workspace(p))
    torch.cuda.synchronize()
    assert_layout_equal(lay, ol, w.mode)
    toks = sample_tokens(ol.send_pos, w.K)
    sp = ol.send_pos.reshape(-1, w.K)[toks]
    assert int(sp.max()) * (w.H // VEC) >= LIMIT
    # the oracle's codes and scales of the sampled tokens: one row per token
    sub = orc.Problem(1, toks.size, w.H, 1, 1, quant=w.quant)
    err, codes, scales = orc.dispatch(sub, x.reshape(-1, w.H)[toks],
                                      np.zeros((1, toks.size, 1), np.int32),
                                      np.arange(toks.size, dtype=np.int32), toks.size)
    assert err == 0
    for k in range(w.K):
        r = sp[:, k].astype(np.int64)
        assert np.array_equal(rows_of(recv.x, r), codes), k
        e, pos = r // RT, r % RT
        for g in range(G):
            got = rows_of(recv.scales.view(torch.int32), (e * G + g) * RT + pos)
            assert np.array_equal(got, scales[g * toks.size:(g + 1) * toks.size].view(np.int32)), (k, g)
    del recv
    torch.cuda.empty_cache()
    say("large ll: combine over a 70.5 GB expert output")
    rows = np.unique(sp[sp >= 0])
    yc = inputs.gen_y(w, rows.size)
    y = torch.zeros((cap, w.H), dtype=torch.bfloat16, device=DEV)
    y[torch.from_numpy(rows.astype(np.int64)).to(DEV)] = torch.from_numpy(yc).view(torch.bfloat16).to(DEV)
    check_combine(w, p, po, lay, ol.send_pos, y, yc, rows, wt, toks)
    del y, lay
    torch.cuda.empty_cache()


def test_message_arenas_past_4_gib():
    """Message mode, bf16 payloads, 8 ranks x 8192 tokens, 64 experts: send
    and receive arenas over 4 GiB (byte offsets past 32 bits) in 2 MiB
    regions.  The table, arena bases and every descriptor against the
    oracle; every message region of the send arena and, after the loopback
    delivery, of the receive arena; the receiver's counts, and its rows and
    source indices on sampled tokens (an unpacked entry sits where
    low-latency dispatch of the same routing puts it, and is its token's
    row)."""
    w = inputs.small("large_msg", R=8, T=8192, H=7168, E=64, K=8, mode=ep.MODE_MESSAGES,
                     quant=ep.QUANT_NONE, seed=31)
    need_memory(80 << 30)
    say("large messages: inputs")
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    gl, ws = gpu_layout(p, topk)
    assert_layout_equal(gl, ol, w.mode)
    send_cap, desc_cap = ep.messages_capacity(p, ol.num_tokens_per_rank)
    assert send_cap > 1 << 32
    msgs = ep.Messages(p, send_cap, desc_cap)
    say("large messages: pack", send_cap, "bytes")
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), msgs=msgs,
                topk_idx=torch.from_numpy(topk).to(DEV), topk_weights=torch.from_numpy(wt).to(DEV),
                ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
    assert om.err == 0
    assert np.array_equal(h(msgs.table), om.table)
    assert np.array_equal(h(msgs.arena_base), om.arena_base)
    assert int(h(msgs.num_descriptors)[0]) == om.num_desc
    assert np.array_equal(h(msgs.descriptors)[:om.num_desc], om.desc)
    sd = om.table.reshape(-1, 8)
    for off, reg in sd[:, [0, 2]]:
        if reg > 0:
            assert np.array_equal(h(msgs.send_arena[off:off + reg]), om.send_arena[off:off + reg]), off
    recv_cap = int(om.arena_base[1, -1])
    assert recv_cap > 1 << 32
    say("large messages: delivery", recv_cap, "bytes")
    arena = torch.full((recv_cap,), 0xA5, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_execute(p, msgs, arena, err)
    torch.cuda.synchronize()
    assert int(h(err)[0]) == 0
    e1, oarena = orc.messages_execute(po, om, recv_cap)
    assert e1 == 0
    for off, reg in sd[:, [1, 2]]:
        if reg > 0:
            assert np.array_equal(h(arena[off:off + reg]), oarena[off:off + reg]), off
    del oarena, om
    say("large messages: receiver")
    out, cnt, src = ep.unpack_buffers(p)
    ep.messages_unpack(p, msgs, arena, gl.num_tokens_per_expert, out, cnt, src, err)
    torch.cuda.synchronize()
    assert int(h(err)[0]) == 0
    oll = orc.layout(orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=orc.MODE_LL), topk)
    assert np.array_equal(h(cnt), oll.recv_tokens_per_expert)
    toks = sample_tokens(oll.send_pos, w.K)
    sp = oll.send_pos.reshape(-1, w.K)[toks]
    xs = x.reshape(-1, w.H)[toks]
    for k in range(w.K):
        assert np.array_equal(rows_of(out.x, sp[:, k]), xs), k
        assert np.array_equal(rows_of(src, sp[:, k]), toks.astype(np.int32)), k
    del out, cnt, src, arena, msgs, gl, ws
    torch.cuda.empty_cache()
