"""Pins of the oracle's message delivery (loopback descriptor execution) and
receiver (unpack into the low-latency layout), on the CPU.

- Execution: every message region arrives byte for byte at its receive
  offset, nothing outside the regions is touched, and the descriptor order
  does not matter (the regions are disjoint), so flags may go last.
- Unpack: equals low-latency dispatch of the same routing (codes or bf16
  rows, scales, recv_src_idx, recv_count) -- a second derivation of the
  same slots, through the layout instead of the messages.
- Unpack, brute force: a struct-level Python parse of the send arena,
  slots counted by sorting all entries, on tiny shapes.
- Malformed messages (flag, header) and short arenas are rejected with the
  error bits and leave their rows unwritten.
"""
import struct

import numpy as np
import pytest

from combine_ep_get_layout_amd import inputs
from oracle import oracle as orc

SHAPES = [
    # R, T, H, E, K, quant, region bytes
    (1, 9, 128, 4, 2, orc.Q_FP8_F32, 256),
    (2, 17, 256, 8, 3, orc.Q_FP8_F32, 64),
    (3, 12, 128, 6, 2, orc.Q_NONE, 4096),
    (4, 20, 256, 16, 4, orc.Q_FP8_UE8M0, 512),
    (5, 7, 384, 10, 5, orc.Q_FP8_F32, 2 << 20),
    (4, 33, 128, 8, 8, orc.Q_NONE, 128),
]


def build_case(shape, seed, mfrac=0.0, dfrac=0.0):
    R, T, H, E, K, quant, rb = shape
    w = inputs.small(f"recv{seed}", R=R, T=T, H=H, E=E, K=K, mode=orc.MODE_MSG, quant=quant,
                     seed=seed, region_bytes=rb)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=seed)
    x, wt = inputs.gen_x(w), inputs.gen_weights(w)
    pm = orc.Problem(R, T, H, E, K, mode=orc.MODE_MSG, quant=quant, region_bytes=rb, epoch=11 + seed)
    # sizes from the oracle itself: a first pass with no room writes nothing
    # but still reports the arena bases and the descriptor count
    probe = orc.messages(pm, x, topk, wt, 0, 0)
    send_cap, desc_cap = int(probe.arena_base[0][-1]), probe.num_desc
    m = orc.messages(pm, x, topk, wt, send_cap, desc_cap)
    assert m.err == 0
    return w, pm, topk, x, wt, m


def regions(m):
    t = m.table.reshape(-1, 8)
    return [(int(r[0]), int(r[1]), int(r[2])) for r in t if r[3] > 0]


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_execute_delivers_every_region_and_nothing_else(si):
    w, pm, topk, x, wt, m = build_case(SHAPES[si], seed=si)
    cap = int(m.arena_base[1][-1])
    arena = np.full(cap + 64, 0xA5, np.uint8)
    err, arena = orc.messages_execute(pm, m, cap, arena)
    assert err == 0
    touched = np.zeros(arena.size, bool)
    for so, ro, reg in regions(m):
        assert np.array_equal(arena[ro:ro + reg], m.send_arena[so:so + reg])
        touched[ro:ro + reg] = True
    assert (arena[~touched] == 0xA5).all()
    # any order of the descriptors gives the same bytes (regions are disjoint)
    rev = orc.Messages(m.err, m.send_arena, m.table, m.arena_base, m.desc[::-1].copy(), m.num_desc)
    err2, arena2 = orc.messages_execute(pm, rev, cap, np.full(cap + 64, 0xA5, np.uint8))
    assert err2 == 0 and np.array_equal(arena2, arena)


def ll_reference(w, topk, x):
    """Low-latency layout and dispatch of the same routing (oracle)."""
    pl = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=orc.MODE_LL, quant=w.quant)
    lay = orc.layout(pl, topk)
    err, recv, sc = orc.dispatch(pl, x, topk, lay.send_pos, w.E * w.R * w.T)
    return lay, recv, sc


@pytest.mark.parametrize("si", range(len(SHAPES)))
@pytest.mark.parametrize("mask", [(0.0, 0.0), (0.3, 0.0), (0.1, 0.3)])
def test_unpack_equals_low_latency_dispatch(si, mask):
    w, pm, topk, x, wt, m = build_case(SHAPES[si], seed=10 + si, mfrac=mask[0], dfrac=mask[1])
    cap = int(m.arena_base[1][-1])
    _, arena = orc.messages_execute(pm, m, cap)
    lay, recv, sc = ll_reference(w, topk, x)
    u = orc.messages_unpack(pm, arena, m.table, lay.num_tokens_per_expert)
    assert u.err == lay.err  # both flag the same low-latency overflow, if any
    assert np.array_equal(u.recv_count, lay.recv_tokens_per_expert)
    rows = np.unique(lay.send_pos[lay.send_pos >= 0])
    assert np.array_equal(u.recv[rows], recv[rows])
    assert np.array_equal(u.recv_src_idx[rows], lay.recv_src_idx[rows])
    written = np.zeros(u.recv_src_idx.size, bool)
    written[rows] = True
    assert (u.recv_src_idx[~written] == -1).all()
    if w.quant != orc.Q_NONE:
        G, RT = w.G, w.R * w.T
        g = np.arange(G)
        si_ = ((rows // RT)[:, None] * G + g[None, :]) * RT + (rows % RT)[:, None]
        assert np.array_equal(u.scales[si_], sc[si_])


def parse_send_arena(w, pm, m):
    """Brute force: {(s, t): (codes or row bytes, scale bytes, ids)} read
    from the send arena with struct, plus the message of each (s, d)."""
    H, K, G = w.H, w.K, w.G
    cb = 2 if w.quant == orc.Q_NONE else 1
    sb = {orc.Q_NONE: 0, orc.Q_FP8_F32: 4, orc.Q_FP8_UE8M0: 1}[w.quant]
    pad = lambda v: (v + 15) // 16 * 16
    tok = {}
    for s in range(w.R):
        for d in range(w.R):
            so, ro, reg, n, body = (int(v) for v in m.table[s, d, :5])
            if n == 0:
                continue
            msg = m.send_arena[so:so + reg].tobytes()
            assert struct.unpack_from("<4I", msg, 0) == (s, d, n, body)
            assert struct.unpack_from("<4I", msg, 16 + body) == (pm.epoch, 0, 0, 0)
            o_codes = 16
            o_sc = o_codes + pad(n * H * cb)
            o_w = o_sc + pad(n * G * sb)
            o_ids = o_w + pad(n * K * 4)
            o_src = o_ids + pad(n * K * 4)
            for j in range(n):
                t = struct.unpack_from("<I", msg, o_src + 4 * j)[0]
                ids = struct.unpack_from(f"<{K}i", msg, o_ids + 4 * K * j)
                codes = msg[o_codes + j * H * cb:o_codes + (j + 1) * H * cb]
                scales = msg[o_sc + j * G * sb:o_sc + (j + 1) * G * sb]
                tok[(s, t)] = (codes, scales, ids)
    return tok


@pytest.mark.parametrize("si", [0, 1, 3, 5])
def test_unpack_bruteforce_tiny(si):
    w, pm, topk, x, wt, m = build_case(SHAPES[si], seed=20 + si, mfrac=0.2)
    cap = int(m.arena_base[1][-1])
    _, arena = orc.messages_execute(pm, m, cap)
    cnt_e = np.zeros((w.R, w.E), np.int32)
    for s in range(w.R):
        for e in topk[s].reshape(-1):
            if e >= 0:
                cnt_e[s, e] += 1
    u = orc.messages_unpack(pm, arena, m.table, cnt_e)
    assert u.err == 0
    tok = parse_send_arena(w, pm, m)
    RT, G = w.R * w.T, w.G
    sb = {orc.Q_NONE: 0, orc.Q_FP8_F32: 4, orc.Q_FP8_UE8M0: 1}[w.quant]
    entries = sorted((int(topk[s, t, k]), s, t, k) for s in range(w.R) for t in range(w.T)
                     for k in range(w.K) if topk[s, t, k] >= 0)
    seen = {}
    for e, s, t, k in entries:
        pos = seen.get(e, 0)
        seen[e] = pos + 1
        codes, scales, ids = tok[(s, t)]
        assert ids[k] == e
        r = e * RT + pos
        assert u.recv[r].tobytes() == codes
        assert u.recv_src_idx[r] == s * w.T + t
        if sb:
            got = b"".join(u.scales.view(np.uint8)[((e * G + g) * RT + pos) * sb:
                                                  ((e * G + g) * RT + pos + 1) * sb].tobytes()
                           for g in range(G))
            assert got == scales
    assert sum(seen.values()) == int(u.recv_count.sum())


def test_unpack_rejects_bad_flag_header_and_short_arena():
    w, pm, topk, x, wt, m = build_case(SHAPES[3], seed=40)
    cap = int(m.arena_base[1][-1])
    _, arena = orc.messages_execute(pm, m, cap)
    lay, recv, sc = ll_reference(w, topk, x)
    good = orc.messages_unpack(pm, arena, m.table, lay.num_tokens_per_expert, fill_codes=0x5C)
    assert good.err == 0
    # stale completion flag on (s=1, d=2), wrong token count in (s=3, d=0)'s header
    bad = arena.copy()
    t12, t30 = m.table[1, 2], m.table[3, 0]
    assert t12[3] > 0 and t30[3] > 0
    bad[t12[1] + 16 + t12[4]] ^= 1
    bad[t30[1] + 8] ^= 1
    u = orc.messages_unpack(pm, bad, m.table, lay.num_tokens_per_expert, fill_codes=0x5C)
    assert u.err == orc.ERR_MESSAGE
    RT = w.R * w.T
    for (s, d) in [(1, 2), (3, 0)]:
        rows = lay.send_pos[s][(lay.send_pos[s] >= 0) & (lay.send_pos[s] // RT // w.L == d)]
        assert rows.size > 0
        assert (u.recv[rows] == 0x5C).all() and (u.recv_src_idx[rows] == -1).all()
    other = lay.send_pos[(lay.send_pos >= 0)]
    keep = np.array([not ((s, (r // RT) // w.L) in [(1, 2), (3, 0)])
                     for s in range(w.R) for r in lay.send_pos[s].reshape(-1) if r >= 0])
    assert np.array_equal(u.recv[other[keep]], good.recv[other[keep]])
    # a receive arena shorter than the address book: capacity error
    u2 = orc.messages_unpack(pm, arena[: cap // 2], m.table, lay.num_tokens_per_expert)
    assert u2.err & orc.ERR_CAPACITY


def test_execute_rejects_bad_descriptors():
    w, pm, topk, x, wt, m = build_case(SHAPES[1], seed=50)
    cap = int(m.arena_base[1][-1])
    d = m.desc.copy()
    d[0, 36] = 0x7F  # source rank far out of range
    bad = orc.Messages(m.err, m.send_arena, m.table, m.arena_base, d, m.num_desc)
    err, _ = orc.messages_execute(pm, bad, cap)
    assert err & orc.ERR_MESSAGE
    end = max(ro + reg for _, ro, reg in regions(m))  # the arena tail is alignment padding
    err2, _ = orc.messages_execute(pm, m, end - 1)
    assert err2 & orc.ERR_CAPACITY
