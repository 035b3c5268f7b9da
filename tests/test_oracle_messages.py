"""Pins for the oracle's message packer and write descriptors.

The byte format is this library's own specification (the pages name a
header, a payload and a completion flag, and 16-byte WQE segments, but give
no field values), so these checks are (1) a brute-force re-derivation of
every byte on tiny shapes, written independently with ``struct`` and
PyTorch's FP8 cast, and (2) structural invariants at larger sizes: headers
match the counts, flags come last, descriptors tile each put exactly in
order, no descriptor crosses a region boundary on either side, and work
queue indices are contiguous per queue pair.
"""
import struct

import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import inputs
from oracle import oracle as orc


def torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def pad16(n):
    return (n + 15) // 16 * 16


def brute_messages(p, x, topk, wts):
    """Expected (per-message region bytes, descriptor tuples)."""
    R, T, H, K, L, G = p.R, p.T, p.H, p.K, p.E // p.R, p.H // 128
    RB = p.region_bytes
    toks = {(s, d): [t for t in range(T)
                     if any(e >= 0 and e // L == d for e in topk[s, t].tolist())]
            for s in range(R) for d in range(R)}
    regions = {}
    for (s, d), tl in toks.items():
        n = len(tl)
        if n == 0:
            continue
        codes, scales = b"", b""
        xf = bf16_to_f32(x)
        for t in tl:
            if p.quant == orc.Q_NONE:
                codes += x[s, t].astype("<u2").tobytes()
                continue
            row = xf[s, t].reshape(G, 128)
            amax = np.maximum(np.abs(row).max(axis=1), np.float32(1e-4)).astype(np.float32)
            sc = (amax / np.float32(448)).astype(np.float32)
            if p.quant == orc.Q_FP8_F32:
                codes += torch_e4m3(row / sc[:, None]).tobytes()
                scales += sc.astype("<f4").tobytes()
            else:
                ex = [int((np.frexp(v)[1] - (1 if np.frexp(v)[0] == 0.5 else 0)) + 127)
                      for v in sc]
                codes += torch_e4m3(np.stack([np.ldexp(row[g], 127 - ex[g])
                                              for g in range(G)]).astype(np.float32)).tobytes()
                scales += bytes(ex)
        secs = [codes, scales,
                b"".join(wts[s, t].astype("<f4").tobytes() for t in tl),
                b"".join(topk[s, t].astype("<i4").tobytes() for t in tl),
                b"".join(struct.pack("<i", t) for t in tl)]
        body = b"".join(sec + bytes(pad16(len(sec)) - len(sec)) for sec in secs)
        regions[(s, d)] = (struct.pack("<4I", s, d, n, len(body)) + body
                           + struct.pack("<4I", p.epoch, 0, 0, 0))
    # arenas
    send_base, recv_base = [0], [0]
    for s in range(R):
        tot = sum(len(regions.get((s, d), b"")) for d in range(R))
        send_base.append(send_base[-1] + (tot + RB - 1) // RB * RB)
    for d in range(R):
        tot = sum(len(regions.get((s, d), b"")) for s in range(R))
        recv_base.append(recv_base[-1] + (tot + RB - 1) // RB * RB)
    descs, offs = [], {}
    for s in range(R):
        so = 0
        for d in range(R):
            if (s, d) not in regions:
                continue
            ro = sum(len(regions.get((s2, d), b"")) for s2 in range(s))
            offs[(s, d)] = (send_base[s] + so, recv_base[d] + ro)
            m = regions[(s, d)]
            body = len(m) - 32
            wqe = 0
            for off, ln in [(16, body), (0, 16), (16 + body, 16)]:
                la, ra, rem = so + off, ro + off, ln
                while rem:
                    c = min(rem, RB - la % RB, RB - ra % RB)
                    rkey, lkey = (d << 16) | (ra // RB), (s << 16) | (la // RB)
                    if la // RB > 0xFFFF or ra // RB > 0xFFFF:  # index past 16 bits
                        rkey = lkey = 0xFFFFFFFF
                    descs.append((wqe, s * R + d, ra, rkey, c, lkey, la))
                    wqe += 1
                    la += c
                    ra += c
                    rem -= c
            so += len(m)
    return regions, offs, send_base, recv_base, descs


def parse_desc(b):
    w0, w1 = struct.unpack(">II", b[0:8])
    assert b[8:11] == b"\0\0\0" and b[11] == 8 and b[12:16] == b"\0" * 4
    assert w0 & 0xFF == 0x08 and w1 & 0xFF == 3
    assert b[28:32] == b"\0" * 4 and b[48:64] == b"\0" * 16
    raddr, = struct.unpack(">Q", b[16:24])
    rkey, ln, lkey = struct.unpack(">III", b[24:28] + b[32:40])
    laddr, = struct.unpack(">Q", b[40:48])
    return (w0 >> 8, w1 >> 8, raddr, rkey, ln, lkey, laddr)


SMALL = [
    # R, T, H, E, K, quant, region bytes
    (2, 5, 128, 4, 2, orc.Q_FP8_F32, 256),
    (3, 7, 256, 6, 3, orc.Q_FP8_UE8M0, 512),
    (4, 6, 128, 8, 3, orc.Q_NONE, 128),
    (4, 9, 256, 8, 4, orc.Q_FP8_F32, 1 << 20),
]


@pytest.mark.parametrize("case", SMALL)
@pytest.mark.parametrize("seed", range(3))
def test_messages_brute_force(case, seed):
    R, T, H, E, K, quant, RB = case
    w = inputs.small(R=R, T=T, H=H, E=E, K=K, mode=orc.MODE_MSG, quant=quant, seed=50 + seed)
    topk = inputs.masked_topk(w, inputs.gen_topk(w), 0.15, 0.1)
    x = inputs.gen_x(w)
    wts = inputs.gen_weights(w)
    p = orc.Problem(R, T, H, E, K, mode=orc.MODE_MSG, quant=quant, region_bytes=RB, epoch=77)
    regions, offs, sb, rb, descs = brute_messages(p, x, topk, wts)
    m = orc.messages(p, x, topk, wts, send_cap=sb[-1], desc_cap=len(descs) + 8)
    assert m.err == 0
    assert m.arena_base[0].tolist() == sb and m.arena_base[1].tolist() == rb
    for s in range(R):
        for d in range(R):
            row = m.table[s, d]
            if (s, d) not in regions:
                assert row[0] == -1 and row[2] == 0
                continue
            so, ro = offs[(s, d)]
            reg = regions[(s, d)]
            assert (row[0], row[1], row[2]) == (so, ro, len(reg))
            assert m.send_arena[so:so + len(reg)].tobytes() == reg, (s, d)
    assert m.num_desc == len(descs)
    assert [parse_desc(bytes(d)) for d in m.desc] == descs


@pytest.mark.parametrize("RB,poisoned", [(16, True), (32, False)])
def test_region_index_past_16_bits(RB, poisoned):
    """Keys hold a region index in 16 bits.  One rank sending 600 bf16 rows of
    hidden 1024 to itself fills a 1,240,832-byte arena: 77,552 regions of 16
    bytes (pieces past region 65535 cannot be named: their keys are all ones,
    a rank no problem has, and the capacity bit is raised) or 38,776 regions
    of 32 bytes (every key fits).  The brute force applies the same rule."""
    R, T, H, E, K = 1, 600, 1024, 2, 2
    w = inputs.small(R=R, T=T, H=H, E=E, K=K, mode=orc.MODE_MSG, quant=orc.Q_NONE, seed=3)
    topk, x, wts = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p = orc.Problem(R, T, H, E, K, mode=orc.MODE_MSG, quant=orc.Q_NONE, region_bytes=RB, epoch=9)
    regions, offs, sb, rb, descs = brute_messages(p, x, topk, wts)
    assert len(regions[(0, 0)]) == 1240832
    m = orc.messages(p, x, topk, wts, send_cap=sb[-1], desc_cap=len(descs))
    assert m.err == (orc.ERR_CAPACITY if poisoned else 0)
    got = [parse_desc(bytes(d)) for d in m.desc]
    assert got == descs
    bad = [q for q in got if q[3] == 0xFFFFFFFF]
    assert all(q[5] == 0xFFFFFFFF and q[6] // RB > 0xFFFF for q in bad)
    assert len(bad) == (1240832 // 16 - 65536 if poisoned else 0)  # regions 65536 .. 77551
    assert m.send_arena[:len(regions[(0, 0)])].tobytes() == regions[(0, 0)]


@pytest.mark.parametrize("RB", [2 << 20, 64 << 10])
def test_messages_invariants_medium(RB):
    w = inputs.small(R=16, T=64, H=1024, E=64, K=8, mode=orc.MODE_MSG,
                     quant=orc.Q_FP8_F32, seed=61)
    topk, x, wts = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=orc.MODE_MSG, quant=w.quant,
                    region_bytes=RB, epoch=5)
    lay = orc.layout(p, topk)
    body_max, _ = orc.msg_body_bytes(p, w.T)
    send_cap = w.R * (w.R * (body_max + 32) + RB)
    m = orc.messages(p, x, topk, wts, send_cap, desc_cap=1 << 16)
    assert m.err == 0
    R = w.R
    nxt = 0
    for s in range(R):
        for d in range(R):
            so, ro, reg, n, body, d0, dc, _ = m.table[s, d].tolist()
            assert n == lay.num_tokens_per_rank[s, d]
            if n == 0:
                assert dc == 0
                continue
            assert so % 16 == 0 and ro % 16 == 0 and body % 16 == 0
            hdr = struct.unpack("<4I", m.send_arena[so:so + 16].tobytes())
            assert hdr == (s, d, n, body)
            assert struct.unpack("<4I", m.send_arena[so + 16 + body:so + 32 + body].tobytes()) == (5, 0, 0, 0)
            src = np.frombuffer(m.send_arena[so + 16:so + 16 + body].tobytes(), np.uint8)
            _, sec = orc.msg_body_bytes(p, n)
            toks = src[sec[4]:sec[4] + 4 * n].view("<i4")
            assert np.array_equal(toks, np.nonzero(lay.is_token_in_rank[s, :, d])[0])
            # descriptors of this message tile payload, header, flag in order
            assert d0 == nxt
            ds = [parse_desc(bytes(b)) for b in m.desc[d0:d0 + dc]]
            nxt += dc
            assert [q[0] for q in ds] == list(range(dc))
            assert all(q[1] == s * R + d for q in ds)
            la0 = so - m.arena_base[0][s]
            ra0 = ro - m.arena_base[1][d]
            cur = [(la0 + 16, ra0 + 16, body), (la0, ra0, 16), (la0 + 16 + body, ra0 + 16 + body, 16)]
            i = 0
            for la, ra, ln in cur:
                while ln:
                    wq, qpn, raddr, rkey, c, lkey, laddr = ds[i]
                    assert (laddr, raddr) == (la, ra)
                    assert laddr // RB == (laddr + c - 1) // RB and raddr // RB == (raddr + c - 1) // RB
                    assert rkey == (d << 16) | (raddr // RB) and lkey == (s << 16) | (laddr // RB)
                    la, ra, ln, i = la + c, ra + c, ln - c, i + 1
            assert i == dc
    assert nxt == m.num_desc
