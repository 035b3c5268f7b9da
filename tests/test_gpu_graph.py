"""The whole step (layout, dispatch, combine) captured once into a HIP graph
and replayed.  Before every replay, fresh routing, tokens and weights are
copied into the captured input buffers and every output is poisoned (eager
work between replays); each replay must then reproduce, bit for bit, an
eager run of the same three calls on the same inputs into separate buffers.
The eager path itself is held to the oracle by the parity tests.

Receive capacities are the worst case (`ep_max_recv_rows`, the
`num_worst_tokens` idea of the "DeepEP" deep dive, sec. 2.1), so nothing in
the step reads a count back to the host."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from gpu_util import DEV, h, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, R, T, H, E, K, mode, quant, fused layout + dispatch
    ("normal_bf16", 4, 40, 256, 16, 4, ep.MODE_NORMAL, ep.QUANT_NONE, False),
    ("normal_ue8m0", 4, 40, 256, 16, 4, ep.MODE_NORMAL, ep.QUANT_FP8_UE8M0, False),
    ("ll_fp8", 4, 24, 256, 8, 3, ep.MODE_LOW_LATENCY, ep.QUANT_FP8_F32, False),
    ("ll_bf16", 2, 33, 128, 8, 2, ep.MODE_LOW_LATENCY, ep.QUANT_NONE, False),
    ("messages_fp8", 4, 20, 256, 16, 4, ep.MODE_MESSAGES, ep.QUANT_FP8_F32, False),
    ("rank_major_fp8", 4, 300, 256, 16, 4, ep.MODE_RANK_MAJOR, ep.QUANT_FP8_F32, False),
    ("fused_normal_fp8", 4, 600, 256, 16, 4, ep.MODE_NORMAL, ep.QUANT_FP8_F32, True),
    ("fused_ll_bf16", 4, 300, 128, 16, 8, ep.MODE_LOW_LATENCY, ep.QUANT_NONE, True),
]


class Bufs:
    """One set of step buffers (inputs, handle, outputs)."""

    def __init__(self, w, p, fused=False):
        self.fused = fused
        self.topk = torch.zeros((w.R, w.T, w.K), dtype=torch.int32, device=DEV)
        self.x = torch.zeros((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)
        self.wt = torch.zeros((w.R, w.T, w.K), dtype=torch.float32, device=DEV)
        self.lay = ep.Layout(p)
        self.ws = ep.workspace(p)
        self.recv = self.msgs = self.out = None
        if w.mode == ep.MODE_MESSAGES:
            send_cap, desc_cap = ep.messages_capacity(p)  # worst case: no read-back
            self.msgs = ep.Messages(p, send_cap, desc_cap)
            # delivery and the receiver, into the low-latency layout
            self.arena = torch.empty(send_cap, dtype=torch.uint8, device=DEV)
            self.unp = ep.unpack_buffers(p)
            self.merr = torch.zeros(1, dtype=torch.int32, device=DEV)
        else:
            self.recv = ep.Recv(p, ep.max_recv_rows(p))
            self.out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)

    def load(self, topk, x, wt):
        self.topk.copy_(torch.from_numpy(topk))
        self.x.copy_(torch.from_numpy(x).view(torch.bfloat16))
        self.wt.copy_(torch.from_numpy(wt))

    def poison(self):
        lay = self.lay
        for t in (lay.num_tokens_per_rank, lay.num_tokens_per_expert, lay.rank_prefix_matrix,
                  lay.recv_tokens_per_expert, lay.expert_start, lay.rows_per_rank, lay.row_base,
                  lay.send_pos, lay.send_head, lay.recv_src_idx):
            if t is not None:
                t.fill_(-77)
        lay.is_token_in_rank.fill_(0xEE)
        lay.err.fill_(0x5A5A)
        if self.recv is not None:
            self.recv.x.view(torch.uint8).fill_(0xA5)
            if self.recv.scales is not None:
                self.recv.scales.view(torch.uint8).fill_(0xA5)
            self.out.view(torch.int16).fill_(0x7F7F)
        if self.recv is not None and self.recv.topk_idx is not None:
            self.recv.topk_idx.fill_(-9)
            self.recv.topk_weights.fill_(-9.0)
        if self.msgs is not None:
            for t in (self.msgs.send_arena, self.msgs.descriptors, self.arena):
                t.fill_(0xA5)
            for t in (self.msgs.table, self.msgs.arena_base, self.msgs.num_descriptors):
                t.fill_(-5)
            self.unp[0].x.view(torch.uint8).fill_(0xA5)
            self.unp[0].scales.view(torch.uint8).fill_(0xA5)
            self.unp[1].fill_(-3)
            self.unp[2].fill_(-1)
            self.merr.zero_()


def step(p, b: Bufs, y):
    if b.fused:
        ep.dispatch_fused(p, b.topk, b.lay, b.x, b.recv, b.ws)
        ep.combine(p, b.lay, b.recv.x if y is None else y, b.wt, b.out)
        return
    ep.get_layout(p, b.topk, b.lay, b.ws)
    if b.msgs is not None:
        ep.dispatch(p, b.lay, b.x, msgs=b.msgs, topk_idx=b.topk, topk_weights=b.wt, ws=b.ws)
        ep.messages_execute(p, b.msgs, b.arena, b.merr)
        ep.messages_unpack(p, b.msgs, b.arena, b.lay.num_tokens_per_expert, *b.unp, b.merr)
        return
    if p.mode == ep.MODE_RANK_MAJOR:
        ep.dispatch(p, b.lay, b.x, recv=b.recv, topk_idx=b.topk, topk_weights=b.wt, ws=b.ws)
        ep.combine(p, b.lay, b.recv.x if y is None else y, None, b.out)
        return
    ep.dispatch(p, b.lay, b.x, recv=b.recv, ws=b.ws)
    ep.combine(p, b.lay, b.recv.x if y is None else y, b.wt, b.out)


def compare(w, g: Bufs, e: Bufs):
    for f in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
              "rank_prefix_matrix", "recv_tokens_per_expert", "expert_start", "rows_per_rank",
              "row_base", "send_pos", "send_head", "err"):
        a, b = getattr(g.lay, f), getattr(e.lay, f)
        if a is not None:
            assert torch.equal(a, b), f
    if g.msgs is not None:
        table = h(g.msgs.table)
        assert np.array_equal(table, h(e.msgs.table))
        assert torch.equal(g.msgs.arena_base, e.msgs.arena_base)
        nd = int(h(g.msgs.num_descriptors)[0])
        assert nd == int(h(e.msgs.num_descriptors)[0])
        assert torch.equal(g.msgs.descriptors[:nd], e.msgs.descriptors[:nd])
        ga, ea = h(g.msgs.send_arena), h(e.msgs.send_arena)
        gr, er = h(g.arena), h(e.arena)
        for off, roff, reg in table.reshape(-1, 8)[:, [0, 1, 2]]:
            if reg > 0:
                assert np.array_equal(ga[off:off + reg], ea[off:off + reg])
                assert np.array_equal(gr[roff:roff + reg], er[roff:roff + reg])
        for a, b in zip((g.unp[0].x, g.unp[0].scales, g.unp[1], g.unp[2], g.merr),
                        (e.unp[0].x, e.unp[0].scales, e.unp[1], e.unp[2], e.merr)):
            assert torch.equal(a, b)
        return
    sp = h(g.lay.send_pos).reshape(-1)
    rows = torch.from_numpy(np.unique(sp[sp >= 0]).astype(np.int64)).to(DEV)
    assert torch.equal(g.lay.recv_src_idx[rows], e.lay.recv_src_idx[rows])
    assert torch.equal(g.recv.x[rows], e.recv.x[rows])
    if g.recv.topk_idx is not None:
        assert torch.equal(g.recv.topk_idx[rows], e.recv.topk_idx[rows])
        assert torch.equal(g.recv.topk_weights[rows], e.recv.topk_weights[rows])
    if w.quant != ep.QUANT_NONE:
        G, RT, cap = w.G, w.R * w.T, g.recv.capacity
        gi = torch.arange(G, device=DEV)
        if w.mode == ep.MODE_LOW_LATENCY:
            si = ((rows // RT)[:, None] * G + gi[None, :]) * RT + (rows % RT)[:, None]
        else:
            si = gi[None, :] * cap + rows[:, None]
        si = si.reshape(-1)
        assert torch.equal(g.recv.scales[si], e.recv.scales[si])
    assert torch.equal(g.out, e.out)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_matches_eager(case):
    name, R, T, H, E, K, mode, quant, fused = case
    say("graph", name)
    w = inputs.small(f"graph_{name}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=31)
    p = ep.Problem(R, T, H, E, K, mode=mode, quant=quant, region_bytes=512, epoch=9)
    cap_bufs, eager_bufs = Bufs(w, p, fused), Bufs(w, p, fused)
    y = None
    if mode != ep.MODE_MESSAGES and quant != ep.QUANT_NONE:
        # bf16 expert outputs in the receive layout, fixed for every replay
        y = torch.from_numpy(inputs.gen_y(w, cap_bufs.recv.capacity)).view(torch.bfloat16).to(DEV)
    cap_bufs.load(inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(p, cap_bufs, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(p, cap_bufs, y)
    torch.cuda.synchronize()
    for rep in range(4):
        wr = inputs.small(f"graph_{name}_{rep}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant,
                          seed=100 + rep)
        topk = inputs.gen_topk(wr)
        if rep % 2 == 1:
            topk = inputs.masked_topk(wr, topk, 0.2, 0.0, seed=rep)
        x, wt = inputs.gen_x(wr), inputs.gen_weights(wr)
        cap_bufs.load(topk, x, wt)
        cap_bufs.poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager_bufs.load(topk, x, wt)
        eager_bufs.poison()
        step(p, eager_bufs, y)
        torch.cuda.synchronize()
        say("graph", name, "replay", rep)
        compare(w, cap_bufs, eager_bufs)
        assert int(h(cap_bufs.lay.err)[0]) == 0
        if cap_bufs.msgs is not None:
            assert int(h(cap_bufs.merr)[0]) == 0
