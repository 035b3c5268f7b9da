"""Reentrancy through the C ABI: the library keeps no state between calls,
so two unrelated problems whose calls are interleaved on two streams (both
at the default priority) give the same results as the oracle gives for each
alone: a normal-mode bf16 step and a low-latency FP8 step."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import DEV, abs_weighted_sum, bf16_to_f32, combine_close, h, problems, say

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, name, **kw):
        self.w = inputs.small(name, seed=77, **kw)
        w = self.w
        self.topk, self.x, self.wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
        self.p, self.po = problems(w)
        self.cap = ep.max_recv_rows(self.p)
        self.lay = ep.Layout(self.p, recv_capacity=self.cap)
        self.ws = ep.workspace(self.p)
        self.recv = ep.Recv(self.p, self.cap)
        self.tk = torch.from_numpy(self.topk).to(DEV)
        self.xg = torch.from_numpy(self.x).view(torch.bfloat16).to(DEV)
        self.wg = torch.from_numpy(self.wt).to(DEV)
        self.y = torch.from_numpy(inputs.gen_y(w, self.cap)).view(torch.bfloat16).to(DEV)
        self.out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=DEV)

    def calls(self, stream):
        return [lambda: ep.get_layout(self.p, self.tk, self.lay, self.ws, stream=stream),
                lambda: ep.dispatch(self.p, self.lay, self.xg, recv=self.recv, ws=self.ws,
                                    stream=stream),
                lambda: ep.combine(self.p, self.lay, self.y, self.wg, self.out, stream=stream)]

    def check(self):
        w, po = self.w, self.po
        ol = orc.layout(po, self.topk)
        assert int(h(self.lay.err)[0]) == ol.err == 0
        assert np.array_equal(h(self.lay.send_pos), ol.send_pos)
        _, orecv, osc = orc.dispatch(po, self.x, self.topk, ol.send_pos, self.cap)
        rows = np.unique(ol.send_pos[ol.send_pos >= 0])
        g = h(self.recv.x.view(torch.uint16) if w.quant == 0 else self.recv.x)
        assert np.array_equal(g[rows], orecv[rows])
        if w.quant:  # low-latency scales: [E][G][R*T]
            rt = w.R * w.T
            gs, os_ = h(self.recv.scales).reshape(-1), np.asarray(osc).reshape(-1)
            for r in rows:
                idx = (r // rt * w.G + np.arange(w.G)) * rt + r % rt
                assert np.array_equal(gs[idx], os_[idx]), r
        y = h(self.y.view(torch.uint16))
        _, oo = orc.combine(po, y, self.wt, ol.send_pos)
        absw = abs_weighted_sum(bf16_to_f32(y), self.wt, ol.send_pos)
        combine_close(h(self.out.view(torch.uint16)).reshape(-1, w.H), oo.reshape(-1, w.H), absw)


def test_two_problems_interleaved_on_two_streams():
    say("two streams")
    a = Case("streams_normal", R=4, T=700, H=256, E=32, K=4, mode=ep.MODE_NORMAL, quant=0)
    b = Case("streams_ll", R=4, T=300, H=512, E=16, K=4, mode=ep.MODE_LOW_LATENCY,
             quant=ep.QUANT_FP8_F32)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for ca, cb in zip(a.calls(sa), b.calls(sb)):  # enqueue alternately
        ca()
        cb()
    torch.cuda.synchronize()
    a.check()
    b.check()
