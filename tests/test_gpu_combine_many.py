"""GPU parity of the combine at 8192 tokens or more through the C ABI,
against the oracle on every token.  The token count and the hidden size
select the kernel form:
 - hidden up to 2048 and 7168-8192: one token per block, one row load in
   flight per wavefront;
 - hidden 2056-4096 (outputs staged in LDS) and 4104-7160: two tokens per
   block with the next token's row loads in flight;
 - rank-major rows wider than 4096: one token per block, eight row loads in
   flight.
Token counts leave a ragged last block.  Covers masked entries, k = 1..8,
rank-major repeats (a token's entries on one rank share a row, summed
once), a receive buffer with no rows (every entry masked), and a receive
buffer shorter than the rows the layout assigns (those entries are dropped
and the capacity error bit is raised)."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import (DEV, abs_weighted_sum, bf16_to_f32, combine_close, gpu_layout, h,
                      problems, say)

pytestmark = pytest.mark.gpu

N_, RM = ep.MODE_NORMAL, ep.MODE_RANK_MAJOR
CASES = [
    # name, R, T, H, E, K, mode, masked, duplicates
    ("k8_masked", 2, 4099, 256, 16, 8, N_, 0.2, 0.0),
    ("k3_ragged", 3, 2731, 128, 9, 3, N_, 0.1, 0.0),
    ("k1", 1, 8195, 128, 4, 1, N_, 0.0, 0.0),
    ("k5_wide", 2, 4097, 1024, 8, 5, N_, 0.05, 0.2),
    ("rm_k8_dups", 4, 2049, 256, 16, 8, RM, 0.1, 0.3),
    ("rm_k5", 3, 2731, 128, 12, 5, RM, 0.2, 0.0),
    ("all_masked", 2, 4097, 128, 8, 4, N_, 1.0, 0.0),
    ("h3072_pipe_staged", 2, 4100, 3072, 8, 4, N_, 0.05, 0.1),
    ("h5120_pipe", 2, 4100, 5120, 8, 4, N_, 0.05, 0.0),
    ("h8192_serial", 1, 8193, 8192, 4, 3, N_, 0.1, 0.0),
    ("rm_h5120_eight", 2, 4100, 5120, 8, 4, RM, 0.05, 0.2),
]


def distinct_abs_sum(yf: np.ndarray, send_pos: np.ndarray, K: int) -> np.ndarray:
    """sum over a token's distinct rows of |y[row]| (rank-major tolerance)."""
    sp = send_pos.reshape(-1, K)
    out = np.zeros((sp.shape[0], yf.shape[1]))
    for i in range(sp.shape[0]):
        for r in sorted({int(r) for r in sp[i] if r >= 0}):
            out[i] += np.abs(yf[r].astype(np.float64))
    return out


def run(c, short_rows=0):
    name, R, T, H, E, K, mode, mfrac, dfrac = c
    w = inputs.small(f"many_{name}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=0, seed=61)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=8)
    wt = inputs.gen_weights(w)
    p, po = problems(w)
    ol = orc.layout(po, topk)
    total = ol.total_rows
    gl, _ = gpu_layout(p, topk)
    rows = max(total - short_rows, 0)
    y = inputs.gen_y(w, max(rows, 1))[:rows]
    out = torch.empty((R, T, H), dtype=torch.bfloat16, device=DEV)
    yg = torch.from_numpy(np.ascontiguousarray(y)).view(torch.bfloat16).to(DEV)
    ep.combine(p, gl, yg, None if mode == RM else torch.from_numpy(wt).to(DEV), out)
    torch.cuda.synchronize()
    # the oracle sees the rows the buffer holds; entries past it are dropped
    sp = np.where(ol.send_pos < rows, ol.send_pos, -1).astype(np.int32)
    _, oo = orc.combine(po, y if rows else np.zeros((1, H), np.uint16), wt, sp)
    yf = bf16_to_f32(y) if rows else np.zeros((1, H), np.float32)
    absw = distinct_abs_sum(yf, sp, K) if mode == RM else abs_weighted_sum(yf, wt, sp)
    go = h(out.view(torch.uint16)).reshape(-1, H)
    rel = combine_close(go, oo.reshape(-1, H), absw)
    return int(h(gl.err)[0]), total, rel


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_many_token_combine(c):
    say("many-token combine", c)
    err, total, rel = run(c)
    say("  rows", total, "max rel err", rel)
    assert err == 0
    if c[0] == "all_masked":
        assert total == 0


SHORT = {c[0]: c for c in CASES}


@pytest.mark.parametrize("c", [SHORT["k8_masked"], SHORT["rm_k8_dups"],
                               SHORT["h3072_pipe_staged"]],
                         ids=["normal", "rank_major", "pipelined"])
def test_many_token_combine_short_buffer(c):
    """The last 37 rows are missing from y: their entries are skipped and
    the capacity error bit is set."""
    say("many-token combine, short buffer", c)
    err, total, _ = run(c, short_rows=37)
    assert total > 37
    assert err & ep.DEVERR_CAPACITY
