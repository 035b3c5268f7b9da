"""Pins of the oracle's rank-major mode (one receive row per (token,
destination rank), the V1 receive buffer of the "DeepEP" deep dive, sec.
2.3), on the CPU.

- Layout: brute force on tiny shapes -- partition d lists the tokens with an
  expert on d, sorted by (source, token); rows are packed partition by
  partition.  Closed forms: rows of d = last row of the rank prefix matrix,
  source s starts at the exclusive prefix, counts and send_head equal the
  expert-major layout's.
- Dispatch: every row holds its source token (bf16 bit for bit, or the same
  FP8 codes and scales the expert-major dispatch stores for that token).
- Receive metadata: per-row local expert ids and weights, brute force.
- Combine: the unweighted sum of a token's distinct rows, against fp64
  numpy sums (exact for these inputs) rounded once; the identity expert
  gives x * sum of weights within two roundings.
"""
import numpy as np
import pytest

from combine_ep_get_layout_amd import inputs
from oracle import oracle as orc

SHAPES = [
    # R, T, H, E, K, quant
    (1, 5, 128, 4, 2, orc.Q_NONE),
    (2, 9, 128, 8, 3, orc.Q_FP8_F32),
    (3, 7, 256, 9, 4, orc.Q_FP8_UE8M0),
    (4, 16, 128, 16, 8, orc.Q_NONE),
    (5, 6, 128, 5, 5, orc.Q_FP8_F32),
    (8, 12, 128, 64, 6, orc.Q_NONE),
]


def case(si, seed, mfrac=0.0, dfrac=0.0):
    R, T, H, E, K, quant = SHAPES[si]
    w = inputs.small(f"rank{si}", R=R, T=T, H=H, E=E, K=K, mode=orc.MODE_RANK, quant=quant,
                     seed=seed)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=seed)
    return w, topk


def brute_rows(w, topk):
    """{(d, s, t): row} and the partition sizes, from sorting."""
    L = w.E // w.R
    parts = [sorted((s, t) for s in range(w.R) for t in range(w.T)
                    if any(0 <= e < w.E and e // L == d for e in topk[s, t])) for d in range(w.R)]
    rows, base = {}, 0
    for d, lst in enumerate(parts):
        for i, (s, t) in enumerate(lst):
            rows[(d, s, t)] = base + i
        base += len(lst)
    return rows, [len(p) for p in parts], base


@pytest.mark.parametrize("si", range(len(SHAPES)))
@pytest.mark.parametrize("mask", [(0.0, 0.0), (0.3, 0.2)])
def test_rank_major_layout_bruteforce_and_closed_forms(si, mask):
    w, topk = case(si, 3 + si, *mask)
    R, T, E, K, L = w.R, w.T, w.E, w.K, w.E // w.R
    p = orc.Problem(R, T, w.H, E, K, mode=orc.MODE_RANK)
    lay = orc.layout(p, topk)
    assert lay.err == 0
    rows, sizes, total = brute_rows(w, topk)
    assert lay.total_rows == total == orc.recv_rows(p, topk)
    assert list(lay.rows_per_rank) == sizes
    assert np.array_equal(lay.rows_per_rank, lay.rank_prefix_matrix[-1])
    for s in range(R):
        for t in range(T):
            for k in range(K):
                e = topk[s, t, k]
                want = rows[(e // L, s, t)] if 0 <= e < E else -1
                assert lay.send_pos[s, t, k] == want
    for (d, s, t), r in rows.items():
        assert lay.recv_src_idx[r] == s * T + t
        # source s's segment of partition d starts at the exclusive prefix
        excl = lay.rank_prefix_matrix[s, d] - lay.num_tokens_per_rank[s, d]
        assert r - lay.row_base[d] - excl == lay.send_head[s, t, d]
    # counts and stream indices are those of the expert-major layout
    ln = orc.layout(orc.Problem(R, T, w.H, E, K), topk)
    for f in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
              "rank_prefix_matrix", "recv_tokens_per_expert", "send_head"):
        assert np.array_equal(getattr(lay, f), getattr(ln, f)), f


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_rank_major_dispatch_rows_and_metadata(si):
    w, topk = case(si, 20 + si, 0.2, 0.3)
    R, T, H, E, K, L = w.R, w.T, w.H, w.E, w.K, w.E // w.R
    x, wt = inputs.gen_x(w), inputs.gen_weights(w)
    p = orc.Problem(R, T, H, E, K, mode=orc.MODE_RANK, quant=w.quant)
    lay = orc.layout(p, topk)
    cap = lay.total_rows
    err, recv, sc = orc.dispatch(p, x, topk, lay.send_pos, cap)
    assert err == 0
    # the expert-major dispatch of the same token stores the same bytes
    pn = orc.Problem(R, T, H, E, K, mode=orc.MODE_NORMAL, quant=w.quant)
    ln = orc.layout(pn, topk)
    _, recv_n, sc_n = orc.dispatch(pn, x, topk, ln.send_pos, ln.total_rows)
    G = w.G
    for r in range(cap):
        s, t = divmod(int(lay.recv_src_idx[r]), T)
        if w.quant == orc.Q_NONE:
            assert np.array_equal(recv[r], x[s, t])
        k = next(k for k in range(K) if lay.send_pos[s, t, k] == r)
        rn = ln.send_pos[s, t, k]
        assert np.array_equal(recv[r], recv_n[rn])
        if w.quant != orc.Q_NONE:
            assert np.array_equal(sc[np.arange(G) * cap + r], sc_n[np.arange(G) * ln.total_rows + rn])
    e2, idx, wts = orc.rank_topk(p, topk, wt, lay.send_pos, cap)
    assert e2 == 0
    rows, _, _ = brute_rows(w, topk)
    for (d, s, t), r in rows.items():
        for k in range(K):
            e = topk[s, t, k]
            on = 0 <= e < E and e // L == d
            assert idx[r, k] == (e - d * L if on else -1)
            assert wts[r, k] == (wt[s, t, k] if on else 0.0)


@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_rank_major_combine_sum_and_identity(si):
    w, topk = case(si, 40 + si, 0.25, 0.2)
    R, T, H, E, K, L = w.R, w.T, w.H, w.E, w.K, w.E // w.R
    p = orc.Problem(R, T, H, E, K, mode=orc.MODE_RANK)
    lay = orc.layout(p, topk)
    cap = lay.total_rows
    y = inputs.gen_y(w, max(cap, 1))
    wt = inputs.gen_weights(w)
    err, out = orc.combine(p, y, wt, lay.send_pos)
    assert err == 0
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for s in range(R):
        for t in range(T):
            rows = sorted({int(r) for r in lay.send_pos[s, t] if r >= 0})
            acc = yf[rows].sum(axis=0) if rows else np.zeros(H)
            want = np.array([orc.bf16_from_double(v) for v in acc], np.uint16)
            assert np.array_equal(out[s, t], want)
    # identity expert: rank d returns bf16(sum of its experts' weights * x)
    x = inputs.gen_x(w)
    _, idx, wts = orc.rank_topk(p, topk, wt, lay.send_pos, cap)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y_id = np.zeros((max(cap, 1), H), np.uint16)
    for r in range(cap):
        s, t = divmod(int(lay.recv_src_idx[r]), T)
        y_id[r] = [orc.bf16_from_double(v) for v in xf[s, t] * wts[r].astype(np.float64).sum()]
    _, out_id = orc.combine(p, y_id, wt, lay.send_pos)
    of = (out_id.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for s in range(R):
        for t in range(T):
            ws = sum(float(wt[s, t, k]) for k in range(K) if topk[s, t, k] >= 0)
            ref = xf[s, t] * ws
            assert np.all(np.abs(of[s, t] - ref) <= 2 * 2.0 ** -8 * np.abs(ref) + 1e-30)
