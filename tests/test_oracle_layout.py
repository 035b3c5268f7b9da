"""Pins for the oracle's layout (counts, rank prefix matrix, slots).

A second derivation by sorting (not by running counters) on tiny shapes,
plus invariants that hold at any size: count sums, the prefix matrix's
closed form, the slot map being a bijection onto the filled rows, and the
(source rank, token, k) order inside every expert segment.
"""
import itertools

import numpy as np
import pytest

from combine_ep_get_layout_amd import inputs
from oracle import oracle as orc


def brute_layout(p: orc.Problem, topk: np.ndarray):
    R, T, E, K, L = p.R, p.T, p.E, p.K, p.E // p.R
    cnt_e = np.zeros((R, E), np.int64)
    cnt_r = np.zeros((R, R), np.int64)
    in_rank = np.zeros((R, T, R), np.uint8)
    for s, t in itertools.product(range(R), range(T)):
        ranks = set()
        for k in range(K):
            e = int(topk[s, t, k])
            if e >= 0:
                cnt_e[s, e] += 1
                ranks.add(e // L)
        for r in ranks:
            cnt_r[s, r] += 1
            in_rank[s, t, r] = 1
    rpm = np.cumsum(cnt_r, axis=0)
    n = cnt_e.sum(axis=0)
    entries = sorted((int(topk[s, t, k]), s, t, k)
                     for s, t, k in itertools.product(range(R), range(T), range(K))
                     if topk[s, t, k] >= 0)
    if p.mode == orc.MODE_LL:
        start = np.arange(E) * R * T
    else:
        al = -(-n // p.align) * p.align
        start = np.concatenate([[0], np.cumsum(al)])[:E]
    send_pos = -np.ones((R, T, K), np.int64)
    for e, grp in itertools.groupby(entries, key=lambda x: x[0]):
        for pos, (_, s, t, k) in enumerate(grp):
            if p.mode == orc.MODE_LL and pos >= R * T:
                continue
            send_pos[s, t, k] = start[e] + pos
    send_head = -np.ones((R, T, R), np.int64)
    for s, d in itertools.product(range(R), range(R)):
        toks = [t for t in range(T) if in_rank[s, t, d]]
        for i, t in enumerate(toks):
            send_head[s, t, d] = i
    return cnt_e, cnt_r, in_rank, rpm, n, start, send_pos, send_head


CASES = [
    # R, T, E, K, align, mode, masked fraction, duplicate fraction
    (1, 5, 4, 2, 1, orc.MODE_NORMAL, 0.0, 0.0),
    (2, 8, 8, 2, 1, orc.MODE_NORMAL, 0.0, 0.0),
    (3, 7, 6, 3, 4, orc.MODE_NORMAL, 0.2, 0.2),
    (4, 16, 16, 4, 1, orc.MODE_NORMAL, 0.1, 0.0),
    (4, 16, 16, 4, 3, orc.MODE_NORMAL, 0.3, 0.3),
    (2, 9, 4, 4, 1, orc.MODE_LL, 0.1, 0.4),
    (4, 12, 8, 3, 1, orc.MODE_LL, 0.0, 0.0),
    (3, 5, 3, 1, 2, orc.MODE_NORMAL, 0.5, 0.0),
    (2, 4, 4, 4, 1, orc.MODE_LL, 0.0, 0.9),   # duplicates overflow R*T rows
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("seed", range(12))
def test_layout_brute_force(case, seed):
    R, T, E, K, align, mode, mfrac, dfrac = case
    w = inputs.small(R=R, T=T, H=128, E=E, K=K, mode=mode, seed=1000 + seed)
    topk = inputs.masked_topk(w, inputs.gen_topk(w), mfrac, dfrac, seed=seed)
    p = orc.Problem(R, T, 128, E, K, align=align, mode=mode)
    lay = orc.layout(p, topk)
    cnt_e, cnt_r, in_rank, rpm, n, start, send_pos, send_head = brute_layout(p, topk)
    assert np.array_equal(lay.num_tokens_per_expert, cnt_e)
    assert np.array_equal(lay.num_tokens_per_rank, cnt_r)
    assert np.array_equal(lay.is_token_in_rank, in_rank)
    assert np.array_equal(lay.rank_prefix_matrix, rpm)
    assert np.array_equal(lay.recv_tokens_per_expert, n)
    assert np.array_equal(lay.expert_start, start)
    assert np.array_equal(lay.send_pos, send_pos)
    assert np.array_equal(lay.send_head, send_head)
    overflow = mode == orc.MODE_LL and (n > R * T).any()
    assert bool(lay.err & orc.ERR_LL_OVERFLOW) == bool(overflow)
    assert not lay.err & orc.ERR_TOPK_RANGE
    # recv_src_idx is the inverse map of send_pos
    src = -np.ones(lay.recv_src_idx.size, np.int64)
    for s, t, k in itertools.product(range(R), range(T), range(K)):
        if send_pos[s, t, k] >= 0:
            src[send_pos[s, t, k]] = s * T + t
    assert np.array_equal(lay.recv_src_idx, src)


def test_layout_out_of_range_sets_error():
    p = orc.Problem(2, 2, 128, 4, 2)
    topk = np.array([[[0, 4], [1, -2]], [[3, 2], [-1, 0]]], np.int32)
    lay = orc.layout(p, topk)
    assert lay.err & orc.ERR_TOPK_RANGE
    assert lay.send_pos.tolist() == [[[0, -1], [2, -1]], [[4, 3], [-1, 1]]]


@pytest.mark.parametrize("name", ["tiny", "ll_decode", "messages"])
def test_layout_invariants_on_workloads(name):
    w = inputs.WORKLOADS[name]
    topk = inputs.gen_topk(w)
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode)
    lay = orc.layout(p, topk)
    assert lay.err == 0
    R, T, K, L = w.R, w.T, w.K, w.L
    # sum of expert counts = T*K per source (all entries valid)
    assert (lay.num_tokens_per_expert.sum(axis=1) == T * K).all()
    # T <= sum_r cnt_rank <= T*min(K,R)
    tot_r = lay.num_tokens_per_rank.sum(axis=1)
    assert (tot_r >= T).all() and (tot_r <= T * min(K, R)).all()
    # per token: number of ranks = distinct ranks of its experts
    distinct = np.array([[len(set((topk[s, t] // L).tolist())) for t in range(T)]
                         for s in range(R)])
    assert np.array_equal(lay.is_token_in_rank.sum(axis=2), distinct)
    # rank prefix matrix: last row = column totals, first differences = counts
    rpm = lay.rank_prefix_matrix
    assert np.array_equal(rpm[-1], lay.num_tokens_per_rank.sum(axis=0))
    assert np.array_equal(np.diff(rpm, axis=0, prepend=0), lay.num_tokens_per_rank)
    if w.mode == orc.MODE_MSG:
        assert (lay.send_pos == -1).all()
        return
    # send_pos is a bijection onto the filled rows, and inside each expert
    # segment (s, t, k) increases with the row
    sp = lay.send_pos.reshape(-1)
    assert len(np.unique(sp)) == sp.size
    e = topk.reshape(-1)
    for ee in range(w.E):
        rows = sp[e == ee]
        flat = np.nonzero(e == ee)[0]
        assert np.array_equal(np.sort(rows), lay.expert_start[ee] + np.arange(rows.size))
        assert np.all(np.diff(flat[np.argsort(rows)]) > 0)


def test_normal_alignment_segments():
    w = inputs.small(R=4, T=32, H=128, E=16, K=4, seed=5)
    topk = inputs.gen_topk(w)
    p = orc.Problem(4, 32, 128, 16, 4, align=8)
    lay = orc.layout(p, topk)
    assert (lay.expert_start % 8 == 0).all()
    assert (lay.rows_per_rank % 8 == 0).all()
    assert np.array_equal(lay.row_base[:-1], np.concatenate([[0], np.cumsum(lay.rows_per_rank)[:-1]]))
    # padding rows carry -1 in recv_src_idx
    filled = np.zeros(lay.total_rows, bool)
    filled[lay.send_pos.reshape(-1)] = True
    assert (lay.recv_src_idx[~filled] == -1).all()
    assert (lay.recv_src_idx[filled] >= 0).all()


try:
    from hypothesis import HealthCheck, given, settings
    from hypothesis import strategies as st
except ImportError:  # pragma: no cover - hypothesis is optional
    given = None


if given is not None:
    @st.composite
    def tiny_routings(draw):
        """Tiny problems with arbitrary ids in [-1, E): masked entries,
        duplicates within a token, every alignment and both slot modes."""
        R = draw(st.integers(1, 4))
        E = R * draw(st.integers(1, 4))
        K = draw(st.integers(1, min(E, 5)))
        T = draw(st.integers(0, 10))
        mode = draw(st.sampled_from([orc.MODE_NORMAL, orc.MODE_LL]))
        align = draw(st.sampled_from([1, 2, 3, 5])) if mode == orc.MODE_NORMAL else 1
        ids = draw(st.lists(st.integers(-1, E - 1), min_size=R * T * K, max_size=R * T * K))
        return R, T, E, K, align, mode, np.array(ids, np.int32).reshape(R, T, K)

    @settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
    @given(tiny_routings())
    def test_layout_matches_brute_force_on_arbitrary_routings(case):
        R, T, E, K, align, mode, topk = case
        p = orc.Problem(R, T, 128, E, K, align=align, mode=mode)
        lay = orc.layout(p, topk)
        cnt_e, cnt_r, in_rank, rpm, n, start, send_pos, send_head = brute_layout(p, topk)
        assert np.array_equal(lay.num_tokens_per_expert, cnt_e)
        assert np.array_equal(lay.num_tokens_per_rank, cnt_r)
        assert np.array_equal(lay.is_token_in_rank, in_rank)
        assert np.array_equal(lay.rank_prefix_matrix, rpm)
        assert np.array_equal(lay.recv_tokens_per_expert, n)
        assert np.array_equal(lay.expert_start, start)
        assert np.array_equal(lay.send_pos, send_pos)
        assert np.array_equal(lay.send_head, send_head)
        overflow = mode == orc.MODE_LL and (n > R * T).any()
        assert bool(lay.err & orc.ERR_LL_OVERFLOW) == bool(overflow)
