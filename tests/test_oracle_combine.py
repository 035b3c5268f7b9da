"""Pins for the oracle's combine (top-k weighted gather-reduce).

Inputs are chosen so the exact result is known independently: dyadic
weights with small-integer or bf16 expert outputs make every partial sum
exact, so the answer is one rounding of an exact rational, computed here
with Python integers/fractions or a single float32 -> bf16 cast.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import inputs
from oracle import oracle as orc


def f32_to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def dyadic_weights(shape, seed):
    g = np.random.default_rng(seed)
    return (g.integers(1, 64, size=shape) / 64.0).astype(np.float32)


@pytest.mark.parametrize("mode", [orc.MODE_NORMAL, orc.MODE_LL])
def test_identity_expert_gives_x_times_weight_sum(mode):
    # y = dispatched rows (identity expert): out = bf16(x * sum_k w_k).
    w = inputs.small(R=3, T=16, H=256, E=12, K=4, mode=mode, seed=21)
    topk = inputs.gen_topk(w)
    x = inputs.gen_x(w)
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=mode)
    lay = orc.layout(p, topk)
    cap = lay.total_rows if mode == orc.MODE_NORMAL else w.E * w.R * w.T
    _, recv, _ = orc.dispatch(p, x, topk, lay.send_pos, cap)
    wt = dyadic_weights((w.R, w.T, w.K), 1)
    err, out = orc.combine(p, recv, wt, lay.send_pos)
    assert err == 0
    # x has 8 significant bits, sum(w) is a multiple of 2^-6 below 4: the
    # product is exact in fp32, so one bf16 cast rounds the exact value.
    want = f32_to_bf16(bf16_to_f32(x) * wt.sum(axis=2, dtype=np.float32)[..., None])
    assert np.array_equal(out, want)


def test_integer_outputs_exact_rational_rounding():
    w = inputs.small(R=2, T=10, H=128, E=8, K=4, seed=22)
    topk = inputs.masked_topk(w, inputs.gen_topk(w), 0.2)
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K)
    lay = orc.layout(p, topk)
    g = np.random.default_rng(5)
    yi = g.integers(-200, 200, size=(lay.total_rows, w.H))
    y = f32_to_bf16(yi.astype(np.float32))      # exact: |y| < 256
    wt = (g.integers(1, 1 << 20, size=(w.R, w.T, w.K)) / float(1 << 20)).astype(np.float32)
    err, out = orc.combine(p, y, wt, lay.send_pos)
    assert err == 0
    for s in range(w.R):
        for t in range(w.T):
            for c in range(0, w.H, 17):
                acc = Fraction(0)
                for k in range(w.K):
                    r = lay.send_pos[s, t, k]
                    if r >= 0:
                        acc += Fraction(float(wt[s, t, k])) * int(yi[r, c])
                # round the exact rational once (a float32 cast first
                # would round twice)
                want = _round_bf16(acc)
                assert out[s, t, c] == want, (s, t, c)


def _round_bf16(x: Fraction) -> int:
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = a / Fraction(2) ** (e - 7)
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2):
        n += 1
    f = np.array([float(Fraction(n) * Fraction(2) ** (e - 7))], np.float32)
    return sign | int(f.view(np.uint32)[0] >> 16)


def test_masked_tokens_give_zero_and_token_list():
    w = inputs.small(R=2, T=6, H=128, E=4, K=2, seed=23)
    topk = inputs.gen_topk(w)
    topk[0, 2, :] = -1
    topk[1, 5, :] = -1
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K)
    lay = orc.layout(p, topk)
    y = inputs.gen_y(w, lay.total_rows)
    wt = inputs.gen_weights(w)
    err, out = orc.combine(p, y, wt, lay.send_pos)
    assert err == 0
    assert (out[0, 2] == 0).all() and (out[1, 5] == 0).all()
    toks = np.array([11, 0, 5], np.int64)
    err, sub = orc.combine(p, y, wt, lay.send_pos, toks)
    assert np.array_equal(sub, out.reshape(-1, w.H)[toks])


def test_cancellation_is_rounded_once():
    # w0*y - w1*y with w0 = w1 + 2^-20: the exact result is 2^-20 * y; a
    # sum rounded to bf16 after each term would lose it.
    p = orc.Problem(1, 1, 128, 2, 2)
    topk = np.array([[[0, 1]]], np.int32)
    lay = orc.layout(p, topk)
    y = np.zeros((2, 128), np.uint16)
    y[0] = f32_to_bf16(np.full(128, 1.0, np.float32))
    y[1] = f32_to_bf16(np.full(128, -1.0, np.float32))
    wt = np.array([[[0.5 + 2.0 ** -20, 0.5]]], np.float32)
    err, out = orc.combine(p, y, wt, lay.send_pos)
    assert (bf16_to_f32(out) == np.float32(2.0 ** -20)).all()
