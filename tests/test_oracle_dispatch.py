"""Pins for the oracle's dispatch (bf16 copy, FP8 quantisation, scale layout).

bf16 rows are checked by plain indexing; FP8 codes against PyTorch's
float8_e4m3fn cast of NumPy fp32 quotients (library routines); scales
against NumPy fp32 division and the power-of-two bound; plus the format's
invariants (each group's largest magnitude encodes to +-448, the
dequantisation error bound).
"""
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


def setup(w, align=1, mfrac=0.0, dfrac=0.0):
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac)
    x = inputs.gen_x(w)
    p = orc.Problem(w.R, w.T, w.H, w.E, w.K, align=align, mode=w.mode, quant=w.quant)
    lay = orc.layout(p, topk)
    cap = lay.total_rows if w.mode == orc.MODE_NORMAL else w.E * w.R * w.T
    return p, topk, x, lay, cap


@pytest.mark.parametrize("mode", [orc.MODE_NORMAL, orc.MODE_LL])
@pytest.mark.parametrize("align,mfrac,dfrac", [(1, 0.0, 0.0), (4, 0.2, 0.2)])
def test_bf16_rows_are_copies(mode, align, mfrac, dfrac):
    w = inputs.small(R=4, T=24, H=256, E=16, K=4, mode=mode, seed=3)
    p, topk, x, lay, cap = setup(w, align, mfrac, dfrac)
    err, recv, sc = orc.dispatch(p, x, topk, lay.send_pos, cap)
    assert err == 0 and sc is None
    filled = np.zeros(cap, bool)
    for s in range(w.R):
        for t in range(w.T):
            for k in range(w.K):
                r = lay.send_pos[s, t, k]
                if r >= 0:
                    assert np.array_equal(recv[r], x[s, t])
                    filled[r] = True
    assert (recv[~filled] == 0).all()


def _check_fp8(w, p, x, lay, recv, scales, cap):
    G, RT = w.G, w.R * w.T
    xf = bf16_to_f32(x).reshape(w.R, w.T, G, 128)
    amax = np.abs(xf).max(axis=3)
    for s in range(w.R):
        for t in range(w.T):
            for k in range(w.K):
                r = int(lay.send_pos[s, t, k])
                if r < 0:
                    continue
                codes = recv[r].reshape(G, 128)
                for g in range(G):
                    if w.mode == orc.MODE_LL:
                        si = (r // RT * G + g) * RT + r % RT
                    else:
                        si = g * cap + r
                    a = np.float32(max(amax[s, t, g], np.float32(1e-4)))
                    if p.quant == orc.Q_FP8_F32:
                        sc = a / np.float32(448.0)
                        assert scales[si] == sc
                        want = torch_e4m3(xf[s, t, g] / sc)
                    else:
                        ex = int(scales[si])
                        sc = np.float32(2.0 ** (ex - 127))
                        r32 = a / np.float32(448.0)
                        assert sc >= r32 and sc / 2 < r32
                        want = torch_e4m3(np.ldexp(xf[s, t, g], 127 - ex).astype(np.float32))
                    assert np.array_equal(codes[g], want), (s, t, k, g)
                    # the largest magnitude of the group lands on +-448 for f32
                    # scales; a power-of-two scale puts it in (224, 448]
                    big = np.argmax(np.abs(xf[s, t, g]))
                    mag = codes[g][big] & 0x7F
                    if p.quant == orc.Q_FP8_F32:
                        assert mag == 0x7E
                    else:
                        assert 0x76 <= mag <= 0x7E
                    # dequantisation error bound (normal codes: 2^-4 relative)
                    deq = np.array([orc.e4m3_decode(c) for c in codes[g]], np.float64) * float(sc)
                    nz = (codes[g] & 0x78) != 0
                    err = np.abs(deq - xf[s, t, g])
                    assert np.all(err[nz] <= 2.0 ** -4 * np.abs(xf[s, t, g][nz]) + 1e-30)
                    assert np.all(err[~nz] <= 2.0 ** -10 * float(sc) + 1e-30)


@pytest.mark.parametrize("mode", [orc.MODE_NORMAL, orc.MODE_LL])
@pytest.mark.parametrize("quant", [orc.Q_FP8_F32, orc.Q_FP8_UE8M0])
def test_fp8_codes_and_scales(mode, quant):
    w = inputs.small(R=2, T=6, H=384, E=8, K=3, mode=mode, quant=quant, seed=4,
                     outlier_frac=0.02, outlier_scale=50.0)
    p, topk, x, lay, cap = setup(w, 1, 0.1, 0.0)
    err, recv, scales = orc.dispatch(p, x, topk, lay.send_pos, cap)
    assert err == 0
    _check_fp8(w, p, x, lay, recv, scales, cap)


def test_fp8_zero_group_uses_floor():
    w = inputs.small(R=1, T=2, H=256, E=2, K=1, mode=orc.MODE_NORMAL, quant=orc.Q_FP8_F32)
    p = orc.Problem(1, 2, 256, 2, 1, quant=orc.Q_FP8_F32)
    x = np.zeros((1, 2, 256), np.uint16)
    topk = np.array([[[0], [1]]], np.int32)
    lay = orc.layout(p, topk)
    err, recv, scales = orc.dispatch(p, x, topk, lay.send_pos, 2)
    assert err == 0 and (recv == 0).all()
    assert np.allclose(scales, np.float32(1e-4) / np.float32(448))
    del w


def test_identity_dequant_is_exact_for_pow2_scales():
    w = inputs.small(R=2, T=8, H=256, E=4, K=2, quant=orc.Q_FP8_UE8M0, seed=9)
    p, topk, x, lay, cap = setup(w)
    err, recv, scales = orc.dispatch(p, x, topk, lay.send_pos, cap)
    rows = np.arange(cap, dtype=np.int32)
    y = orc.dequant_rows(p, recv, scales, cap, rows)
    # code * 2^k is a bf16 number whenever it is an fp32 number with <= 4 bits
    deq = np.array([[orc.e4m3_decode(c) for c in r] for r in recv], np.float32)
    for r in range(cap):
        for g in range(w.G):
            deq[r, g * 128:(g + 1) * 128] *= np.float32(2.0 ** (int(scales[g * cap + r]) - 127))
    assert np.array_equal(bf16_to_f32(y), deq)


@pytest.mark.parametrize("mode", [orc.MODE_NORMAL, orc.MODE_LL])
def test_dequant_fp32_scales_round_the_exact_product_once(mode):
    """The identity expert for fp32 scales: y = bf16(decode(code) * scale),
    the product exact (a 4-bit code times a 24-bit scale) and rounded once,
    to nearest even.  Checked against the exact rational product of
    PyTorch's float8_e4m3fn decode and the fp32 scale, rounded by integer
    arithmetic, for every finite code, scales from 2^-30 to 2^10 (bf16
    subnormal products included) and short dyadic scales whose products
    fall exactly halfway between two bf16 numbers; scales read at their
    column-major place of each layout."""
    from fractions import Fraction

    from test_oracle_codecs import _bf16_exact

    R, T, H, E, K = 2, 4, 256, 4, 2
    G = H // 128
    p = orc.Problem(R, T, H, E, K, mode=mode, quant=orc.Q_FP8_F32)
    cap = 12 if mode == orc.MODE_NORMAL else E * R * T
    rng = np.random.default_rng(17)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    codes = rng.choice(finite, (cap, H)).astype(np.uint8)
    codes[0, :finite.size] = finite
    codes[1, :finite.size] = finite[::-1]
    nsc = G * (cap if mode == orc.MODE_NORMAL else E * R * T)
    scales = np.exp2(rng.uniform(-30, 10, nsc)).astype(np.float32)
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, 1.5, 2.0 ** -20 * (1 + 2.0 ** -5),
                     np.float32(1e-4) / np.float32(448.0), 1.0], np.float32)
    scales[:ties.size] = ties
    rows = np.arange(cap, dtype=np.int32)[::-1].copy()
    y = orc.dequant_rows(p, codes, scales, cap, rows)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    RT = R * T
    for i, r in enumerate(rows.tolist()):
        for g in range(G):
            si = g * cap + r if mode == orc.MODE_NORMAL else ((r // RT) * G + g) * RT + r % RT
            sc = Fraction(float(scales[si]))
            # a zero code keeps its sign (IEEE: -0 times a positive scale is -0)
            want = [_bf16_exact(Fraction(float(v)) * sc) if v != 0 else
                    (0x8000 if np.signbit(v) else 0) for v in dec[r, g * 128:(g + 1) * 128]]
            assert y[i, g * 128:(g + 1) * 128].tolist() == want, (r, g)
