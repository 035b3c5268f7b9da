"""Pins for the oracle's scalar codecs (FP8 E4M3, bf16 rounding, scales).

Each check ties the oracle to something other than itself: the OCP E4M3
closed form, PyTorch's own float8_e4m3fn / bfloat16 casts (library
routines), exact rational arithmetic, or invariants of the format.
"""
import concurrent.futures as cf
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from oracle import oracle as orc


def torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_closed_form():
    # OCP E4M3 (no infinities): value = (-1)^s * 2^(e-7) * (1 + m/8), e > 0;
    # (-1)^s * 2^-6 * (m/8) for e == 0; S.1111.111 is NaN.  Also against
    # torch's float8_e4m3fn -> float32 conversion.
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        got = orc.e4m3_decode(c)
        if e == 15 and m == 7:
            assert math.isnan(got) and math.isnan(ref[c])
            continue
        mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        want = -mag if s else mag
        assert got == want == ref[c], c


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = np.array([orc.e4m3_decode(c) for c in codes], np.float32)
    assert np.array_equal(orc.e4m3_encode(vals), codes)


def _chunk(lo: int, hi: int) -> int:
    bits = np.arange(lo, hi, dtype=np.uint32)
    v = bits.view(np.float32)
    a = orc.e4m3_encode(v)
    b = torch_e4m3(v)
    return int((a != b).sum())


def test_encode_exhaustive_vs_torch():
    """Every non-negative fp32 bit pattern below 464 (above it the cast is
    saturating by this oracle's reading and NaN for torch)."""
    hi = int(np.array([464.0], np.float32).view(np.uint32)[0])
    step = 1 << 24
    jobs = [(lo, min(hi, lo + step)) for lo in range(0, hi, step)]
    with cf.ThreadPoolExecutor(8) as ex:
        bad = sum(ex.map(lambda j: _chunk(*j), jobs))
    assert bad == 0


def test_encode_negative_sample_and_sign():
    g = np.random.default_rng(5)
    bits = g.integers(0, 0x43E80000, size=1 << 22, dtype=np.uint32) | np.uint32(0x80000000)
    v = bits.view(np.float32)
    assert np.array_equal(orc.e4m3_encode(v), torch_e4m3(v))
    assert orc.e4m3_encode(np.array([-0.0, -1e-30, 0.0], np.float32)).tolist() == [0x80, 0x80, 0]


def test_encode_saturates_above_448():
    v = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e6, 3e38], np.float32)
    assert orc.e4m3_encode(v).tolist() == [0x7E] * 7
    assert orc.e4m3_encode(-v).tolist() == [0xFE] * 7


def _bf16_exact(x: Fraction) -> int:
    """Round a rational to bf16 (nearest-even) by integer arithmetic."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)               # subnormal spacing below 2^-126
    q = a / Fraction(2) ** (e - 7)  # 8 significant bits
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** (e - 7)
    f = np.array([float(val)], np.float32)
    return sign | int(f.view(np.uint32)[0] >> 16)


def test_bf16_from_double_exact_rational():
    g = np.random.default_rng(11)
    vals = list(g.standard_normal(3000) * 10.0 ** g.integers(-30, 30, 3000))
    # ties and near-ties at 8 significant bits, including double-rounding traps
    for base in [1.0, 1.5, 3.0, 255.0, 2.0 ** -120]:
        ulp = base * 2.0 ** -8
        vals += [base + ulp / 2, base + ulp / 2 + base * 2.0 ** -40, base + ulp * 1.5,
                 base + ulp / 2 - base * 2.0 ** -40, -(base + ulp / 2)]
    vals += [2.0 ** -130, 3 * 2.0 ** -134, 2.0 ** -127 * 1.3]
    for v in vals:
        assert orc.bf16_from_double(v) == _bf16_exact(Fraction(v)), v


def test_bf16_from_double_vs_torch_on_float_values():
    # double -> bf16 in torch goes through float; for inputs that are floats
    # already this is a single rounding, so the results must agree.
    g = np.random.default_rng(3)
    v = (g.standard_normal(20000) * 50).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_double(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, ref)


def test_fp8_scale_f32_is_ieee_division():
    g = np.random.default_rng(7)
    amax = np.abs(g.standard_normal(5000).astype(np.float32)) * np.float32(3)
    amax[:10] = 0
    want = np.maximum(amax, np.float32(1e-4)) / np.float32(448.0)  # numpy fp32 divide
    got = np.array([orc.fp8_scale_f32(float(a)) for a in amax], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fp8_scale_ue8m0_is_ceil_pow2():
    g = np.random.default_rng(8)
    amax = np.abs(g.standard_normal(5000).astype(np.float32)) * np.float32(100)
    amax = np.concatenate([amax, np.float32(448.0) * 2.0 ** np.arange(-20, 20, dtype=np.float32)])
    for a in amax:
        ex = orc.fp8_scale_ue8m0(float(a))
        r = Fraction(float(np.float32(max(a, np.float32(1e-4))) / np.float32(448.0)))
        sc = Fraction(2) ** (ex - 127)
        assert sc >= r and sc / 2 < r, (a, ex)
