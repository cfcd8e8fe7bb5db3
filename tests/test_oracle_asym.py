"""Pins for the oracle's asymmetric (KIVI-style) quantizer and the canary built on it.

EchoKV, "Show the math - what the canary actually computes": the canary's quant_b quantizes each
group asymmetrically, after KIVI -- per group a zero point and a scale spanning [min, max].
The oracle's reading: zero point = the group minimum m, scale s = RU16((max - m) / (2^b - 1)),
codes round-half-even((x - m) / s) in [0, 2^b - 1], value m + code * s.

What pins it (none of these re-types the oracle's formula):
  * hand-worked groups;
  * the scale against exact rational arithmetic: s >= (max - m)/(2^b - 1) and the fp16 value
    below s is smaller than that quotient (minimality), over sampled fp16 ranges of every size;
  * the codes against a literal argmin over all 2^b codes in exact rationals, ties to even;
  * the round-trip bound |x - value| <= s/2, with s above (max - m) / (2^b - 1) by less than one
    fp16 step;
  * special cases: a constant group (scale 0, exact), signed zeros, values on an exact grid
    (the copy is exact, and the canary then reads exactly 0 KL).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

POS_FINITE = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)


def f16(bits) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def as_bits(vals) -> np.ndarray:
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


def test_worked_groups():
    s, z, q = oracle.quantize_group_asym(as_bits([1.0, 2.0, 0.0, -1.0]), 2)
    assert (f16(s), f16(z), list(q)) == (1.0, -1.0, [2, 3, 1, 0])
    s, z, q = oracle.quantize_group_asym(as_bits([0.0, 0.5, 7.5, 3.25]), 4)
    # range 7.5 over 15 steps: s = 0.5; 3.25 / 0.5 = 6.5 -> 6 (ties to even)
    assert (f16(s), f16(z), list(q)) == (0.5, 0.0, [0, 1, 15, 6])
    s, z, q = oracle.quantize_group_asym(as_bits([-3.0, -1.0]), 8)
    # range 2 over 255 steps: RU16(2/255) = the fp16 just above 0.0078431...
    assert f16(s) >= 2 / 255 and f16(z) == -3.0 and list(q) == [0, 255]


def exact_scale_ok(s_bits, lo, hi, bits):
    quot = (Fraction(f16(hi)) - Fraction(f16(lo))) / ((1 << bits) - 1)
    s = Fraction(f16(s_bits))
    if quot == 0:
        return s_bits == 0
    below = Fraction(f16(s_bits - 1)) if s_bits > 0 else Fraction(-1)
    return s >= quot and below < quot


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_scale_is_least_fp16_above_exact_quotient(bits):
    g = np.random.default_rng(bits)
    vals = POS_FINITE.view(np.float16).astype(np.float64)
    for _ in range(4000):
        a, b = g.integers(0, POS_FINITE.size, 2)
        sa, sb = g.integers(0, 2, 2)
        x = np.array([vals[a] * (-1) ** sa, vals[b] * (-1) ** sb])
        xb = as_bits(x)
        s, z, _ = oracle.quantize_group_asym(xb, bits)
        lo, hi = (xb[0], xb[1]) if x[0] <= x[1] else (xb[1], xb[0])
        assert exact_scale_ok(s, lo, hi, bits), (x, bits, s)
        assert f16(z) == min(x)


def argmin_code(x, m, s, bits):
    best, err = None, None
    for q in range((1 << bits)):
        e = abs(x - (m + q * s))
        if err is None or e < err or (e == err and q % 2 == 0 and best % 2 == 1):
            best, err = q, e
    return best


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_are_the_argmin_and_bounded(bits):
    g = np.random.default_rng(10 + bits)
    for trial in range(60):
        n = int(g.integers(1, 17))
        kind = trial % 4
        if kind == 0:
            x = g.standard_normal(n)
        elif kind == 1:
            x = g.uniform(1.0, 2.0, n)                     # all positive: the zero point matters
        elif kind == 2:
            x = g.standard_normal(n) * 2.0 ** -16           # subnormal scales
        else:
            x = np.concatenate([g.standard_normal(n - 1), [g.choice([-1, 1]) * 300.0]])
        xb = as_bits(x)
        s, z, q = oracle.quantize_group_asym(xb, bits)
        m, sd = Fraction(f16(z)), Fraction(f16(s))
        xs = [Fraction(f16(h)) for h in xb]
        hi = max(xs)
        for xi, qi in zip(xs, q):
            if sd == 0:
                assert qi == 0 and xi == m
                continue
            assert qi == argmin_code(xi, m, sd, bits), (x, bits)
            assert abs(xi - (m + qi * sd)) <= sd / 2
            # the scale exceeds the exact quotient by less than one fp16 step: 2^-10 of it
            # for normal scales, 2^-24 absolute for subnormal ones
            quot = (hi - m) / ((1 << bits) - 1)
            assert sd <= quot * (1 + Fraction(1, 1024)) or sd - quot < Fraction(1, 1 << 24)


def test_constant_group_and_signed_zero():
    s, z, q = oracle.quantize_group_asym(as_bits([3.5, 3.5, 3.5]), 4)
    assert s == 0 and f16(z) == 3.5 and list(q) == [0, 0, 0]
    s, z, q = oracle.quantize_group_asym(as_bits([-0.0, 0.0, 1.0]), 2)
    assert z == 0x0000 and f16(s) == 1 / 3 or f16(s) >= 1 / 3
    assert list(q)[:2] == [0, 0]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_grid_values_are_exact(bits):
    g = np.random.default_rng(20 + bits)
    top = (1 << bits) - 1
    for _ in range(50):
        s = 2.0 ** int(g.integers(-8, 2))
        m = float(np.float16(g.standard_normal()))
        k = np.concatenate([[0, top], g.integers(0, top + 1, 14)])
        x = m + k * s
        if not np.array_equal(np.asarray(x, np.float16).astype(np.float64), x):
            continue                                       # not representable: skip
        sb, zb, q = oracle.quantize_group_asym(as_bits(x), bits)
        assert f16(sb) == s and f16(zb) == m and np.array_equal(q, k)


def test_canary_reads_zero_on_an_exact_grid_and_positive_otherwise():
    g = np.random.default_rng(7)
    H, HQ, D, R = 2, 4, 64, 64
    og = oracle.geom(HQ, H, D, 16, R)
    N = 40
    # every (page, channel) group of the ring sits on a 3-step grid: INT2 asymmetric is exact
    ring = np.zeros((1, R, H, D), dtype=np.float64)
    for p in range(N):
        ring[0, p] = g.integers(0, 4, size=(H, D)) * 0.25 - 0.5
    for page in range(0, N, 16):                           # make every group span the full grid
        ring[0, page, :, :] = -0.5
        ring[0, min(page + 1, N - 1), :, :] = 0.25
    rb = ring.astype(np.float16).view(np.uint16)
    q = g.standard_normal((1, HQ, D)).astype(np.float16).view(np.uint16)
    kl, rows = oracle.canary_kl(og, rb, np.array([N], np.int32), q, 0.125, asymmetric=True)
    assert np.all(rows >= 0)
    assert kl[0] == 0.0                                    # INT2: the copy is the keys
    assert 0.0 <= kl[1] < 1e-4 and 0.0 <= kl[2] < 1e-4    # the grid is off by < 1 scale step
    # the symmetric copy of the same keys is not exact at INT2 (its three levels are -s, 0, s)
    kls, _ = oracle.canary_kl(og, rb, np.array([N], np.int32), q, 0.125, asymmetric=False)
    assert kls[0] > 0.0
