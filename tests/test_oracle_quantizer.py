"""Pins for the oracle's fp16 codec and symmetric quantizer.

What pins them (none of these re-types the oracle's own formula):
  * fp16 decode / round-to-nearest: numpy's IEEE binary16 over all 65,536 bit patterns.
  * round-up: closed-form minimality (result >= x, predecessor < x) in exact rationals.
  * scale: exact rational arithmetic (fractions) over every positive finite fp16 absmax and
    every qmax in {1, 7, 127}; the oracle decides in binary32, the test in exact arithmetic.
  * codes: literal argmin over all codes (b = 2, 4) and exact rational round-half-even (b = 8),
    over every fp16 value inside the group's range, for several scales including subnormal ones.
  * invariants: |x - q*s| <= s/2 for every element (the round-trip bound), absmax -> +-qmax.

Quantizer: symmetric uniform integer codes with one scale per group -- keys per channel, values
per token (Behavior-Guided KV-Cache Quantization, "K/V Role-Aware Low-Bit Quantization";
KV-Kaizen summary, "Three Non-Eviction Compression Axes").
"""
from fractions import Fraction

import numpy as np
import pytest

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
POS_FINITE = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16)   # +subnormal .. 65504


def f16(bits) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def frac16(bits) -> Fraction:
    return Fraction(f16(bits))


def test_f16_decode_exhaustive(orc):
    ref = ALL.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(h)) for h in ALL])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_round_nearest_matches_numpy(orc):
    vals = ALL.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    v = np.sort(vals[finite & (vals >= 0)])
    mids = (v[:-1] + v[1:]) / 2            # exact ties between neighbours (exact in double)
    probes = np.concatenate([v, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                             -mids, [65519.0, 65520.0, 1e-9, 2.0 ** -25, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = probes.astype(np.float16).view(np.uint16)
    got = np.array([orc.f64_to_f16_rne(float(x)) for x in probes], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_f16_round_up_minimal(orc):
    g = np.random.default_rng(1)
    probes = np.concatenate([g.uniform(0, 65504, 3000), np.exp(g.uniform(-20, 11, 3000)),
                             ALL.view(np.float16).astype(np.float64)[POS_FINITE.astype(np.int64)][::7],
                             [0.0, 2.0 ** -30, 65504.0]])
    for x in probes:
        h = orc.f64_to_f16_ru(float(x))
        assert Fraction(f16(h)) >= Fraction(float(x))
        if h > 0:
            assert Fraction(f16(h - 1)) < Fraction(float(x))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_scale_exhaustive_exact(orc, bits):
    """scale = smallest fp16 >= absmax/qmax, in exact rationals, for every fp16 absmax."""
    qmax = (1 << (bits - 1)) - 1
    bad = 0
    for a in POS_FINITE:
        s, codes = orc.quantize_group(np.array([a], dtype=np.uint16), bits)
        exact = frac16(a) / qmax
        if not (frac16(s) >= exact and (s == 0 or frac16(s - 1) < exact)):
            bad += 1
        # the group's absmax maps to +qmax whenever the scale is a normal fp16; at the subnormal
        # floor (absmax/qmax < 2^-24) the scale is 2^-24 and the code is absmax / 2^-24
        want = qmax if s >= 0x0400 else round(frac16(a) / frac16(s))
        if codes[0] != want:
            bad += 1
    assert bad == 0


def _group_range(a_bits: int):
    """every fp16 x with |x| <= value(a), both signs"""
    a = f16(a_bits)
    vals = POS_FINITE.view(np.float16).astype(np.float64)
    pos = POS_FINITE[vals <= a]
    return np.concatenate([[0], pos, pos | 0x8000]).astype(np.uint16)


ABSMAX_CASES = [0x3C00, 0x4248, 0x57F0, 0x7BFF, 0x1E66, 0x0400, 0x03FF, 0x0007, 0x4C00, 0x6A5B]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("a_bits", ABSMAX_CASES)
def test_codes_brute_force(orc, bits, a_bits):
    """each code is the nearest multiple of the scale (ties to the even code)."""
    qmax = (1 << (bits - 1)) - 1
    xs = _group_range(a_bits)
    if bits == 8 and xs.size > 4000:        # exact round-half-even on a sample for INT8
        g = np.random.default_rng(a_bits)
        xs = np.concatenate([xs[:200], g.choice(xs, 3000, replace=False)])
    group = np.concatenate([[a_bits], xs]).astype(np.uint16)
    s, codes = orc.quantize_group(group, bits)
    S = frac16(s)
    assert S > 0
    for x, q in zip(xs, codes[1:]):
        X = frac16(x)
        if bits < 8:                          # literal argmin over every code
            best = min(range(-qmax, qmax + 1), key=lambda c: (abs(X - c * S), c % 2))
        else:                                 # exact round-half-even of the quotient
            r = X / S
            fl = r.numerator // r.denominator
            d = r - fl
            best = fl + (1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2) else 0)
            best = max(-qmax, min(qmax, best))
        assert q == best, (hex(int(x)), int(q), best)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_roundtrip_bound_random_groups(orc, bits):
    g = np.random.default_rng(bits)
    for trial in range(300):
        n = int(g.integers(1, 129))
        scale = float(np.exp(g.uniform(-12, 9)))
        x = (g.standard_normal(n) * scale).astype(np.float16)
        x[np.abs(x) > 60000] = 0
        s, codes = orc.quantize_group(x.view(np.uint16), bits)
        S = f16(s)
        err = np.abs(x.astype(np.float64) - codes * S)
        assert np.all(err <= S / 2), (trial, err.max(), S)
        assert np.all(np.abs(codes) <= (1 << (bits - 1)) - 1)


def test_zero_group(orc):
    s, codes = orc.quantize_group(np.zeros(16, dtype=np.uint16), 4)
    assert s == 0 and np.all(codes == 0)
    s, codes = orc.quantize_group(np.array([0x8000, 0], dtype=np.uint16), 8)   # -0 and +0
    assert s == 0 and np.all(codes == 0)
