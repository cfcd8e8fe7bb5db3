"""Property tests of the oracle (hypothesis, derandomized: every run draws the same cases).

Each property is stated from its definition, not from the oracle's code:
- the symmetric quantizer (Behavior-Guided KV-Cache Quantization, "K/V Role-Aware Low-Bit
  Quantization"; readings R2-R4): for any finite fp16 group, the scale is the least fp16 at or
  above max|x| / qmax and each code is the round-half-even of x / s, checked in exact rationals;
- the asymmetric quantizer (EchoKV, "Show the math": KIVI-style groups with a zero point;
  reading R33): zero point = the group minimum, scale = least fp16 at or above
  (max - min) / (2^b - 1), code = round-half-even((x - min) / s) in [0, 2^b - 1];
- packing round-trips any code tuple at every width (whole 32-bit words of codes);
- the write (EchoKV, "How EchoKV works"; reading R7): however the tokens of a sequence are
  split into calls, the cache bytes and the ring come out the same;
- decode attention reads each page through the block table, so moving blocks to other physical
  slots leaves the output unchanged;
- the canary's divergence (EchoKV, "Show the math") is non-negative, zero for identical logits,
  and unchanged when either logit vector is shifted by a constant (softmax is).
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle

SETTINGS = dict(deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
QMAX = {2: 1, 4: 7, 8: 127}

finite_f16 = st.integers(0, 0xFFFF).filter(lambda b: (b >> 10) & 0x1F != 0x1F)


def f16(bits: int) -> Fraction:
    """the exact value of an fp16 bit pattern (every fp16 value is exact in binary64)"""
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def rne(x: Fraction) -> int:
    return round(x)                      # Fraction rounding: half to even


def least_f16_at_or_above(bits: int, target: Fraction) -> bool:
    """bits (a non-negative fp16) is the least fp16 value >= target"""
    if f16(bits) < target:
        return False
    return bits == 0 or f16(bits - 1) < target


@settings(max_examples=200, **SETTINGS)
@given(st.lists(finite_f16, min_size=1, max_size=128), st.sampled_from([2, 4, 8]))
def test_symmetric_quantizer_from_its_definition(group, bits):
    x = np.array(group, dtype=np.uint16)
    s_bits, codes = oracle.quantize_group(x, bits)
    qmax = QMAX[bits]
    a = max(abs(f16(b)) for b in group)
    if a == 0:
        assert s_bits == 0 and not codes.any()
        return
    assert s_bits < 0x8000, "the scale is not negative"
    assert least_f16_at_or_above(s_bits, a / qmax)
    s = f16(s_bits)
    for b, q in zip(group, codes):
        exact = rne(f16(b) / s)
        assert q == exact and -qmax <= q <= qmax
        assert abs(f16(b) - q * s) <= s / 2


@settings(max_examples=200, **SETTINGS)
@given(st.lists(finite_f16, min_size=1, max_size=128), st.sampled_from([2, 4, 8]))
def test_asymmetric_quantizer_from_its_definition(group, bits):
    x = np.array(group, dtype=np.uint16)
    s_bits, z_bits, codes = oracle.quantize_group_asym(x, bits)
    vals = [f16(b) for b in group]
    lo, hi = min(vals), max(vals)
    top = (1 << bits) - 1
    assert f16(z_bits) == lo                     # the zero point is the minimum, kept exactly
    if hi == lo:
        assert f16(s_bits) == 0 and not codes.any()
        return
    assert least_f16_at_or_above(s_bits, (hi - lo) / top)
    s = f16(s_bits)
    for v, u in zip(vals, codes):
        assert u == min(top, max(0, rne((v - lo) / s)))
        assert abs(v - (lo + u * s)) <= s / 2


@settings(max_examples=100, **SETTINGS)
@given(st.sampled_from([2, 4, 8]), st.data())
def test_pack_round_trips_any_codes(bits, data):
    qmax = QMAX[bits]
    n = data.draw(st.integers(1, 16)) * (32 // bits)         # whole 32-bit words
    q = np.array(data.draw(st.lists(st.integers(-qmax, qmax), min_size=n, max_size=n)), dtype=np.int32)
    packed = oracle.pack(q, bits)
    assert packed.size == n * bits // 8
    assert np.array_equal(oracle.unpack(packed, n, bits), q)


def _layer(tiers, seed, d=64, hkv=2):
    """an oracle layer whose pages have the given tiers (0..3), blocks in a seeded shuffled order"""
    g = oracle.geom(4 * hkv, hkv, d)
    cap = [sum(t == k for t in tiers) for k in range(4)]
    rng = np.random.default_rng(seed)
    slot = {k: list(rng.permutation(max(1, cap[k]))) for k in range(4)}
    bt = np.full((1, len(tiers) + 1), 0xFFFFFFFF, dtype=np.uint32)
    for p, t in enumerate(tiers):
        bt[0, p] = (t << 30) | int(slot[t].pop())
    return g, cap, bt


@settings(max_examples=40, **SETTINGS)
@given(st.integers(1, 90), st.data())
def test_write_does_not_depend_on_how_tokens_are_split_into_calls(n, data):
    pages = (n + 15) // 16
    tiers = data.draw(st.lists(st.integers(0, 3), min_size=pages, max_size=pages))
    seed = data.draw(st.integers(0, 2**16))
    cuts = sorted(set(data.draw(st.lists(st.integers(1, n - 1), max_size=6)) if n > 1 else []))
    g, cap, bt = _layer(tiers, seed)
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((1, n, g.num_kv_heads, g.head_dim)).astype(np.float16).view(np.uint16)
    V = rng.standard_normal((1, n, g.num_kv_heads, g.head_dim)).astype(np.float16).view(np.uint16)
    results = []
    for bounds in ([0, n], [0] + cuts + [n]):
        pools = oracle.Pools(g, cap)
        ring = np.zeros((1, g.ring_size, g.num_kv_heads, g.head_dim), dtype=np.uint16)
        for a, b in zip(bounds[:-1], bounds[1:]):
            oracle.quant_write(g, pools, bt, np.array([a], dtype=np.int32), K[:, a:b], V[:, a:b], ring)
        results.append(([arr.copy() for arr in pools.arrays], ring.copy()))
    (p1, r1), (p2, r2) = results
    assert all(np.array_equal(a, b) for a, b in zip(p1, p2)) and np.array_equal(r1, r2)


@settings(max_examples=30, **SETTINGS)
@given(st.integers(1, 70), st.integers(0, 2**16), st.data())
def test_attention_does_not_depend_on_where_blocks_live(n, seed, data):
    pages = (n + 15) // 16
    tiers = data.draw(st.lists(st.integers(0, 3), min_size=pages, max_size=pages))
    outs = []
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((1, n, 2, 64)).astype(np.float16).view(np.uint16)
    V = rng.standard_normal((1, n, 2, 64)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((1, 8, 64)).astype(np.float16).view(np.uint16)
    for layout_seed in (seed, seed + 1):
        g, cap, bt = _layer(tiers, layout_seed)
        pools = oracle.Pools(g, cap)
        ring = np.zeros((1, g.ring_size, 2, 64), dtype=np.uint16)
        oracle.quant_write(g, pools, bt, np.array([0], dtype=np.int32), K, V, ring)
        outs.append(oracle.decode_attn(g, pools, bt, np.array([n], dtype=np.int32), q, 0.125))
    assert np.array_equal(outs[0], outs[1])


finite_logits = st.lists(st.floats(-30, 30, allow_nan=False), min_size=1, max_size=64)


@settings(max_examples=200, **SETTINGS)
@given(finite_logits, st.data(), st.floats(-50, 50), st.floats(-50, 50))
def test_kl_is_nonnegative_zero_on_equal_logits_and_shift_invariant(l, data, c, e):
    m = data.draw(st.lists(st.floats(-30, 30, allow_nan=False), min_size=len(l), max_size=len(l)))
    l, m = np.array(l), np.array(m)
    kl = oracle.kl_logits(l, m)
    assert kl >= 0.0
    assert oracle.kl_logits(l, l) == 0.0
    # softmax ignores a constant added to its logits; so does the divergence, up to rounding
    assert oracle.kl_logits(l + c, m + e) == pytest.approx(kl, rel=1e-9, abs=1e-9)
