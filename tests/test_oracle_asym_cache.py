"""Pins for the oracle's asymmetric cache format (the geometry flag `asymmetric`).

EchoKV, "Future work" (upstreaming into vLLM): its fork keeps the paged cache itself at INT2/4/8
in KIVI's form, i.e. with the asymmetric quantizer ("Show the math": zero point and scale from a
group's minimum and maximum). The reading here keeps the cache's groups (Behavior-Guided KV-Cache
Quantization, "K/V Role-Aware Low-Bit Quantization": keys per page and channel, values per token)
and gives every group a zero point m (its minimum), a scale s = RU16((max - m) / (2^b - 1)) and
codes u in [0, 2^b - 1], an element being m + u * s.

Nothing below re-types the oracle's formula or reads the pools through the oracle's own
accessors: the test decodes the section bytes from the layout the header describes and checks
  * every code against a literal argmin over all 2^b codes in exact rationals (ties to the even
    code), every zero point against the group's exact minimum and every scale against the least
    fp16 at or above the exact quotient;
  * the round trip |x - (m + u s)| <= s/2 with s above (max - m) / (2^b - 1) by less than one fp16
    step, so the error stays within (max - min) / (2 (2^b - 1)) plus half that step;
  * inputs on an exact grid come back bit for bit, and attention over them equals softmax
    attention over the inputs themselves;
  * writing a page token by token leaves the same bytes as writing it at once (the open page's
    keys are re-quantized from the FP16 ring on every write);
  * the section size P*D*b/4 + 4*D + 4*P.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from mixed_precision_quantized_kv_amd import synth

P, R = 16, 64
TIER = {2: 0, 4: 1, 8: 2, 16: 3}


def f16(bits) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def ru16_exact(x: Fraction) -> int:
    """bits of the smallest fp16 >= x (x >= 0), by bisection over the ordered positive patterns"""
    lo, hi = 0, 0x7C00
    while lo < hi:
        mid = (lo + hi) // 2
        if Fraction(f16(mid)) >= x:
            hi = mid
        else:
            lo = mid + 1
    return lo


def field(sec: np.ndarray, off: int, i: int, bits: int) -> int:
    """code i of the code sequence at byte `off`, as the header lays it out"""
    per = 32 // bits
    w, k = divmod(i, per)
    word = int.from_bytes(bytes(sec[off + 4 * w: off + 4 * w + 4]), "little")
    return (word >> (16 * (k % 2) + bits * (k // 2))) & ((1 << bits) - 1)


def rd16(sec, off) -> int:
    return int(sec[off]) | (int(sec[off + 1]) << 8)


class Section:
    """one asymmetric section decoded from its bytes"""

    def __init__(self, sec, bits, d):
        cb = P * d * bits // 8
        self.sec, self.bits, self.d = sec, bits, d
        self.kzero = [rd16(sec, cb + 2 * c) for c in range(d)]
        self.kscale = [rd16(sec, cb + 2 * d + 2 * c) for c in range(d)]
        self.voff = cb + 4 * d
        self.vzero = [rd16(sec, 2 * cb + 4 * d + 2 * t) for t in range(P)]
        self.vscale = [rd16(sec, 2 * cb + 4 * d + 2 * P + 2 * t) for t in range(P)]

    def kcode(self, t, c):
        return field(self.sec, 0, t * self.d + c, self.bits)

    def vcode(self, t, c):
        return field(self.sec, self.voff, ((t // 4) * self.d + c) * 4 + t % 4, self.bits)


def section(g, pools, handle, kv, bits):
    tier, idx = handle >> 30, handle & 0x3FFFFFFF
    sb = oracle.section_bytes(g, bits)
    base = (idx * g.num_kv_heads + kv) * sb
    return pools.arrays[tier][base: base + sb]


def check_group(xs, zero_bits, scale_bits, codes, bits):
    """the asymmetric quantizer of one group, against exact rationals"""
    top = (1 << bits) - 1
    X = [Fraction(f16(x)) for x in xs]
    mn, mx = min(X), max(X)
    assert Fraction(f16(zero_bits)) == mn
    if mn == 0:
        assert zero_bits == 0                          # +0, whatever the zeros' signs
    quot = (mx - mn) / top
    if quot == 0:
        assert scale_bits == 0 and all(u == 0 for u in codes)
        return
    assert scale_bits == ru16_exact(quot)
    s = Fraction(f16(scale_bits))
    assert s - quot < Fraction(f16(scale_bits)) - Fraction(f16(scale_bits - 1))
    for x, u in zip(X, codes):
        dist = [abs(x - (mn + v * s)) for v in range(top + 1)]
        best = min(dist)
        cands = [v for v in range(top + 1) if dist[v] == best]
        want = cands[0] if len(cands) == 1 else [v for v in cands if v % 2 == 0][0]
        assert u == want, (float(x), u, want)
        assert abs(x - (mn + u * s)) <= s / 2


def write(g, bt, K, V, chunks, cap=(64, 64, 64, 64)):
    pools = oracle.Pools(g, list(cap))
    ring = np.zeros((K.shape[0], R, g.num_kv_heads, g.head_dim), dtype=np.uint16)
    p = 0
    for n in chunks:
        oracle.quant_write(g, pools, bt, np.full(K.shape[0], p, np.int32), K[:, p:p + n],
                           V[:, p:p + n], ring)
        p += n
    return pools, ring


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_section_size(bits):
    for d in (64, 128):
        g = oracle.geom(8, 2, d, asymmetric=True)
        assert oracle.section_bytes(g, bits) == P * d * bits // 4 + 4 * d + 4 * P
        assert oracle.block_bytes(g, bits) == 2 * (P * d * bits // 4 + 4 * d + 4 * P)
        assert oracle.section_bytes(g, 16) == 4 * P * d      # the FP16 tier is unchanged
        gs = oracle.geom(8, 2, d)
        assert oracle.section_bytes(gs, bits) == P * d * bits // 4 + 2 * d + 2 * P


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_are_the_exact_argmin(bits):
    n, hkv, d = 37, 2, 64                               # pages 0, 1 full, page 2 holds 5 tokens
    g = oracle.geom(4, hkv, d, asymmetric=True)
    rng = np.random.default_rng(40 + bits)
    mult = np.where(np.arange(d) % 13 == 5, 10.0, 1.0).astype(np.float32)
    K = synth.normal_f16(rng, (1, n, hkv, d), mult)
    V = synth.normal_f16(rng, (1, n, hkv, d))
    K[0, 3, 0, 7] = 0x8000                              # a negative zero in a group
    V[0, 20, 1, :] = V[0, 20, 1, 0]                      # a constant value vector
    bt = synth.block_table([[TIER[bits]] * 3], 8, [64, 64, 64, 64], rng)
    pools, _ = write(g, bt, K, V, [9, 20, 8])
    for kv in range(hkv):
        for page in range(3):
            sec = Section(section(g, pools, int(bt[0, page]), kv, bits), bits, d)
            toks = list(range(page * P, min(n, page * P + P)))
            for c in range(d):
                xs = [int(K[0, t, kv, c]) for t in toks]
                codes = [sec.kcode(t - page * P, c) for t in toks]
                check_group(xs, sec.kzero[c], sec.kscale[c], codes, bits)
            for t in toks:
                slot = t - page * P
                xs = [int(V[0, t, kv, c]) for c in range(d)]
                codes = [sec.vcode(slot, c) for c in range(d)]
                check_group(xs, sec.vzero[slot], sec.vscale[slot], codes, bits)
            for slot in range(len(toks), P):            # empty slots: zero code, scale, zero point
                assert sec.vzero[slot] == 0 and sec.vscale[slot] == 0
                assert all(sec.kcode(slot, c) == 0 and sec.vcode(slot, c) == 0 for c in range(d))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequant_matches_the_bytes_and_the_bound(bits):
    n, hkv, d = 40, 1, 64
    g = oracle.geom(2, hkv, d, asymmetric=True)
    rng = np.random.default_rng(bits)
    K = synth.normal_f16(rng, (1, n, hkv, d))
    V = synth.normal_f16(rng, (1, n, hkv, d))
    bt = synth.block_table([[TIER[bits]] * 3], 8, [64, 64, 64, 64], rng)
    pools, _ = write(g, bt, K, V, [n])
    Kd, Vd = oracle.dequant_kv(g, pools, bt[0], n, 0)
    top = (1 << bits) - 1
    Kf = K[0, :, 0].view(np.float16).astype(np.float64)
    Vf = V[0, :, 0].view(np.float16).astype(np.float64)
    for t in range(n):
        page, slot = divmod(t, P)
        sec = Section(section(g, pools, int(bt[0, page]), 0, bits), bits, d)
        for c in range(d):
            s, m = f16(sec.kscale[c]), f16(sec.kzero[c])
            assert Kd[t, c] == m + sec.kcode(slot, c) * s
            toks = range(page * P, min(n, page * P + P))
            rng_k = max(Kf[u, c] for u in toks) - min(Kf[u, c] for u in toks)
            assert abs(Kf[t, c] - Kd[t, c]) <= s / 2
            assert s / 2 <= rng_k / (2 * top) + (s - f16(sec.kscale[c] - 1)) / 2 + 1e-300
        s, m = f16(sec.vscale[slot]), f16(sec.vzero[slot])
        for c in range(d):
            assert Vd[t, c] == m + sec.vcode(slot, c) * s
            assert abs(Vf[t, c] - Vd[t, c]) <= s / 2


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_grid_round_trip_and_attention(bits):
    """groups spanning m .. m + (2^b - 1) * 2^e exactly: the cache returns its inputs, and the
    attention over it is softmax attention over the inputs"""
    n, hkv, hq, d = 45, 2, 6, 64
    top = (1 << bits) - 1
    g = oracle.geom(hq, hkv, d, asymmetric=True)
    rng = np.random.default_rng(7 * bits)
    K = np.zeros((n, hkv, d))
    V = np.zeros((n, hkv, d))
    for page in range(3):
        toks = np.arange(page * P, min(n, page * P + P))
        for kv in range(hkv):
            for c in range(d):
                e = -6 + (c + 3 * page + kv) % 5
                m = -(int(rng.integers(0, 9)) + (c % 3)) * 2.0 ** e
                u = rng.integers(0, top + 1, size=toks.size)
                u[(c + page) % toks.size] = 0
                u[(c + page + 1) % toks.size] = top
                K[toks, kv, c] = m + u * 2.0 ** e
    for t in range(n):
        for kv in range(hkv):
            e = -5 + (t + kv) % 4
            m = -(int(rng.integers(0, 5))) * 2.0 ** e
            u = rng.integers(0, top + 1, size=d)
            u[t % d], u[(t + 1) % d] = 0, top
            V[t, kv] = m + u * 2.0 ** e
    K16, V16 = K.astype(np.float16), V.astype(np.float16)
    assert np.array_equal(K16.astype(np.float64), K) and np.array_equal(V16.astype(np.float64), V)
    Kb, Vb = K16.view(np.uint16)[None], V16.view(np.uint16)[None]
    bt = synth.block_table([[TIER[bits]] * 3], 8, [64, 64, 64, 64], rng)
    pools, _ = write(g, bt, Kb, Vb, [1, 14, 30])
    for kv in range(hkv):
        Kd, Vd = oracle.dequant_kv(g, pools, bt[0], n, kv)
        assert np.array_equal(Kd, K[:, kv]) and np.array_equal(Vd, V[:, kv])
    q = synth.normal_f16(rng, (1, hq, d))
    scale = np.float32(1 / 8)
    out = oracle.decode_attn(g, pools, bt, np.array([n], np.int32), q, float(scale))
    qf = q[0].view(np.float16).astype(np.float64)
    for h in range(hq):
        kv = h // (hq // hkv)
        lg = float(scale) * (K[:, kv] @ qf[h])
        w = np.exp(lg - lg.max())
        ref = (w @ V[:, kv]) / w.sum()
        assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_token_by_token_equals_one_write(bits):
    n, hkv, d = 35, 2, 64
    g = oracle.geom(4, hkv, d, asymmetric=True)
    rng = np.random.default_rng(300 + bits)
    K = synth.normal_f16(rng, (2, n, hkv, d))
    V = synth.normal_f16(rng, (2, n, hkv, d))
    bt = synth.block_table([[TIER[bits]] * 3, [TIER[bits]] * 3], 8, [64, 64, 64, 64], rng)
    a, ra = write(g, bt, K, V, [1] * n)
    b, rb = write(g, bt, K, V, [n])
    for t in range(4):
        assert np.array_equal(a.arrays[t], b.arrays[t])
    assert np.array_equal(ra, rb)


def test_striped_widths_and_fp16_pages():
    """pages of one sequence at different widths (and FP16) in one asymmetric geometry"""
    n, hkv, d = 70, 1, 64
    g = oracle.geom(2, hkv, d, asymmetric=True)
    rng = np.random.default_rng(5)
    K = synth.normal_f16(rng, (1, n, hkv, d))
    V = synth.normal_f16(rng, (1, n, hkv, d))
    widths = [8, 2, 16, 4, 2]
    bt = synth.block_table([[TIER[b] for b in widths]], 8, [64, 64, 64, 64], rng)
    pools, _ = write(g, bt, K, V, [n])
    Kd, Vd = oracle.dequant_kv(g, pools, bt[0], n, 0)
    Kf = K[0, :, 0].view(np.float16).astype(np.float64)
    Vf = V[0, :, 0].view(np.float16).astype(np.float64)
    for page, b in enumerate(widths):
        toks = slice(page * P, min(n, page * P + P))
        if b == 16:
            assert np.array_equal(Kd[toks], Kf[toks]) and np.array_equal(Vd[toks], Vf[toks])
        else:
            sec = Section(section(g, pools, int(bt[0, page]), 0, b), b, d)
            ks = np.array([f16(x) for x in sec.kscale])
            assert np.all(np.abs(Kd[toks] - Kf[toks]) <= ks / 2)
