"""GPU parity of the asymmetric cache format (kv_geometry.asymmetric = 1) against the oracle.

EchoKV, "Future work": the paged cache itself held at INT2/4/8 in KIVI's form; "Show the math": the
KIVI-style quantizer (zero point and scale from a group's minimum and maximum). Same bar as the
symmetric format: packed codes, zero points, scales and the ring bit-exact; attention rows within
2e-3 of the oracle's fp64 result (per row: max |err| / max |ref|); the fused step equal to the
write followed by the attention, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
import oracle
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import DEV, LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3


def banner(msg):
    print(f"\n[case] asymmetric {msg}", flush=True)


def kv_inputs(rng, B, n, hkv, d, outlier_every=13, v_shift=0.75):
    """keys with x10 outlier channels; values with a per-token offset, so the zero points matter"""
    mult = np.where(np.arange(d) % outlier_every == 5, 10.0, 1.0).astype(np.float32)
    K = synth.normal_f16(rng, (B, n, hkv, d), mult)
    V = synth.normal_f16(rng, (B, n, hkv, d))
    shift = (rng.standard_normal((B, n, hkv, 1)) * v_shift).astype(np.float32)
    V = (V.view(np.float16).astype(np.float32) + shift).astype(np.float16).view(np.uint16)
    return K, V


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tier", [0, 1, 2])
def test_write_bytes(tier, d):
    banner(f"write tier {tier} D {d}")
    L = LayerPair(8, 2, d, 2, 8, [[tier] * 6] * 2, seed=tier, asymmetric=True)
    rng = np.random.default_rng(10 * tier + d)
    K, V = kv_inputs(rng, 2, 90, 2, d)
    checks = (0, 1, 15, 16, 17, 40, 63, 64, 65)
    for p in range(66):
        L.write(K[:, p:p + 1], V[:, p:p + 1])
        if p in checks:
            bad, ring_ok = L.compare_bytes()
            assert not bad and ring_ok, (p, bad[:3])
    L.write(K[:, 66:90], V[:, 66:90])                # a chunk over a page boundary
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_attention_tiny(tier):
    banner(f"tiny tier {tier}")
    N = 512
    pages = synth.pages_for(N)
    L = LayerPair(8, 2, 64, 1, pages + 2, [[tier] * pages], seed=tier, asymmetric=True)
    rng = np.random.default_rng(tier)
    K, V = kv_inputs(rng, 1, N, 2, 64)
    p = 0
    for n in (100, 16, 200, 195, 1):
        L.write(K[:, p:p + n], V[:, p:p + n])
        p += n
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.normal_f16(rng, (1, 8, 64))
    ref = L.oracle_attn(q)
    for pps in (0, 16, 4):
        got, ws = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max())
        assert L.tickets_zero(ws)


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_attention_14b_shape(tier):
    """40 query heads over 8 KV heads, D 128, a 3000-token context in one prefill chunk"""
    banner(f"14B shape tier {tier}")
    N = 3000
    pages = synth.pages_for(N)
    L = LayerPair(40, 8, 128, 1, pages + 2, [[tier] * pages], seed=tier, asymmetric=True)
    rng = np.random.default_rng(100 + tier)
    K, V = kv_inputs(rng, 1, N, 8, 128, outlier_every=97)
    L.write(K[:, :N - 1], V[:, :N - 1])
    L.write(K[:, N - 1:], V[:, N - 1:])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.normal_f16(rng, (1, 40, 128))
    ref = L.oracle_attn(q)
    for pps in (0, 16):
        got, ws = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max())
        assert L.tickets_zero(ws)


@pytest.mark.parametrize("d", [128, 64])
def test_attention_wide_group_mixed_widths_and_fp16(d):
    """a 16-head group (the two-page-per-tile layout does not apply), pages striped over INT8,
    INT2, FP16 and INT4, two sequences of different lengths"""
    banner(f"group 16, striped widths, D {d}")
    widths = [2, 0, 3, 1, 0, 2, 1, 3, 0, 1, 2, 0]
    L = LayerPair(32, 2, d, 2, 14, [widths, widths[::-1]], seed=5, asymmetric=True)
    rng = np.random.default_rng(5)
    K, V = kv_inputs(rng, 2, 190, 2, d)
    L.write(K[:, :150], V[:, :150])
    L.write(K[:1, 150:190], V[:1, 150:190], rows=[0])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.normal_f16(rng, (2, 32, d))
    ref = L.oracle_attn(q)
    for pps in (0, 2, 4):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max())


def test_attention_half_group_mixed_widths():
    """groups of at most 8 heads, pages of every width in one chunk (the general loop)"""
    banner("group 5, mixed widths, ragged batch")
    rows = [[0, 1, 2, 3, 2, 1, 0, 0, 1, 2], [2, 2, 1, 1, 0, 0, 3, 3, 2, 1], [1] * 10]
    L = LayerPair(10, 2, 128, 3, 12, rows, seed=9, asymmetric=True)
    rng = np.random.default_rng(9)
    K, V = kv_inputs(rng, 3, 160, 2, 128)
    L.write(K[:, :100], V[:, :100])
    L.write(K[1:2, 100:160], V[1:2, 100:160], rows=[1])
    L.write(K[2:3, 100:117], V[2:3, 100:117], rows=[2])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.normal_f16(rng, (3, 10, 128))
    ref = L.oracle_attn(q)
    for pps in (0, 2, 6):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max())


@pytest.mark.parametrize("n_new", [1, 17])
def test_fused_step_equals_write_then_attention(n_new):
    banner(f"fused step, {n_new} new tokens")
    N0 = 700
    pages = synth.pages_for(N0 + n_new)
    rows = [[1] * pages, [0] * pages]

    def build():
        L = LayerPair(40, 8, 128, 2, pages + 2, rows, seed=3, asymmetric=True)
        rng = np.random.default_rng(3)
        K, V = kv_inputs(rng, 2, N0 + n_new, 8, 128)
        L.write(K[:, :N0], V[:, :N0])
        return L, K, V, rng

    A, K, V, rng = build()
    q = synth.normal_f16(rng, (2, 40, 128))
    rows_fused, ws = A.step(K[:, N0:], V[:, N0:], q)
    assert A.tickets_zero(ws)
    bad, ring_ok = A.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    B, _, _, _ = build()
    B.write(K[:, N0:], V[:, N0:])
    rows_sep, _ = B.attn(q)
    assert np.array_equal(rows_fused, rows_sep)
    ref = A.oracle_attn(q)
    err = rowwise_rel_err(rows_fused, ref)
    print(f"  max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL
    # the allocation-free entry point on a third copy: the same rows and bytes
    C, _, _, _ = build()
    pos = C.len.copy()
    out = torch.empty((2, 40, 128), dtype=torch.float32, device=DEV)
    kvq.kv_decode_step_noalloc(C.g, C.pools, C.bt_dev, to_dev_i32(pos), 2, n_new,
                               to_dev_f16(K[:, N0:]), to_dev_f16(V[:, N0:]), C.ring,
                               int((pos + n_new).max()), to_dev_f16(q),
                               float(np.float32(1 / math.sqrt(128))), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), rows_fused)


def test_canary_uses_the_cache_quantizer():
    """on a geometry in the asymmetric format the canary builds asymmetric copies: kv_canary_kl
    equals kv_canary_kl_asym bit for bit and the oracle's asymmetric canary within 1e-4, and the
    one-launch firing over several layers equals the single-layer calls"""
    banner("canary follows the format")
    L = LayerPair(10, 2, 128, 3, 12, [[1] * 10] * 3, seed=11, asymmetric=True)
    rng = np.random.default_rng(11)
    K, V = kv_inputs(rng, 3, 150, 2, 128)
    for s, n in enumerate((150, 40, 97)):
        L.write(K[s:s + 1, :n], V[s:s + 1, :n], rows=[s])
    q = synth.normal_f16(rng, (3, 10, 128))
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    assert np.abs(kl - okl).max() <= 1e-4 and np.abs(rows - orows).max() <= 1e-4
    scale = float(np.float32(1 / math.sqrt(128)))
    wsb = kvq.kv_canary_workspace_bytes(L.g, 3)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    ka = torch.zeros(3, dtype=torch.float32, device=DEV)
    ra = torch.zeros((3, 10, 3), dtype=torch.float32, device=DEV)
    seq = to_dev_i32(L.len)
    kvq.kv_canary_kl_asym(L.g, L.ring, seq, 3, to_dev_f16(q), scale, ka, ra, ws, wsb)
    torch.cuda.synchronize()
    assert np.array_equal(ka.cpu().numpy().astype(np.float64), kl)
    assert np.array_equal(ra.cpu().numpy().astype(np.float64), rows)
    # the symmetric copies differ (the format matters)
    sk, _ = oracle.canary_kl(L.og, L.oring, L.len, q, np.float32(scale), asymmetric=False)
    assert np.abs(sk - okl).max() > 1e-6
    # one launch for two layers (the same ring and queries twice) equals the single calls
    g2 = kvq.geometry(2, 10, 2, 128, 3, 12, asymmetric=True)
    lwsb = kvq.kv_canary_layers_workspace_bytes(g2, 2, 3)
    lws = torch.zeros(lwsb, dtype=torch.uint8, device=DEV)
    kl2 = torch.zeros((2, 3), dtype=torch.float32, device=DEV)
    qd = to_dev_f16(q)
    kvq.kv_canary_kl_layers(g2, [L.ring, L.ring], seq, 3, [qd, qd], scale, kl2, None, lws, lwsb)
    torch.cuda.synchronize()
    assert np.array_equal(kl2.cpu().numpy().astype(np.float64), np.stack([kl, kl]))
