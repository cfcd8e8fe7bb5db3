"""Pins of the oracle's FP16 tier (EchoKV, "How EchoKV works": a layer's cache starts at FP16
before the canary first fires; the tier then stays with the blocks written in it).

  * layout by hand: one token's key and value land at the byte offsets of the FP16 section
    (keys at t*D + c, values at ((t/4)*D + c)*4 + t%4, two bytes each), empty slots stay +0;
  * storage is exact: the dequantized cache is the fp16 input itself;
  * attention over an all-FP16 layer equals torch's float64 scaled_dot_product_attention on the
    fp16 keys and values with the query heads sharing KV heads by repeat_interleave;
  * token-by-token writes equal a one-shot write; a layer striped FP16 -> INT4 reads each page
    at its own width (attention over the concatenation of the two dequantized parts).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mixed_precision_quantized_kv_amd import synth

P, R = 16, 64
F16 = 3


def make(tiers_per_page, n, hq=8, hkv=2, d=64, seed=0, step=None):
    g = oracle.geom(hq, hkv, d)
    rng = np.random.default_rng(seed)
    cap = [8, 8, 8, 8]
    bt = synth.block_table([tiers_per_page], len(tiers_per_page), cap, np.random.default_rng(seed + 1))
    pools = oracle.Pools(g, cap)
    ring = np.zeros((1, R, hkv, d), dtype=np.uint16)
    K = synth.normal_f16(rng, (1, n, hkv, d))
    V = synth.normal_f16(rng, (1, n, hkv, d))
    if step is None:
        oracle.quant_write(g, pools, bt, np.zeros(1, np.int32), K, V, ring)
    else:
        for p0 in range(0, n, step):
            k = min(step, n - p0)
            oracle.quant_write(g, pools, bt, np.array([p0], np.int32), K[:, p0:p0 + k],
                               V[:, p0:p0 + k], ring)
    return g, pools, bt, ring, K, V, rng


def test_layout_by_hand():
    hkv, d = 2, 64
    g, pools, bt, _, K, V, _ = make([F16, F16], 5, hkv=hkv, d=d)
    sec_bytes = 4 * P * d
    assert oracle.section_bytes(g, 16) == sec_bytes
    h = int(bt[0, 0])
    assert h >> 30 == 3
    blk = pools.arrays[3][(h & 0x3FFFFFFF) * hkv * sec_bytes:((h & 0x3FFFFFFF) + 1) * hkv * sec_bytes]
    for kv in range(hkv):
        sec = blk[kv * sec_bytes:(kv + 1) * sec_bytes].view(np.uint16)
        for t in range(P):
            for c in (0, 1, 17, d - 1):
                kval = sec[t * d + c]
                vval = sec[P * d + ((t // 4) * d + c) * 4 + t % 4]
                if t < 5:
                    assert kval == K[0, t, kv, c] and vval == V[0, t, kv, c]
                else:
                    assert kval == 0 and vval == 0


def test_storage_is_exact():
    g, pools, bt, _, K, V, _ = make([F16] * 3, 40)
    for kv in range(2):
        Kd, Vd = oracle.dequant_kv(g, pools, bt[0], 40, kv)
        assert np.array_equal(Kd, K[0, :, kv].view(np.float16).astype(np.float64))
        assert np.array_equal(Vd, V[0, :, kv].view(np.float16).astype(np.float64))


@pytest.mark.parametrize("hq,hkv,d,n", [(8, 2, 64, 45), (40, 8, 128, 33), (16, 1, 64, 16)])
def test_fp16_attention_is_plain_sdpa(hq, hkv, d, n):
    g, pools, bt, _, K, V, rng = make([F16] * ((n + 15) // 16), n, hq=hq, hkv=hkv, d=d)
    q = synth.normal_f16(rng, (1, hq, d))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out = oracle.decode_attn(g, pools, bt, np.array([n], np.int32), q, scale)
    qt = torch.from_numpy(q.view(np.float16).astype(np.float64))[:, :, None, :]   # [1][hq][1][d]
    kt = torch.from_numpy(K.view(np.float16).astype(np.float64)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(V.view(np.float16).astype(np.float64)).permute(0, 2, 1, 3)
    kt = kt.repeat_interleave(hq // hkv, dim=1).contiguous()
    vt = vt.repeat_interleave(hq // hkv, dim=1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, :, 0].numpy()
    assert np.abs(out - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_token_by_token_equals_one_shot():
    a = make([F16] * 3, 37, seed=4)
    b = make([F16] * 3, 37, seed=4, step=1)
    c = make([F16] * 3, 37, seed=4, step=5)
    assert np.array_equal(a[1].arrays[3], b[1].arrays[3])
    assert np.array_equal(a[1].arrays[3], c[1].arrays[3])
    assert np.array_equal(a[3], b[3]) and np.array_equal(a[3], c[3])


def test_striped_fp16_then_int4():
    n = 50
    g, pools, bt, _, K, V, rng = make([F16, F16, 1, 1], n)
    q = synth.normal_f16(rng, (1, 8, 64))
    out = oracle.decode_attn(g, pools, bt, np.array([n], np.int32), q, 0.125)
    for kv in range(2):
        Kd, Vd = oracle.dequant_kv(g, pools, bt[0], n, kv)
        # the first two pages are the inputs themselves; the rest is the INT4 copy
        assert np.array_equal(Kd[:32], K[0, :32, kv].view(np.float16).astype(np.float64))
        assert not np.array_equal(Kd[32:], K[0, 32:, kv].view(np.float16).astype(np.float64))
        for h in range(kv * 4, kv * 4 + 4):
            qd = q[0, h].view(np.float16).astype(np.float64)
            l = 0.125 * Kd @ qd
            w = np.exp(l - l.max())
            assert np.allclose(out[0, h], (w @ Vd) / w.sum(), rtol=0, atol=1e-12)
