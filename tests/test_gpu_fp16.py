"""The FP16 tier on the GPU (EchoKV, "How EchoKV works": a layer starts at FP16 until the canary
first fires; the pages written then stay FP16): bytes bit-exact against the oracle, attention
against the oracle's fp64 attention (per row, 2e-3 like the INT tiers; the FP16 path itself is
far closer), over all-FP16 layers (the width-specialised loop), layers striped FP16 -> INT and
pages of all four widths mixed (the general loop), token-by-token writes, and the fused step."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3
F16 = 3


def fill(L, lens, g):
    for s, n in enumerate(lens):
        if n:
            K = synth.normal_f16(g, (1, n, L.hkv, L.d))
            V = synth.normal_f16(g, (1, n, L.hkv, L.d))
            L.write(K, V, rows=[s])


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (40, 8, 128), (64, 8, 128), (32, 2, 128),
                                      (16, 1, 64)])
def test_fp16_layer(hq, hkv, d):
    print(f"\n[case] fp16 layer hq={hq} hkv={hkv} d={d}", flush=True)
    lens = [0, 1, 15, 16, 17, 300, 1000, 777]
    g = np.random.default_rng(hq + d)
    L = LayerPair(hq, hkv, d, len(lens), 64, [[F16] * 64 for _ in lens], seed=hq)
    fill(L, lens, g)
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    q = synth.normal_f16(g, (len(lens), hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 2, 16):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL
    assert not got[0].any()


@pytest.mark.parametrize("layout", ["striped_to_int4", "striped_to_int2", "all_widths"])
def test_fp16_mixed_with_int(layout):
    print(f"\n[case] fp16 mixed {layout}", flush=True)
    hq, hkv, d = 40, 8, 128
    lens = [1, 17, 33, 300, 1000, 777]
    g = np.random.default_rng(7)
    if layout == "striped_to_int4":
        tiers = [[F16] * 5 + [1] * 59 for _ in lens]
    elif layout == "striped_to_int2":
        tiers = [[F16] * 3 + [0] * 61 for _ in lens]
    else:
        tiers = [list(g.integers(0, 4, size=64)) for _ in lens]
    L = LayerPair(hq, hkv, d, len(lens), 64, tiers, seed=9)
    fill(L, lens, g)
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    q = synth.normal_f16(g, (len(lens), hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 2, 16):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL


def test_fp16_token_by_token():
    print("\n[case] fp16 token by token", flush=True)
    L = LayerPair(8, 2, 64, 2, 8, [[F16] * 6] * 2, seed=11)
    g = np.random.default_rng(11)
    K = synth.normal_f16(g, (2, 90, 2, 64))
    V = synth.normal_f16(g, (2, 90, 2, 64))
    for p in range(90):
        L.write(K[:, p:p + 1], V[:, p:p + 1])
        if p in (0, 1, 3, 4, 15, 16, 17, 63, 64, 89):
            bad, ring_ok = L.compare_bytes()
            assert not bad and ring_ok, (p, bad[:3])
    q = synth.normal_f16(g, (2, 8, 64))
    got, _ = L.attn(q)
    assert rowwise_rel_err(got, L.oracle_attn(q)).max() <= ATTN_TOL


def test_fp16_fused_step_equals_separate():
    print("\n[case] fp16 fused step", flush=True)
    hq, hkv, d = 40, 8, 128
    lens = [1, 15, 16, 31, 300]
    g = np.random.default_rng(13)
    tiers = [[F16] * 3 + [1, F16, 2] + [F16] * 20 for _ in lens]
    A = LayerPair(hq, hkv, d, len(lens), 26, tiers, seed=13)
    B = LayerPair(hq, hkv, d, len(lens), 26, tiers, seed=13)
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, hkv, d))
        V = synth.normal_f16(g, (1, n, hkv, d))
        A.write(K, V, rows=[s])
        B.write(K, V, rows=[s])
    scale = float(np.float32(1.0 / math.sqrt(d)))
    for step, nn in enumerate([1, 3, 16, 64, 1]):       # 64: five pages, three rounds
        k_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        v_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        q = synth.normal_f16(g, (len(lens), hq, d))
        A.write(k_new, v_new)
        ref, _ = A.attn(q, pages_per_split=2)
        pos = B.len.copy()
        max_ctx = int((pos + nn).max())
        wsb = kvq.kv_decode_workspace_bytes(B.g, B.batch, max_ctx, 2)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        out = torch.empty((B.batch, hq, d), dtype=torch.float32, device="cuda")
        kvq.kv_decode_step(B.g, B.pools, B.bt_dev, to_dev_i32(pos), B.batch, nn, to_dev_f16(k_new),
                           to_dev_f16(v_new), B.ring, max_ctx, to_dev_f16(q), scale, out, ws, wsb, 2)
        torch.cuda.synchronize()
        import oracle
        oracle.quant_write(B.og, B.opools, B.bt, pos, k_new, v_new, B.oring)
        B.len += nn
        got = out.cpu().numpy().astype(np.float64)
        for a, b in zip(A.pools_t, B.pools_t):
            assert torch.equal(a, b), f"step {step}: pool bytes differ"
        assert torch.equal(A.ring, B.ring)
        assert np.array_equal(got, ref), f"step {step}"
    bad, ring_ok = B.compare_bytes()
    assert not bad and ring_ok
    err = rowwise_rel_err(got, B.oracle_attn(q))
    print(f"  fused vs oracle: max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL
