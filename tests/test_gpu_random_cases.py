"""Randomized GPU parity (hypothesis, derandomized: the same cases in every run).

Each case draws a layer shape the geometry allows (group size 1..16, head size 64 or 128, either
storage format), a batch of ragged lengths (zero included), page widths per page (uniform or
mixed, FP16 pages included), a split plan and a fused step of 0..64 new tokens. The prefill goes
through kv_quant_write in random chunks, the step through kv_decode_step; the oracle does the
same. Bar: pool bytes and ring bit-exact, attention rows within 2e-3 of the oracle, ticket
counters back at zero. A second test draws canaries the same way (KL within 1e-4).
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import mixed_precision_quantized_kv_amd as kvq
import oracle
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3

SHAPES = [(1, 1), (2, 4), (8, 5), (4, 7), (8, 8), (2, 16)]       # (KV heads, group size)


@settings(max_examples=24, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(st.data())
def test_random_layers_against_oracle(data):
    hkv, grp = data.draw(st.sampled_from(SHAPES))
    hq = hkv * grp
    d = data.draw(st.sampled_from([64, 128]))
    asym = data.draw(st.booleans())
    batch = data.draw(st.integers(1, 4))
    lens = data.draw(st.lists(st.integers(0, 500), min_size=batch, max_size=batch))
    n_new = data.draw(st.sampled_from([0, 1, 3, 17, 64]))
    pps = data.draw(st.sampled_from([0, 2, 4, 16]))
    seed = data.draw(st.integers(0, 2**16))
    max_pages = (max(lens) + n_new + 15) // 16 + 1
    if data.draw(st.booleans()):
        tier = data.draw(st.integers(0, 3))
        tiers = [[tier] * max_pages for _ in lens]
    else:
        tiers = [data.draw(st.lists(st.integers(0, 3), min_size=max_pages, max_size=max_pages))
                 for _ in lens]
    print(f"\n[case] hq={hq} hkv={hkv} d={d} asym={asym} lens={lens} n_new={n_new} pps={pps} "
          f"seed={seed} tiers={'uniform ' + str(tiers[0][0]) if len(set(sum(tiers, []))) == 1 else 'mixed'}",
          flush=True)
    g = np.random.default_rng(seed)
    L = LayerPair(hq, hkv, d, batch, max_pages, tiers, seed=seed, asymmetric=asym)
    for s, n in enumerate(lens):                    # prefill in up to three chunks
        cuts = sorted(set(int(c) for c in g.integers(1, max(2, n), size=2))) if n > 2 else []
        bounds = [0] + [c for c in cuts if 0 < c < n] + [n]
        K = synth.normal_f16(g, (1, n, hkv, d))
        V = synth.normal_f16(g, (1, n, hkv, d))
        for a, b in zip(bounds[:-1], bounds[1:]):
            if b > a:
                L.write(K[:, a:b], V[:, a:b], rows=[s])
    k_new = synth.normal_f16(g, (batch, n_new, hkv, d))
    v_new = synth.normal_f16(g, (batch, n_new, hkv, d))
    q = synth.normal_f16(g, (batch, hq, d))
    got, ws = L.step(k_new, v_new, q, pages_per_split=pps)
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    ref = L.oracle_attn(q)
    err = rowwise_rel_err(got, ref)
    print(f"  max row err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL
    assert not got[L.len == 0].any()                # empty sequences give zero rows
    assert L.tickets_zero(ws)


@settings(max_examples=20, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(st.data())
def test_random_canaries_against_oracle(data):
    """the canary over rings of every allowed size, filled below, to and past their size (a
    wrapped ring, a partial oldest page), with the cache's own copies and, on a symmetric cache,
    the forced asymmetric copies; KL within 1e-4 of the oracle on the mean and every row"""
    hkv, grp = data.draw(st.sampled_from(SHAPES))
    hq = hkv * grp
    d = data.draw(st.sampled_from([64, 128]))
    R = data.draw(st.sampled_from([16, 32, 64, 128]))
    asym = data.draw(st.booleans())
    batch = data.draw(st.integers(1, 4))
    lens = data.draw(st.lists(st.integers(1, 3 * R), min_size=batch, max_size=batch))
    outliers = data.draw(st.booleans())
    seed = data.draw(st.integers(0, 2**16))
    print(f"\n[case] canary hq={hq} hkv={hkv} d={d} R={R} asym={asym} lens={lens} outliers={outliers} "
          f"seed={seed}", flush=True)
    g = np.random.default_rng(seed)
    max_pages = max(lens) // 16 + 2
    tiers = [[1] * max_pages for _ in lens]
    L = LayerPair(hq, hkv, d, batch, max_pages, tiers, seed=seed, R=R, asymmetric=asym)
    mult = np.where(np.arange(d) % 9 == 0, 10, 1).astype(np.float32) if outliers else None
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, hkv, d), mult)
        V = synth.normal_f16(g, (1, n, hkv, d))
        half = n // 2
        for a, b in ((0, half), (half, n)):
            if b > a:
                L.write(K[:, a:b], V[:, a:b], rows=[s])
    q = synth.normal_f16(g, (batch, hq, d))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    print(f"  kl {kl} max row err {np.abs(rows - orows).max():.3e}", flush=True)
    assert np.abs(kl - okl).max() <= 1e-4 and np.abs(rows - orows).max() <= 1e-4
    if not asym:                                     # the forced asymmetric copies
        wsb = kvq.kv_canary_workspace_bytes(L.g, batch)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        kla = torch.zeros(3, dtype=torch.float32, device="cuda")
        rowsa = torch.zeros((batch, hq, 3), dtype=torch.float32, device="cuda")
        kvq.kv_canary_kl_asym(L.g, L.ring, to_dev_i32(L.len), batch, to_dev_f16(q), scale, kla, rowsa,
                              ws, wsb)
        torch.cuda.synchronize()
        okla, orowsa = oracle.canary_kl(L.og, L.oring, L.len, q, scale, asymmetric=True)
        assert np.abs(kla.cpu().numpy() - okla).max() <= 1e-4
        assert np.abs(rowsa.cpu().numpy() - orowsa).max() <= 1e-4
