"""The fused decode step (kv_decode_step: the write of the step's tokens and the attention over
them in one launch) against the two separate calls, bit for bit: the same pool bytes, the same
ring, the same attention rows; and against the oracle."""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3


def make_pair(hq, hkv, d, lens, tiers, max_pages, seed):
    """two identical layers (same block table, same prefill)"""
    g = np.random.default_rng(seed)
    A = LayerPair(hq, hkv, d, len(lens), max_pages, tiers, seed=seed)
    B = LayerPair(hq, hkv, d, len(lens), max_pages, tiers, seed=seed)
    for s, n in enumerate(lens):
        if n:
            K = synth.normal_f16(g, (1, n, hkv, d))
            V = synth.normal_f16(g, (1, n, hkv, d))
            A.write(K, V, rows=[s])
            B.write(K, V, rows=[s])
    return A, B, g


@pytest.mark.parametrize("case", ["tiny_token_by_token", "ragged_mixed_n3", "ragged_mixed_n16",
                                  "ragged_mixed_n64", "split_boundary", "library_plan"])
def test_fused_equals_separate(case):
    print(f"\n[case] fused {case}", flush=True)
    if case == "tiny_token_by_token":
        hq, hkv, d, lens, pps, nn, steps = 8, 2, 64, [37], 2, 1, 20
        tiers = [[1] * 8]
        max_pages = 8
    elif case.startswith("ragged"):
        hq, hkv, d, lens, pps, steps = 32, 8, 128, [0, 1, 15, 16, 17, 300, 1000, 777], 16, 3
        nn = int(case.split("_n")[1])       # 64: up to five touched pages, in three rounds
        gt = np.random.default_rng(11)
        max_pages = 80 if nn > 16 else 70
        tiers = [list(gt.integers(0, 3, size=max_pages)) for _ in lens]
    elif case == "split_boundary":          # the two touched pages fall in different splits
        hq, hkv, d, lens, pps, nn, steps = 40, 8, 128, [16 * 5 + 10], 2, 10, 1
        tiers = [[0, 1, 2, 0, 1, 2, 0, 1, 2]]
        max_pages = 9
    else:                   # pages_per_split = 0: the library's fused-step plan (shorter last split)
        hq, hkv, d, lens, pps, nn, steps = 32, 8, 128, [600] * 8, 0, 1, 2
        gt = np.random.default_rng(12)
        tiers = [list(gt.integers(0, 3, size=45)) for _ in lens]
        max_pages = 45
    A, B, g = make_pair(hq, hkv, d, lens, tiers, max_pages, seed=5)
    for step in range(steps):
        k_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        v_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        q = synth.normal_f16(g, (len(lens), hq, d))
        sep_pps = pps
        if pps == 0:        # the separate attention at the plan the fused step makes for itself
            sep_pps = kvq.kv_decode_step_pages_per_split_for(B.g, B.len, nn)
            assert sep_pps != kvq.kv_decode_pages_per_split_for(B.g, B.len + nn)
        A.write(k_new, v_new)
        ref_sep, _ = A.attn(q, pages_per_split=sep_pps)
        got, ws = B.step(k_new, v_new, q, pps)   # B side: one kv_decode_step
        torch.cuda.synchronize()
        for a, b in zip(A.pools_t, B.pools_t):
            assert torch.equal(a, b), f"step {step}: pool bytes differ"
        assert torch.equal(A.ring, B.ring), f"step {step}: ring differs"
        assert np.array_equal(got, ref_sep), f"step {step}: attention differs"
        assert B.tickets_zero(ws)
    bad, ring_ok = B.compare_bytes()
    assert not bad and ring_ok, bad[:5]
    err = rowwise_rel_err(got, B.oracle_attn(q))
    print(f"  fused vs oracle: max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL


def test_fused_rejects_too_many_tokens():
    L = LayerPair(8, 2, 64, 1, 8, [[1] * 8], seed=1)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 8, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, 65, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(kvq.KVError):
        kvq.kv_decode_step(L.g, L.pools, L.bt_dev, to_dev_i32(np.zeros(1, np.int32)), 1, 65, z, z,
                           L.ring, 65, z, 0.1, out, ws, ws.numel(), 0)
