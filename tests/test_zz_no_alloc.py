"""kv_decode_step_noalloc -- the fused decode step with its workspace in the library's fixed
device array -- against kv_decode_step with a caller workspace: the same pool bytes, ring and
attention rows bit for bit, on two calls in a row (the second smaller, on another geometry),
and rows within the attention bar of the oracle."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

ATTN_TOL = 2e-3


def twin_layers(hq, hkv, d, lens, max_pages, seed):
    g = np.random.default_rng(seed)
    tiers = [list(g.integers(0, 3, size=max_pages)) for _ in lens]
    A = LayerPair(hq, hkv, d, len(lens), max_pages, tiers, seed=seed)
    B = LayerPair(hq, hkv, d, len(lens), max_pages, tiers, seed=seed)
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, hkv, d))
        V = synth.normal_f16(g, (1, n, hkv, d))
        A.write(K, V, rows=[s])
        B.write(K, V, rows=[s])
    return A, B, g


def noalloc_step(L, k_new, v_new, q, pps):
    n = k_new.shape[1]
    pos = L.len.copy()
    max_ctx = int((pos + n).max())
    scale = float(np.float32(1.0 / math.sqrt(L.d)))
    out = torch.empty((L.batch, L.hq, L.d), dtype=torch.float32, device="cuda")
    kvq.kv_decode_step_noalloc(L.g, L.pools, L.bt_dev, to_dev_i32(pos), L.batch, n,
                               to_dev_f16(k_new), to_dev_f16(v_new), L.ring, max_ctx,
                               to_dev_f16(q), scale, out, pps)
    torch.cuda.synchronize()
    import oracle
    oracle.quant_write(L.og, L.opools, L.bt, pos, k_new, v_new, L.oring)
    L.len += n
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.gpu
def test_noalloc_step_equals_workspace_step_twice():
    # first call: the 14B shape's heads, three ragged sequences, 3 new tokens, the library's plan;
    # second call: a smaller input on another geometry (tiny heads, one sequence, one token)
    cases = [(40, 8, 128, [3000, 1500, 777], 3, 0, 11), (8, 2, 64, [100], 1, 4, 12)]
    for hq, hkv, d, lens, nn, pps, seed in cases:
        print(f"\n[case] noalloc step: heads {hq}/{hkv}, D {d}, lengths {lens}, {nn} new", flush=True)
        max_pages = max(lens) // 16 + 3
        A, B, g = twin_layers(hq, hkv, d, lens, max_pages, seed)
        k_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        v_new = synth.normal_f16(g, (len(lens), nn, hkv, d))
        q = synth.normal_f16(g, (len(lens), hq, d))
        ref, ws = A.step(k_new, v_new, q, pages_per_split=pps)
        got = noalloc_step(B, k_new, v_new, q, pps)
        assert np.array_equal(got, ref), "rows differ from kv_decode_step"
        for a, b in zip(A.pools_t, B.pools_t):
            assert torch.equal(a, b), "pool bytes differ"
        assert torch.equal(A.ring, B.ring)
        bad, ring_ok = B.compare_bytes()
        assert not bad and ring_ok, bad[:5]
        err = rowwise_rel_err(got, B.oracle_attn(q))
        print(f"  max rel err vs oracle {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL


def test_noalloc_step_rejects_oversized_calls():
    """sizes beyond the static array are rejected on the host, before anything is launched"""
    pools = kvq.layer_pools([256, 256, 256], [1, 1, 1])
    g = kvq.geometry(1, 8, 8, 128, 1024, 64)           # 1024 sequences x 8 KV heads > 4096 groups
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_decode_step_noalloc(g, pools, 256, 256, 1024, 1, 256, 256, 256, 100, 256, 0.1, 256,
                                   0, stream=0)
    assert e.value.status == kvq.KV_EINVAL and "groups" in str(e.value)
    # 2048 groups x 256 splits x 16 heads x 128 channels of partials: far beyond 15 MiB
    g = kvq.geometry(1, 128, 8, 128, 256, 8192)
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_decode_step_noalloc(g, pools, 256, 256, 256, 1, 256, 256, 256, 8192 * 16, 256, 0.1,
                                   256, 64, stream=0)
    assert e.value.status == kvq.KV_EINVAL and "partials" in str(e.value)
