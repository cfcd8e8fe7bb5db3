"""GPU parity with pools whose unwritten slots hold NaN bit patterns.

A sequence's last page is partly written, and a freshly handed-out block holds whatever its
memory held before. Attention masks the slots past a sequence's length: their codes and scales
must never reach an output, whatever bits they hold. Here every GPU pool starts filled with
0xFF bytes (the fp16 scales of unwritten slots are NaN, their codes all ones) while the oracle's
start at zero; the written bytes are still compared with the oracle wherever tokens were
written, and attention rows (separate write and attention calls, then one fused step) within
2e-3. Lengths end inside pages for every width, with chunks of odd and even page counts, and
the mixed-width loop is covered by a striped sequence.
"""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3


def full_pages_differing(L):
    """the full pages (every byte written on both sides) that differ from the oracle's; a
    partly written page keeps the fill in its unwritten slots on the GPU side, zeros on the
    oracle's"""
    torch.cuda.synchronize()
    bad = []
    for (s, p, t, i) in L.used_blocks():
        if int(L.len[s]) - 16 * p >= 16:
            nb = kvq.kv_block_bytes(L.g, kvq.TIER_BITS[t])
            a = L.pools_t[t][i * nb:(i + 1) * nb].cpu().numpy()
            b = L.opools.arrays[t][i * nb:(i + 1) * nb]
            if not np.array_equal(a, b):
                bad.append((s, p, t, i))
    return bad


@pytest.mark.parametrize("d,hq,hkv", [(128, 40, 8), (64, 8, 2)])
@pytest.mark.parametrize("asym", [False, True])
def test_poisoned_pools(d, hq, hkv, asym):
    print(f"\n[case] poisoned pools D={d} {hq}/{hkv} asymmetric={asym}", flush=True)
    lens = [1000, 517, 33, 700]
    pages = [synth.pages_for(n + 1) for n in lens]
    mp = max(pages) + 1
    tiers = [[0] * mp, [1] * mp, [2] * mp, [(p // 3) % 3 for p in range(mp)]]
    L = LayerPair(hq, hkv, d, len(lens), mp, tiers, seed=7, asymmetric=asym, fill=0xFF)
    g = np.random.default_rng(11)
    scale_k = np.where(np.arange(d) % 13 == 0, 10, 1).astype(np.float32)
    N = max(lens)
    K = synth.normal_f16(g, (len(lens), N + 1, hkv, d), scale_k)
    V = synth.normal_f16(g, (len(lens), N + 1, hkv, d))
    for s, n in enumerate(lens):
        L.write(K[s:s + 1, :n], V[s:s + 1, :n], rows=[s])
    assert not full_pages_differing(L)
    q = synth.normal_f16(g, (len(lens), hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 2, 6, 16, 64):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}", flush=True)
        assert np.isfinite(got).all() and err.max() <= ATTN_TOL, (pps, err.max())
    # one fused step: the new token lands in a partly written page (or opens one)
    k1 = np.stack([K[s, lens[s]:lens[s] + 1] for s in range(len(lens))])
    v1 = np.stack([V[s, lens[s]:lens[s] + 1] for s in range(len(lens))])
    got, ws = L.step(k1, v1, q)
    assert L.tickets_zero(ws)
    err = rowwise_rel_err(got, L.oracle_attn(q))
    print(f"  fused step max rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all() and err.max() <= ATTN_TOL, err.max()
    assert not full_pages_differing(L)
