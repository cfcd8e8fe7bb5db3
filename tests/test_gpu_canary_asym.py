"""The canary with KIVI-style asymmetric copies (kv_canary_kl_asym) against the oracle's
asymmetric canary: KL within 1e-4 absolute, on the mean and on every row, over ring fragments
(fewer keys than the ring, a partial oldest page, a ring that has wrapped), GQA shapes, both head
sizes and a full-size 14B-shaped layer; plus an exact grid on which the INT2 copy is exact."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
import oracle
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
KL_TOL = 1e-4


def gpu_canary_asym(L, q_u16, scale):
    wsb = kvq.kv_canary_workspace_bytes(L.g, L.batch)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    kl = torch.zeros(3, dtype=torch.float32, device="cuda")
    rows = torch.zeros((L.batch, L.hq, 3), dtype=torch.float32, device="cuda")
    kvq.kv_canary_kl_asym(L.g, L.ring, to_dev_i32(L.len), L.batch, to_dev_f16(q_u16), scale, kl,
                          rows, ws, wsb)
    torch.cuda.synchronize()
    return kl.cpu().numpy().astype(np.float64), rows.cpu().numpy().astype(np.float64)


CASES = {
    # name: (hq, hkv, d, lengths, ring)
    "tiny_d64": (8, 2, 64, [40, 1, 64, 100], 64),
    "gqa16_d128": (32, 2, 128, [17, 64, 200], 64),
    "qwen14b_shape": (40, 8, 128, [300, 1000], 64),
    "ring128_wrapped": (28, 4, 128, [130, 500, 129], 128),
    "ring16": (8, 1, 64, [5, 16, 33], 16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_asym_canary_matches_oracle(name):
    hq, hkv, d, lens, R = CASES[name]
    print(f"\n[case] asym canary {name}", flush=True)
    g = np.random.default_rng(100 + sorted(CASES).index(name))
    max_pages = max(lens) // 16 + 2
    tiers = [[1] * max_pages for _ in lens]
    L = LayerPair(hq, hkv, d, len(lens), max_pages, tiers, seed=3, R=R)
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, hkv, d))
        V = synth.normal_f16(g, (1, n, hkv, d))
        L.write(K, V, rows=[s])
    q = synth.normal_f16(g, (len(lens), hq, d))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    kl, rows = gpu_canary_asym(L, q, scale)
    okl, orows = oracle.canary_kl(L.og, L.oring, L.len, q, scale, asymmetric=True)
    print(f"  kl {kl} oracle {okl} max row err {np.abs(rows - orows).max():.3e}", flush=True)
    assert np.abs(kl - okl).max() <= KL_TOL
    assert np.abs(rows - orows).max() <= KL_TOL
    assert np.all(rows >= 0)
    # the asymmetric INT2 copy has four levels where the symmetric one has three
    skl, _ = L.canary(q)
    print(f"  symmetric kl {skl}", flush=True)


def test_asym_canary_exact_grid():
    print("\n[case] asym canary exact grid", flush=True)
    hq, hkv, d, N = 8, 2, 64, 48
    L = LayerPair(hq, hkv, d, 1, 4, [[2] * 4], seed=4)
    g = np.random.default_rng(8)
    K = (g.integers(0, 4, size=(1, N, hkv, d)) * 0.25 - 0.5)
    for page in range(0, N, 16):                # every (page, channel) group spans the grid
        K[0, page] = -0.5
        K[0, page + 1] = 0.25
    Kb = K.astype(np.float16).view(np.uint16)
    V = synth.normal_f16(g, (1, N, hkv, d))
    L.write(Kb, V)
    q = synth.normal_f16(g, (1, hq, d))
    kl, rows = gpu_canary_asym(L, q, 0.125)
    okl, _ = oracle.canary_kl(L.og, L.oring, L.len, q, 0.125, asymmetric=True)
    print(f"  kl {kl} oracle {okl}", flush=True)
    assert okl[0] == 0.0 and kl[0] == 0.0
    assert np.abs(kl - okl).max() <= KL_TOL
