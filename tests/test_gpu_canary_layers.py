"""One canary firing for every layer in one launch (kv_canary_kl_layers) against the oracle's
canary of each layer and against the single-layer call, bit for bit.

EchoKV, "Show the math": a firing gives one reading per (layer, width), 3L numbers. Each layer
here has its own ring and its own queries; the sequences share their lengths across layers.
"""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
import oracle
from mixed_precision_quantized_kv_amd import synth

pytestmark = pytest.mark.gpu
KL_TOL = 1e-4
DEV = "cuda:0"


def make_layers(L, B, hq, hkv, d, seed):
    g = np.random.default_rng(seed)
    mult = np.where(np.arange(d) % 13 == 5, 10.0, 1.0).astype(np.float32)
    rings = [synth.normal_f16(g, (B, 64, hkv, d), mult) for _ in range(L)]
    qs = [synth.normal_f16(g, (B, hq, d)) for _ in range(L)]
    return rings, qs


@pytest.mark.parametrize("shape", ["qwen14b", "tiny", "gqa7"])
def test_layers_match_oracle_and_single_calls(shape):
    L, B, hq, hkv, d, lens = {
        "qwen14b": (48, 1, 40, 8, 128, [32769]),
        "tiny": (4, 1, 8, 2, 64, [512]),
        "gqa7": (5, 6, 28, 4, 128, [1, 17, 40, 64, 65, 3000]),
    }[shape]
    print(f"\n[case] canary layers {shape}: {L} layers, batch {B}", flush=True)
    rings, qs = make_layers(L, B, hq, hkv, d, seed=L)
    g = kvq.geometry(L, hq, hkv, d, B, 4096)
    og = oracle.geom(hq, hkv, d, 16, 64)
    scale = np.float32(1.0 / math.sqrt(d))
    seq = np.array(lens, dtype=np.int32)
    rings_t = [torch.from_numpy(r.view(np.float16)).to(DEV) for r in rings]
    qs_t = [torch.from_numpy(q.view(np.float16)).to(DEV) for q in qs]
    seq_t = torch.from_numpy(seq).to(DEV)
    wsb = kvq.kv_canary_layers_workspace_bytes(g, L, B)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    kl = torch.zeros((L, 3), dtype=torch.float32, device=DEV)
    rows = torch.zeros((L, B, hq, 3), dtype=torch.float32, device=DEV)
    kvq.kv_canary_kl_layers(g, rings_t, seq_t, B, qs_t, float(scale), kl, rows, ws, wsb)
    torch.cuda.synchronize()
    assert not ws[:L * 3 * 256].any()                          # every ticket back at zero
    kl_h, rows_h = kl.cpu().numpy().astype(np.float64), rows.cpu().numpy().astype(np.float64)
    # the single-layer call on each layer: the same bits
    sws = torch.zeros(kvq.kv_canary_workspace_bytes(g, B), dtype=torch.uint8, device=DEV)
    for l in range(L):
        k1 = torch.zeros(3, dtype=torch.float32, device=DEV)
        r1 = torch.zeros((B, hq, 3), dtype=torch.float32, device=DEV)
        kvq.kv_canary_kl(g, rings_t[l], seq_t, B, qs_t[l], float(scale), k1, r1, sws)
        torch.cuda.synchronize()
        assert torch.equal(k1, kl[l]) and torch.equal(r1, rows[l]), f"layer {l}"
    worst = 0.0
    for l in range(L):
        okl, orows = oracle.canary_kl(og, rings[l], seq, qs[l], scale)
        worst = max(worst, np.abs(kl_h[l] - okl).max(), np.abs(rows_h[l] - orows).max())
        assert np.abs(kl_h[l] - okl).max() <= KL_TOL, (l, kl_h[l], okl)
        assert np.abs(rows_h[l] - orows).max() <= KL_TOL, l
    print(f"  max abs err vs oracle {worst:.3e}", flush=True)


def test_workspace_reused_across_layer_counts_and_batches():
    """one workspace for firings over 6 layers x batch 4, then 2 layers x batch 1, then 6 x 4
    again: each call's readings equal those of a fresh workspace"""
    hq, hkv, d = 8, 2, 64
    g = kvq.geometry(6, hq, hkv, d, 4, 64)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rings, qs = make_layers(6, 4, hq, hkv, d, seed=3)
    rings_t = [torch.from_numpy(r.view(np.float16)).to(DEV) for r in rings]
    qs_t = [torch.from_numpy(q.view(np.float16)).to(DEV) for q in qs]
    seq_t = torch.tensor([100, 7, 64, 300], dtype=torch.int32, device=DEV)
    wsb = kvq.kv_canary_layers_workspace_bytes(g, 6, 4)
    shared = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    for L, B in ((6, 4), (2, 1), (6, 4)):
        outs = []
        for ws in (shared, torch.zeros(wsb, dtype=torch.uint8, device=DEV)):
            kl = torch.zeros((L, 3), dtype=torch.float32, device=DEV)
            kvq.kv_canary_kl_layers(g, rings_t[:L], seq_t, B, qs_t[:L], scale, kl, None, ws, wsb)
            outs.append(kl)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), (L, B)
        assert not shared[:6 * 3 * 256].any()        # the tickets of all six layers
