"""The three kernels under HIP graph capture: a captured decode step (write, attention, canary)
replayed several times, with eager work and synchronizations between the replays, gives the
eager step's results bit for bit every time (writing the same token again is idempotent, the
split-merge and canary tickets reset themselves)."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu


def step_fn(L, pos, k1, v1, ctx, q, ws, out, kl, rows, cws, pps):
    scale = float(np.float32(1.0 / math.sqrt(L.d)))
    wsb, cwsb = ws.numel(), cws.numel()
    max_ctx = int(ctx.max().item())

    def run(stream):
        kvq.kv_quant_write(L.g, L.pools, L.bt_dev, pos, L.batch, 1, k1, v1, L.ring, stream=stream)
        kvq.kv_decode_attn(L.g, L.pools, L.bt_dev, ctx, L.batch, max_ctx, q, scale, out, ws, wsb,
                           pps, stream=stream)
        kvq.kv_canary_kl(L.g, L.ring, ctx, L.batch, q, scale, kl, rows, cws, cwsb, stream=stream)
    return run


@pytest.mark.parametrize("case", ["tiny_int8", "ragged_mixed", "ragged_mixed_asymmetric"])
def test_graph_replays_match_eager(case):
    print(f"\n[case] graph {case}", flush=True)
    g = np.random.default_rng(7)
    if case == "tiny_int8":
        hq, hkv, d, lens, tiers, pps = 8, 2, 64, [300], [[2] * 20], 0
    else:
        hq, hkv, d, lens, pps = 32, 8, 128, [300, 1000, 777], 16
        tiers = [list(g.integers(0, 3, size=66)) for _ in lens]
    L = LayerPair(hq, hkv, d, len(lens), 66 if case != "tiny_int8" else 20, tiers, seed=3,
                  asymmetric=case.endswith("asymmetric"))
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n - 1, hkv, d))
        V = synth.normal_f16(g, (1, n - 1, hkv, d))
        L.write(K, V, rows=[s])
    B = len(lens)
    pos = to_dev_i32(L.len.copy())
    ctx = to_dev_i32(L.len + 1)
    k1 = to_dev_f16(synth.normal_f16(g, (B, 1, hkv, d)))
    v1 = to_dev_f16(synth.normal_f16(g, (B, 1, hkv, d)))
    q = to_dev_f16(synth.normal_f16(g, (B, hq, d)))
    wsb = kvq.kv_decode_workspace_bytes(L.g, B, int(L.len.max()) + 1, pps)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    cws = torch.zeros(kvq.kv_canary_workspace_bytes(L.g, B), dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, hq, d), dtype=torch.float32, device="cuda")
    kl = torch.zeros(3, dtype=torch.float32, device="cuda")
    rows = torch.zeros((B, hq, 3), dtype=torch.float32, device="cuda")
    run = step_fn(L, pos, k1, v1, ctx, q, ws, out, kl, rows, cws, pps)

    run(torch.cuda.current_stream().cuda_stream)          # eager
    torch.cuda.synchronize()
    ref = [out.clone(), kl.clone(), rows.clone(), L.ring.clone()] + [p.clone() for p in L.pools_t]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        out.zero_(); kl.zero_(); rows.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out, kl, rows, L.ring] + list(L.pools_t)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (out * 2).sum().item()                        # eager work between replays
    assert L.tickets_zero(ws) and not cws[:768].any()    # tickets left at zero


def test_graph_replays_of_the_allocation_free_step():
    """kv_decode_step_noalloc -- the entry point for callers that cannot allocate, such as code
    under graph capture -- captured after one eager call and replayed four times with eager work
    between the replays: every replay gives the eager call's outputs, ring and pools bit for
    bit, and the captured step equals kv_decode_step with a caller workspace"""
    print("\n[case] graph of kv_decode_step_noalloc", flush=True)
    g = np.random.default_rng(8)
    hq, hkv, d, lens = 32, 8, 128, [300, 1000, 777]
    tiers = [list(g.integers(0, 4, size=66)) for _ in lens]
    L = LayerPair(hq, hkv, d, len(lens), 66, tiers, seed=5)
    for s, n in enumerate(lens):
        L.write(synth.normal_f16(g, (1, n - 1, hkv, d)), synth.normal_f16(g, (1, n - 1, hkv, d)),
                rows=[s])
    B = len(lens)
    pos_np = L.len.copy()
    pos = to_dev_i32(pos_np)
    k1_np = synth.normal_f16(g, (B, 1, hkv, d))
    v1_np = synth.normal_f16(g, (B, 1, hkv, d))
    q_np = synth.normal_f16(g, (B, hq, d))
    k1, v1, q = to_dev_f16(k1_np), to_dev_f16(v1_np), to_dev_f16(q_np)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    max_ctx = int(L.len.max()) + 1
    out = torch.zeros((B, hq, d), dtype=torch.float32, device="cuda")

    def run():
        kvq.kv_decode_step_noalloc(L.g, L.pools, L.bt_dev, pos, B, 1, k1, v1, L.ring, max_ctx, q,
                                   scale, out, 0, stream=torch.cuda.current_stream().cuda_stream)

    run()                                                 # eager
    torch.cuda.synchronize()
    ref = [out.clone(), L.ring.clone()] + [p.clone() for p in L.pools_t]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip([out, L.ring] + list(L.pools_t), ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (out * 2).sum().item()                        # eager work between replays
    # the same step through kv_decode_step with a caller workspace, on the same (already
    # written: the write is idempotent) cache
    got, ws = L.step(k1_np, v1_np, q_np)
    assert np.array_equal(got, ref[0].cpu().numpy().astype(np.float64))
    assert L.tickets_zero(ws)
