"""The whole EchoKV loop on the GPU: decode steps write through the cache, the canary fires every
few steps on every layer, its readings drive the library's controller, and the controller's
widths route the blocks allocated afterwards. The oracle runs the same loop on the CPU with
its own write, canary and controller, fed the same inputs and the same block tables.

Checked: the GPU readings against the oracle's (1e-4 absolute); the library controller's
widths, given the GPU readings, equal the oracle controller's given the same readings (the
width is an integer decided by comparisons, so both take it from identical values); every
written block and ring bit-exact; blocks allocated before a width change keep their bytes;
attention over the resulting striped layers against the oracle (2e-3 per row)."""
import math

import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
import oracle
from oracle import controller as oc
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import f16_bits, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_controller_loop():
    print("\n[case] controller loop: 3 layers, batch 2, canary every 8 steps", flush=True)
    L, HQ, HKV, D, B, MAXP, R = 3, 8, 2, 64, 2, 16, 64
    q_gain = [0.05, 1.0, 6.0]          # per layer: flat, plain and sharp attention
    g = kvq.geometry(L, HQ, HKV, D, B, MAXP, ring_size=R)
    og = oracle.geom(HQ, HKV, D, 16, R)
    cap = np.full((L, 3), B * MAXP, dtype=np.uint32)
    alloc = kvq.KVAlloc(g, cap, [8] * L, shuffle_seed=99)
    pools_t, pools, rings, opools, orings = [], [], [], [], []
    for l in range(L):
        pt = [torch.zeros(int(cap[l, t]) * kvq.kv_block_bytes(g, kvq.TIER_BITS[t]), dtype=torch.uint8,
                          device=DEV) for t in range(cap.shape[1])]
        pools_t.append(pt)
        pools.append(kvq.layer_pools(pt, cap[l]))
        rings.append(torch.zeros((B, R, HKV, D), dtype=torch.float16, device=DEV))
        opools.append(oracle.Pools(og, cap[l]))
        orings.append(np.zeros((B, R, HKV, D), dtype=np.uint16))
    lens = np.zeros(B, dtype=np.int32)
    rng = np.random.default_rng(2024)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    ctrl = kvq.KVController([8] * L)
    octrl = oc.Controller(L, [8] * L)
    snapshots = []                      # (blocks, bytes) taken at each width change

    def write(n):
        pos = lens.copy()
        for s in range(B):
            alloc.kv_alloc_extend(s, int(lens[s]) + n)
        for l in range(L):
            k = synth.normal_f16(rng, (B, n, HKV, D))
            v = synth.normal_f16(rng, (B, n, HKV, D))
            bt = alloc.bt[l]
            kvq.kv_quant_write(g, pools[l], to_dev_i32(bt), to_dev_i32(pos), B, n, to_dev_f16(k),
                               to_dev_f16(v), rings[l])
            oracle.quant_write(og, opools[l], bt, pos, k, v, orings[l])
        lens[:] += n

    write(40)
    firings = 0
    for step in range(64):
        write(1)
        if step % 8 == 7:
            kl_gpu = np.zeros((L, 3), dtype=np.float32)
            for l in range(L):
                q = synth.normal_f16(rng, (B, HQ, D))
                qg = (q.view(np.float16).astype(np.float32) * q_gain[l]).astype(np.float16).view(np.uint16)
                wsb = kvq.kv_canary_workspace_bytes(g, B)
                ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
                kl = torch.zeros(3, dtype=torch.float32, device=DEV)
                kvq.kv_canary_kl(g, rings[l], to_dev_i32(lens), B, to_dev_f16(qg), scale, kl, None,
                                 ws, wsb)
                torch.cuda.synchronize()
                kl_gpu[l] = kl.cpu().numpy()
                ref, _ = oracle.canary_kl(og, orings[l], lens, qg, scale)
                assert np.abs(kl_gpu[l] - ref).max() <= 1e-4, (l, kl_gpu[l], ref)
            ctx = float(lens.mean())
            before = list(octrl.bits)
            got = ctrl.kv_controller_observe(kl_gpu, ctx)
            ref_bits = octrl.observe(kl_gpu.astype(np.float64).tolist(), ctx)
            assert list(got) == ref_bits, (firings, list(got), ref_bits)
            firings += 1
            print(f"  firing {firings}: ctx {ctx:.0f} tau {oc.tau(ctx):.4f} readings "
                  f"{np.array2string(kl_gpu, precision=5)} -> widths {ref_bits}", flush=True)
            if ref_bits != before:
                torch.cuda.synchronize()
                snapshots.append((lens.copy(), [[t.cpu().numpy().copy() for t in pt] for pt in pools_t]))
            ctrl.kv_controller_apply(alloc)
    alloc.kv_check_block_table()
    widths = [ctrl.kv_controller_state()[1][l] for l in range(L)]
    tiers_used = {int(h >> 30) for h in alloc.bt[alloc.bt != kvq.KV_NO_BLOCK].ravel()}
    print(f"  final widths {widths}, tiers in use {sorted(tiers_used)}", flush=True)
    assert len(tiers_used) >= 2, "no width change happened: the loop did not exercise routing"

    # every written block and every ring bit-exact against the oracle
    for l in range(L):
        gp = [t.cpu().numpy() for t in pools_t[l]]
        for s in range(B):
            for p in range((int(lens[s]) + 15) // 16):
                h = int(alloc.bt[l, s, p])
                t, i = h >> 30, h & 0x3FFFFFFF
                nb = oracle.block_bytes(og, kvq.TIER_BITS[t])
                assert np.array_equal(gp[t][i * nb:(i + 1) * nb], opools[l].arrays[t][i * nb:(i + 1) * nb]), (l, s, p)
        assert np.array_equal(f16_bits(rings[l]), orings[l])
    # pages complete when a width changed kept their bytes, whatever the layer's later width
    checked = 0
    for snap_lens, snap in snapshots:
        for l in range(L):
            for s in range(B):
                for p in range(int(snap_lens[s]) // 16):
                    h = int(alloc.bt[l, s, p])
                    t, i = h >> 30, h & 0x3FFFFFFF
                    nb = kvq.kv_block_bytes(g, kvq.TIER_BITS[t])
                    now = pools_t[l][t][i * nb:(i + 1) * nb].cpu().numpy()
                    assert np.array_equal(now, snap[l][t][i * nb:(i + 1) * nb]), (l, s, p)
                    checked += 1
    assert checked > 0
    # attention over the striped layers
    for l in range(L):
        q = synth.normal_f16(rng, (B, HQ, D))
        max_ctx = int(lens.max())
        wsb = kvq.kv_decode_workspace_bytes(g, B, max_ctx, 0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        out = torch.empty((B, HQ, D), dtype=torch.float32, device=DEV)
        kvq.kv_decode_attn(g, pools[l], to_dev_i32(alloc.bt[l]), to_dev_i32(lens), B, max_ctx,
                           to_dev_f16(q), scale, out, ws, wsb, 0)
        torch.cuda.synchronize()
        ref = oracle.decode_attn(og, opools[l], alloc.bt[l], lens, q, scale)
        err = rowwise_rel_err(out.cpu().numpy().astype(np.float64), ref)
        print(f"  layer {l}: attention max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= 2e-3
