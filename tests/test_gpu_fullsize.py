"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

For each full-size workload the test takes one layer of every bit-width the workload draws, builds
the whole cache of that layer at full context on both sides (prefill of N - 1 tokens), writes the
decode token and attends with the launch the benchmark times (kv_decode_step at the fused step's
split plan), and compares every written block and the ring bit-exactly, every attention row
against the oracle's fp64 rows, the fused launch against the two separate calls bit for bit, the
rows of the library's other split plans, and the canary. The batched workload also
switches the layer's tier mid-run and writes 64 tokens per sequence per step.
"""
import numpy as np
import pytest
import torch

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3
KL_TOL = 1e-4


def first_layer_of_each_width(name):
    w = synth.WORKLOADS[name]
    seen = {}
    for l, b in enumerate(synth.layer_bits(w)):
        seen.setdefault(b, l)
    return [(name, l, b) for b, l in sorted(seen.items())]


CASES = (first_layer_of_each_width("llama8b_8k") + first_layer_of_each_width("qwen14b_32k")
         + first_layer_of_each_width("llama70b_128k"))


def check_attention_and_canary(L, q):
    ref = L.oracle_attn(q)
    plans = [0]                                         # 0: the library's plan from the longest length
    pps_for = kvq.kv_decode_pages_per_split_for(L.g, L.len)
    if pps_for != kvq.kv_decode_pages_per_split(L.g, L.batch, int(L.len.max())):
        plans.append(pps_for)                           # the plan for the lengths (ragged batches)
    for pps in plans:
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attention rows {err.size} (pages per split {pps}): max rel err {err.max():.3e}",
              flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max(), np.unravel_index(np.argmax(err), err.shape))
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    print(f"  canary {kl} vs {okl}; max row err {np.abs(rows - orows).max():.3e}", flush=True)
    assert np.abs(kl - okl).max() <= KL_TOL
    assert np.abs(rows - orows).max() <= KL_TOL


@pytest.mark.parametrize("name,layer,bits", CASES, ids=[f"{n}-L{l}-int{b}" for n, l, b in CASES])
def test_full_context_layer(name, layer, bits):
    full_context_layer(name, layer, bits, asymmetric=False)


ASYM_CASES = first_layer_of_each_width("qwen14b_32k")


@pytest.mark.parametrize("name,layer,bits", ASYM_CASES, ids=[f"{n}-L{l}-int{b}" for n, l, b in ASYM_CASES])
def test_full_context_layer_asymmetric(name, layer, bits):
    """the same at 32K with the asymmetric cache format (zero point and scale per group)"""
    full_context_layer(name, layer, bits, asymmetric=True)


def full_context_layer(name, layer, bits, asymmetric):
    w = synth.WORKLOADS[name]
    N = w.context
    B = w.batch
    print(f"\n[case] {name} layer {layer} INT{bits}{' asymmetric' if asymmetric else ''}: "
          f"batch {B}, context {N}", flush=True)
    pages = synth.pages_for(N)
    tier = synth.TIER_OF_BITS[bits]
    L = LayerPair(w.num_q_heads, w.num_kv_heads, w.head_dim, B, pages + 1, [[tier] * pages] * B,
                  seed=w.config_id * 100 + layer, asymmetric=asymmetric)
    K, V = synth.keys_values(w, layer, N, synth.S_PREFILL_K, synth.S_PREFILL_V)
    L.write(K[:, :N - 1], V[:, :N - 1])                 # prefill in one call per layer
    k1, v1 = K[:, N - 1:].copy(), V[:, N - 1:].copy()
    del K, V
    q = synth.queries(w, layer)
    # The decode step's own token through the launch the benchmark times: kv_decode_step at the
    # fused step's plan (write, then attention over N tokens, in one launch).
    pre_pools = [t.clone() for t in L.pools_t]
    pre_ring = L.ring.clone()
    pps = kvq.kv_decode_step_pages_per_split_for(L.g, L.len, 1)
    got, ws = L.step(k1, v1, q, pages_per_split=pps)
    bad, ring_ok = L.compare_bytes()
    print(f"  fused step (pages per split {pps}): blocks compared {len(L.used_blocks())}, "
          f"mismatching {len(bad)}", flush=True)
    assert not bad, bad[:5]
    assert ring_ok
    assert L.tickets_zero(ws)
    err = rowwise_rel_err(got, L.oracle_attn(q))
    print(f"  fused step attention rows {err.size}: max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL, (err.max(), np.unravel_index(np.argmax(err), err.shape))
    # the same step as two launches from the same state: identical bytes, ring and rows
    fused_pools = [t.clone() for t in L.pools_t]
    fused_ring = L.ring.clone()
    for t, p in zip(L.pools_t, pre_pools):
        t.copy_(p)
    L.ring.copy_(pre_ring)
    del pre_pools, pre_ring
    pos = to_dev_i32(L.len - 1)
    kvq.kv_quant_write(L.g, L.pools, L.bt_dev, pos, B, 1, to_dev_f16(k1), to_dev_f16(v1), L.ring)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(L.pools_t, fused_pools))
    assert torch.equal(L.ring, fused_ring)
    del fused_pools, fused_ring
    sep, _ = L.attn(q, pages_per_split=pps)
    assert np.array_equal(sep, got), "fused step differs from the two separate calls"
    check_attention_and_canary(L, q)


def switching_layer(w):
    """first layer whose tier changes at the mid-run redraw"""
    before, after = synth.layer_bits(w), synth.layer_bits(w, redraw=1)
    for l, (a, b) in enumerate(zip(before, after)):
        if a != b:
            return l, a, b
    raise AssertionError("no layer switches tier")


def test_batched_ragged_tier_switch():
    """64 sequences, lengths log-uniform in [1024, 32768], shuffled blocks; 64 new tokens per
    sequence per step; the layer's tier is redrawn between the two steps: pages opened after the
    switch come from the new pool, blocks written before it stay byte-identical"""
    w = synth.WORKLOADS["qwen7b_batched"]
    layer, b0, b1 = switching_layer(w)
    batched_layer(w, layer, b0, b1)


def batched_layer(w, layer, b0, b1):
    """the two steps of the batched workload on one layer whose width is b0 before the mid-run
    redraw and b1 after it (b0 == b1: no switch)"""
    t0, t1 = synth.TIER_OF_BITS[b0], synth.TIER_OF_BITS[b1]
    lens = synth.seq_lengths(w)                         # tokens at the first step's attention
    B, nn = w.batch, w.new_tokens
    print(f"\n[case] qwen7b_batched layer {layer}: INT{b0} -> INT{b1}, sum N {int(lens.sum())}",
          flush=True)
    final = lens + nn                                   # after the second step
    page_tiers = []
    for s in range(B):
        open_pages = synth.pages_for(int(lens[s]))      # allocated before the switch
        page_tiers.append([t0] * open_pages + [t1] * (synth.pages_for(int(final[s])) - open_pages))
    max_pages = max(len(p) for p in page_tiers) + 1
    L = LayerPair(w.num_q_heads, w.num_kv_heads, w.head_dim, B, max_pages, page_tiers,
                  seed=w.config_id * 100 + layer)
    KV = []
    for s in range(B):                                  # prefill N_s - 64 tokens per sequence
        k, v = synth.sequence_keys_values(w, layer, s, int(final[s]))
        KV.append((k, v))
        n = int(lens[s]) - nn
        L.write(k[:, :n], v[:, :n], rows=[s])
    print("  prefill written", flush=True)

    def step_tokens(first):                             # [B][64] new tokens from position first[s]
        ks = np.concatenate([KV[s][0][:, int(first[s]):int(first[s]) + nn] for s in range(B)])
        vs = np.concatenate([KV[s][1][:, int(first[s]):int(first[s]) + nn] for s in range(B)])
        return ks, vs

    # step 1: 64 new tokens for every sequence in one call, then attention at N_s
    L.write(*step_tokens(lens - nn))
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:5]
    check_attention_and_canary(L, synth.queries(w, layer, step=1))
    before = L.used_blocks()
    snap = [t.cpu().numpy().copy() for t in L.pools_t]
    # tier switch, step 2: 64 more tokens; new pages come from the new pool
    L.write(*step_tokens(lens))
    del KV
    bad, ring_ok = L.compare_bytes()
    print(f"  after the switch: blocks {len(L.used_blocks())}, mismatching {len(bad)}", flush=True)
    assert not bad and ring_ok, bad[:5]
    closed = [(s, p, t, i) for (s, p, t, i) in before if (p + 1) * 16 <= int(lens[s])]
    now = [t.cpu().numpy() for t in L.pools_t]
    nbytes = {t: kvq.kv_block_bytes(L.g, kvq.TIER_BITS[t]) for t in range(3)}
    for (s, p, t, i) in closed:                         # full pages written before the switch
        nb = nbytes[t]
        assert np.array_equal(snap[t][i * nb:(i + 1) * nb], now[t][i * nb:(i + 1) * nb]), (s, p)
    new_pages = [(s, p, t) for (s, p, t, i) in L.used_blocks()
                 if p >= synth.pages_for(int(lens[s]))]
    assert new_pages and all(t == t1 for (_, _, t) in new_pages)
    check_attention_and_canary(L, synth.queries(w, layer, step=2))
