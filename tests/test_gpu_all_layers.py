"""GPU parity of every layer of the full-size workloads, in the launch the benchmark times.

For each layer of the 8B shape (32 layers, batch 8 at 8K) and of the 14B shape (48 layers at 32K),
and for layers 0, 1, 39, 40, 78 and 79 of the 70B shape at 128K, the layer's cache is built at full
context on both sides (prefill of N - 1 tokens at the layer's drawn width), the decode token is
written and attended with one kv_decode_step at the fused step's split plan, and every written
block and the ring are compared bit for bit with the oracle and every attention row within 2e-3
(per row: max |err| / max |ref|). The one-layer-per-width cases of test_gpu_fullsize.py add the
two-launch comparison, the other split plans and the canary.
"""
import os

import numpy as np
import pytest

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

from gpu_cases import LayerPair, rowwise_rel_err

pytestmark = pytest.mark.gpu
ATTN_TOL = 2e-3


def layers(name, which=None):
    w = synth.WORKLOADS[name]
    bits = synth.layer_bits(w)
    return [(name, l, bits[l]) for l in (which if which is not None else range(w.num_layers))]


CASES = (layers("llama8b_8k") + layers("qwen14b_32k")
         + layers("llama70b_128k", [0, 1, 39, 40, 78, 79]))


@pytest.mark.parametrize("name,layer,bits", CASES, ids=[f"{n}-L{l}-int{b}" for n, l, b in CASES])
def test_layer_decode_step(name, layer, bits):
    w = synth.WORKLOADS[name]
    N, B = w.context, w.batch
    print(f"\n[case] {name} layer {layer} INT{bits}: batch {B}, context {N}", flush=True)
    pages = synth.pages_for(N)
    tier = synth.TIER_OF_BITS[bits]
    L = LayerPair(w.num_q_heads, w.num_kv_heads, w.head_dim, B, pages + 1, [[tier] * pages] * B,
                  seed=w.config_id * 100 + layer)
    K, V = synth.keys_values(w, layer, N, synth.S_PREFILL_K, synth.S_PREFILL_V)
    L.write(K[:, :N - 1], V[:, :N - 1])
    k1, v1 = K[:, N - 1:].copy(), V[:, N - 1:].copy()
    del K, V
    q = synth.queries(w, layer)
    pps = kvq.kv_decode_step_pages_per_split_for(L.g, L.len, 1)
    got, ws = L.step(k1, v1, q, pages_per_split=pps)
    bad, ring_ok = L.compare_bytes()
    assert not bad, bad[:5]
    assert ring_ok
    assert L.tickets_zero(ws)
    err = rowwise_rel_err(got, L.oracle_attn(q))
    print(f"  blocks {len(L.used_blocks())} bit-exact; rows {err.size}: max rel err {err.max():.3e}",
          flush=True)
    assert err.max() <= ATTN_TOL, (err.max(), np.unravel_index(np.argmax(err), err.shape))


BATCHED = synth.WORKLOADS["qwen7b_batched"]
BATCHED_CASES = list(zip(range(BATCHED.num_layers), synth.layer_bits(BATCHED),
                         synth.layer_bits(BATCHED, redraw=1)))


@pytest.mark.skipif(os.environ.get("KVQ_ALL_LAYERS") != "1",
                    reason="every layer of the batched shape takes ~10 minutes; KVQ_ALL_LAYERS=1 runs it")
@pytest.mark.parametrize("layer,b0,b1", BATCHED_CASES,
                         ids=[f"qwen7b_batched-L{l}-int{a}-int{b}" for l, a, b in BATCHED_CASES])
def test_batched_layer(layer, b0, b1):
    """every layer of the batched 7B shape: 64 ragged sequences, two steps of 64 new tokens with
    the layer's mid-run redraw between them (test_gpu_fullsize.batched_layer)"""
    from test_gpu_fullsize import batched_layer
    batched_layer(BATCHED, layer, b0, b1)
