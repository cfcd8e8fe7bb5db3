"""Host-side checks of bench.py (no GPU): the algorithmic byte counts behind the roofline figure
agree with the storage format's own block sizes, and a run asking for more than one GPU stops
with a message before touching a device."""
import importlib.util
import os
import subprocess
import sys

import pytest

import mixed_precision_quantized_kv_amd as kvq
from mixed_precision_quantized_kv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("workload", ["qwen14b_32k", "llama70b_128k", "llama8b_8k"])
@pytest.mark.parametrize("asym", [False, True])
def test_attention_bytes_of_whole_pages_are_the_blocks_read(bench, workload, asym):
    """for a context of whole pages the attention's algorithmic bytes are exactly the pages'
    blocks (every KV head's section) plus one 4-byte block-table entry a page"""
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    w = synth.WORKLOADS[workload]
    g = kvq.geometry(1, w.num_q_heads, w.num_kv_heads, w.head_dim, 1, 16, asymmetric=asym)
    for bits in (2, 4, 8):
        for pages in (1, 7, 2048):
            assert bench.attn_bytes(w, 16 * pages, bits, asym) == \
                pages * (kvq.kv_block_bytes(g, bits) + 4), (bits, pages)


def test_write_bytes_of_one_token(bench):
    """one token written at the start of a page: its key and value in, the page's codes and
    scales out (one token present), its V codes and scale out, its key into the ring"""
    w = synth.WORKLOADS["qwen14b_32k"]
    D, H = w.head_dim, w.num_kv_heads
    for bits in (2, 4, 8):
        expect = H * (D * 2 + D * 2 + (16 * D * bits // 8 + 2 * D) + (D * bits // 8 + 2) + D * 2)
        assert bench.write_bytes(w, 32, 1, bits) == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stdout
