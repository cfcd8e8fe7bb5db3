"""Seeded synthetic inputs for the five workload shapes.

This module draws numbers and lays out input structure (per-layer tier choices, outlier channels,
sequence lengths, shuffled physical block tables). It holds none of the method's arithmetic: no
quantizer, packing, attention or divergence. Tests feed the same arrays to the GPU library and to
the CPU oracle; the benchmark uses it to build its cache.

The workloads stand in for the pages' evaluation runs (RULER, GSM8K-Hard, tau-Bench, the 14B/32K
decode timing of the behavior-guided thesis): only their shapes are taken -- model geometry,
batch, context -- and the values are standard-normal fp16 with outlier key channels.

Random streams: numpy PCG64 seeded by SeedSequence([0, config_id, layer, stream, step]).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

PAGE = 16
RING = 64
MASTER_SEED = 0

# stream ids
S_PREFILL_K, S_PREFILL_V, S_Q, S_KNEW, S_VNEW, S_OUTLIER, S_TIER, S_LEN, S_SHUFFLE, S_REDRAW = range(10)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    batch: int
    context: int                       # tokens cached at attention time (uniform batches)
    tier_mix: Optional[Dict[int, float]] = None      # per-layer draw; None -> fixed_bits
    fixed_bits: Optional[Sequence[int]] = None
    edge_layers: int = 0               # 70B-shape: first/last layers drawn from edge_mix
    edge_mix: Optional[Dict[int, float]] = None
    outlier_frac: float = 0.0          # fraction of (kv head, channel) key channels scaled
    outlier_scale: float = 1.0
    outlier_channels: Optional[Sequence[int]] = None  # explicit channels of every kv head
    ragged: bool = False               # lengths log-uniform in [len_lo, len_hi]
    len_lo: int = 0
    len_hi: int = 0
    new_tokens: int = 1                # tokens written per sequence per decode step
    page_size: int = PAGE
    ring_size: int = RING

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


MIX_8B = {2: 0.2, 4: 0.6, 8: 0.2}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, 4, 8, 2, 64, 1, 512, fixed_bits=(2, 4, 8, 4),
                     outlier_channels=(3, 17, 40, 59), outlier_scale=10.0),
    "llama8b_8k": Workload("llama8b_8k", 1, 32, 32, 8, 128, 8, 8192, tier_mix=MIX_8B,
                           outlier_frac=0.02, outlier_scale=8.0),
    "qwen14b_32k": Workload("qwen14b_32k", 2, 48, 40, 8, 128, 1, 32768, tier_mix=MIX_8B,
                            outlier_frac=0.01, outlier_scale=10.0),
    "llama70b_128k": Workload("llama70b_128k", 3, 80, 64, 8, 128, 1, 131072,
                              tier_mix={2: 0.4, 4: 0.6}, edge_layers=8,
                              edge_mix={8: 0.8, 4: 0.2}),
    "qwen7b_batched": Workload("qwen7b_batched", 4, 28, 28, 4, 128, 64, 0, tier_mix=MIX_8B,
                               ragged=True, len_lo=1024, len_hi=32768, new_tokens=64),
}


def rng(w: Workload, layer: int, stream: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([MASTER_SEED, w.config_id, layer, stream, step])))


def _draw(mix: Dict[int, float], g: np.random.Generator) -> int:
    keys = sorted(mix)
    return int(g.choice(keys, p=[mix[k] for k in keys]))


def layer_bits(w: Workload, redraw: int = 0) -> List[int]:
    """Per-layer bit-width; redraw > 0 gives the tier vector after a mid-run switch."""
    if w.fixed_bits is not None and redraw == 0:
        return list(w.fixed_bits)
    out = []
    for l in range(w.num_layers):
        g = rng(w, l, S_REDRAW if redraw else S_TIER, redraw)
        edge = w.edge_layers and (l < w.edge_layers or l >= w.num_layers - w.edge_layers)
        mix = w.edge_mix if edge else (w.tier_mix or MIX_8B)
        out.append(_draw(mix, g))
    return out


def seq_lengths(w: Workload) -> np.ndarray:
    """Tokens cached at attention time, per sequence."""
    if not w.ragged:
        return np.full(w.batch, w.context, dtype=np.int32)
    u = rng(w, 0, S_LEN).uniform(math.log(w.len_lo), math.log(w.len_hi), size=w.batch)
    return np.rint(np.exp(u)).astype(np.int32)


def outlier_mask(w: Workload, layer: int) -> np.ndarray:
    """[H_kv][D] float32 multipliers for the key channels."""
    m = np.ones((w.num_kv_heads, w.head_dim), dtype=np.float32)
    if w.outlier_channels is not None:
        m[:, list(w.outlier_channels)] = w.outlier_scale
    elif w.outlier_frac > 0:
        total = w.num_kv_heads * w.head_dim
        k = int(round(w.outlier_frac * total))
        idx = rng(w, layer, S_OUTLIER).choice(total, size=k, replace=False)
        m.reshape(-1)[idx] = w.outlier_scale
    return m


def normal_f16(g: np.random.Generator, shape, mult: Optional[np.ndarray] = None) -> np.ndarray:
    """standard_normal in float32, optional float32 multiplier, cast to fp16 (RNE); uint16 bits."""
    x = g.standard_normal(shape, dtype=np.float32)
    if mult is not None:
        x = x * mult
    return x.astype(np.float16).view(np.uint16)


def keys_values(w: Workload, layer: int, n_tokens: int, stream_k: int, stream_v: int,
                step: int = 0, batch: Optional[int] = None):
    """K and V, [B][n][H_kv][D] uint16 fp16 bits; keys carry the outlier channels."""
    B = w.batch if batch is None else batch
    shape = (B, n_tokens, w.num_kv_heads, w.head_dim)
    k = normal_f16(rng(w, layer, stream_k, step), shape, outlier_mask(w, layer))
    v = normal_f16(rng(w, layer, stream_v, step), shape)
    return k, v


def sequence_keys_values(w: Workload, layer: int, seq: int, n_tokens: int):
    """K and V of one sequence, [1][n][H_kv][D] uint16 fp16 bits, from a stream of its own (ragged
    batches draw each sequence separately, so no array spans the longest length times the batch)."""
    shape = (1, n_tokens, w.num_kv_heads, w.head_dim)
    gk = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [MASTER_SEED, w.config_id, layer, S_PREFILL_K, 0, seq])))
    gv = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [MASTER_SEED, w.config_id, layer, S_PREFILL_V, 0, seq])))
    return normal_f16(gk, shape, outlier_mask(w, layer)), normal_f16(gv, shape)


def queries(w: Workload, layer: int, step: int = 0, batch: Optional[int] = None) -> np.ndarray:
    B = w.batch if batch is None else batch
    return normal_f16(rng(w, layer, S_Q, step), (B, w.num_q_heads, w.head_dim))


def handle(tier: int, index: int) -> int:
    return (int(tier) << 30) | int(index)


TIER_OF_BITS = {2: 0, 4: 1, 8: 2, 16: 3}
NO_BLOCK = 0xFFFFFFFF


def block_table(page_tiers: Sequence[Sequence[int]], max_pages: int, capacity: Sequence[int],
                g: np.random.Generator) -> np.ndarray:
    """Shuffled physical blocks: page_tiers[s][i] is the tier index of page i of sequence s.

    Each tier pool hands out its blocks in a seeded random order; returns [B][max_pages] uint32.
    """
    order = [list(g.permutation(int(c))) for c in capacity]
    nxt = [0] * len(capacity)
    bt = np.full((len(page_tiers), max_pages), NO_BLOCK, dtype=np.uint32)
    for s, tiers in enumerate(page_tiers):
        for i, t in enumerate(tiers):
            if nxt[t] >= len(order[t]):
                raise ValueError("synthetic pool too small")
            bt[s, i] = handle(t, order[t][nxt[t]])
            nxt[t] += 1
    return bt


def pages_for(n_tokens: int, page: int = PAGE) -> int:
    return (n_tokens + page - 1) // page
