"""Shared setup for the GPU parity tests: one layer's cache on the device (through the C ABI) and
the same layer in the oracle, fed with identical seeded inputs.

Inputs come from mixed_precision_quantized_kv_amd.synth; nothing here computes any part of the
method. Expected values come only from the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import mixed_precision_quantized_kv_amd as kvq
import oracle
from mixed_precision_quantized_kv_amd import synth

DEV = "cuda:0"


def to_dev_f16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.float16)).to(DEV)


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


class LayerPair:
    """One layer: GPU pools + ring (via libkvq) and oracle pools + ring, same block table."""

    def __init__(self, hq, hkv, d, batch, max_pages, page_tiers, capacity=None, seed=0, R=64,
                 asymmetric=False, fill=0):
        self.hq, self.hkv, self.d, self.batch, self.R = hq, hkv, d, batch, R
        self.g = kvq.geometry(1, hq, hkv, d, batch, max_pages, ring_size=R, asymmetric=asymmetric)
        self.og = oracle.geom(hq, hkv, d, 16, R, asymmetric=asymmetric)
        if capacity is None:
            capacity = [max(1, sum(t == tier for row in page_tiers for t in row)) for tier in range(4)]
        self.capacity = list(capacity)
        self.bt = synth.block_table(page_tiers, max_pages, self.capacity,
                                    np.random.default_rng(seed + 1000))
        # fill: the byte the GPU pools start with (the oracle's start at zero); a fill other than 0
        # leaves those bytes in every slot no token has been written to yet
        self.pools_t = [torch.full((max(16, c * kvq.kv_block_bytes(self.g, b)),), fill, dtype=torch.uint8,
                                   device=DEV) for c, b in zip(self.capacity, kvq.TIER_BITS)]
        self.pools = kvq.layer_pools(self.pools_t, self.capacity)
        self.bt_dev = to_dev_i32(self.bt)
        self.ring = torch.zeros((batch, R, hkv, d), dtype=torch.float16, device=DEV)
        self.opools = oracle.Pools(self.og, self.capacity)
        self.oring = np.zeros((batch, R, hkv, d), dtype=np.uint16)
        self.len = np.zeros(batch, dtype=np.int32)

    def write(self, k_new: np.ndarray, v_new: np.ndarray, rows=None):
        """append n tokens to sequences `rows` (all when None) on both sides"""
        n = k_new.shape[1]
        if rows is None:
            pos = self.len.copy()
            kvq.kv_quant_write(self.g, self.pools, self.bt_dev, to_dev_i32(pos), self.batch, n,
                               to_dev_f16(k_new), to_dev_f16(v_new), self.ring)
            oracle.quant_write(self.og, self.opools, self.bt, pos, k_new, v_new, self.oring)
            self.len += n
            return
        for i, s in enumerate(rows):       # one sequence at a time, through row offsets
            pos = self.len[s:s + 1].copy()
            mp = self.g.max_pages_per_seq
            bt_row = self.bt_dev[s:s + 1]
            ring_row = self.ring[s:s + 1]
            kvq.kv_quant_write(self.g, self.pools, bt_row, to_dev_i32(pos), 1, n,
                               to_dev_f16(k_new[i:i + 1]), to_dev_f16(v_new[i:i + 1]), ring_row)
            oring = self.oring[s:s + 1].copy()
            oracle.quant_write(self.og, self.opools, self.bt[s:s + 1], pos, k_new[i:i + 1],
                               v_new[i:i + 1], oring)
            self.oring[s:s + 1] = oring
            self.len[s] += n
            del mp

    def used_blocks(self):
        out = []
        for s in range(self.batch):
            for p in range((int(self.len[s]) + 15) // 16):
                h = int(self.bt[s, p])
                out.append((s, p, h >> 30, h & 0x3FFFFFFF))
        return out

    def compare_bytes(self, blocks=None):
        """bit-exact comparison of the written blocks and the ring; returns mismatching blocks"""
        torch.cuda.synchronize()
        gp = [t.cpu().numpy() for t in self.pools_t]
        bad = []
        for (s, p, t, i) in (blocks if blocks is not None else self.used_blocks()):
            nb = oracle.block_bytes(self.og, kvq.TIER_BITS[t])
            a = gp[t][i * nb:(i + 1) * nb]
            b = self.opools.arrays[t][i * nb:(i + 1) * nb]
            if not np.array_equal(a, b):
                bad.append((s, p, t, i, int(np.sum(a != b))))
        ring_ok = np.array_equal(f16_bits(self.ring), self.oring)
        return bad, ring_ok

    def step(self, k_new: np.ndarray, v_new: np.ndarray, q_u16, pages_per_split=0, scale=None):
        """kv_decode_step on the GPU (write of the new tokens, then attention over them, one
        launch), the same write on the oracle side; returns the attention rows and the workspace"""
        B, n = self.batch, k_new.shape[1]
        pos = self.len.copy()
        max_ctx = int((pos + n).max())
        scale = np.float32(1.0 / math.sqrt(self.d)) if scale is None else np.float32(scale)
        wsb = kvq.kv_decode_workspace_bytes(self.g, B, max_ctx, pages_per_split)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        out = torch.empty((B, self.hq, self.d), dtype=torch.float32, device=DEV)
        kvq.kv_decode_step(self.g, self.pools, self.bt_dev, to_dev_i32(pos), B, n, to_dev_f16(k_new),
                           to_dev_f16(v_new), self.ring, max_ctx, to_dev_f16(q_u16), float(scale),
                           out, ws, wsb, pages_per_split)
        torch.cuda.synchronize()
        oracle.quant_write(self.og, self.opools, self.bt, pos, k_new, v_new, self.oring)
        self.len += n
        return out.cpu().numpy().astype(np.float64), ws

    def tickets_zero(self, ws: torch.Tensor) -> bool:
        """the split-ticket counters at the head of an attention workspace -- one 256-byte line
        per (sequence slot, KV head) of the geometry, plus one line -- are all back at zero"""
        n = self.g.max_seqs * self.g.num_kv_heads * 256 + 256
        return not ws[:n].any()

    def attn(self, q_u16, ctx=None, scale=None, pages_per_split=0):
        ctx = self.len.copy() if ctx is None else np.asarray(ctx, dtype=np.int32)
        scale = np.float32(1.0 / math.sqrt(self.d)) if scale is None else np.float32(scale)
        max_ctx = int(ctx.max()) if ctx.size else 0
        wsb = kvq.kv_decode_workspace_bytes(self.g, self.batch, max_ctx, pages_per_split)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        out = torch.empty((self.batch, self.hq, self.d), dtype=torch.float32, device=DEV)
        kvq.kv_decode_attn(self.g, self.pools, self.bt_dev, to_dev_i32(ctx), self.batch, max_ctx,
                           to_dev_f16(q_u16), float(scale), out, ws, wsb, pages_per_split)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), ws

    def oracle_attn(self, q_u16, ctx=None, scale=None):
        ctx = self.len.copy() if ctx is None else np.asarray(ctx, dtype=np.int32)
        scale = np.float32(1.0 / math.sqrt(self.d)) if scale is None else np.float32(scale)
        return oracle.decode_attn(self.og, self.opools, self.bt, ctx, q_u16, scale)

    def canary(self, q_u16, seq_len=None, scale=None):
        seq_len = self.len.copy() if seq_len is None else np.asarray(seq_len, dtype=np.int32)
        scale = np.float32(1.0 / math.sqrt(self.d)) if scale is None else np.float32(scale)
        wsb = kvq.kv_canary_workspace_bytes(self.g, self.batch)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        kl = torch.zeros(3, dtype=torch.float32, device=DEV)
        rows = torch.zeros((self.batch, self.hq, 3), dtype=torch.float32, device=DEV)
        kvq.kv_canary_kl(self.g, self.ring, to_dev_i32(seq_len), self.batch, to_dev_f16(q_u16),
                         float(scale), kl, rows, ws, wsb)
        torch.cuda.synchronize()
        return kl.cpu().numpy().astype(np.float64), rows.cpu().numpy().astype(np.float64)

    def oracle_canary(self, q_u16, seq_len=None, scale=None):
        seq_len = self.len.copy() if seq_len is None else np.asarray(seq_len, dtype=np.int32)
        scale = np.float32(1.0 / math.sqrt(self.d)) if scale is None else np.float32(scale)
        return oracle.canary_kl(self.og, self.oring, seq_len, q_u16, scale)


def rowwise_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """per output row: max_c |got - ref| / max_c |ref| (rows of ref that are all zero: absolute)"""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)
