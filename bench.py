#!/usr/bin/env python3
"""Decode-step benchmark of the mixed-precision quantized KV-cache path on one MI355X.

A step is one pass of the whole hot path over one synthetic decode token: for every layer,
quantize-on-write of the new key/value (kv_quant_write) followed by decode attention over the
paged mixed-precision cache (kv_decode_attn); once every 64 steps the KL canary fires for every
layer (kv_canary_kl_layers, one launch). The write and the attention of a layer run as one
launch (kv_decode_step; --unfused times the two separate calls). Inputs are resident in HBM
before timing starts; each timed step is replayed from a HIP graph holding exactly the eager
step's launches. The step time is the window of K steps divided by K plus one canary firing,
timed in windows of its own, divided by 64 -- the same charge whatever K is.

    python bench.py [--gpus 1] [--steps 256] [--warmup 10] [--workload qwen14b_32k]
                    [--also llama70b_128k] [--asymmetric] [--no-asym-leg]

Prints one JSON line. `value` is the effective cache bytes the attention kernels must read per
step divided by the step time (GB/s); steps/s is reported beside it. `also` holds the same
figures for a second workload (by default the 70B shape at 128K context), `asymmetric_format`
for the workload stored in the asymmetric format (a zero point beside every scale).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized decode-attn achieved HBM GB/s + decode steps/s, 14B-shape @32K"
HBM_PEAK_GBS = 8000.0
CANARY_EVERY = 64
CANARY_FIRINGS_TIMED = 8
ATTN_SRC = [os.path.join(ROOT, "mixed_precision_quantized_kv_amd", "csrc", f)
            for f in ("kv_attn.hip", "kvq_write_dev.hpp", "kvq_device.hpp")]

# HBM bytes per attention launch on the default workload, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) scaled by the same counters' reading for a plain copy kernel of known
# size. It describes the kernel sources with this digest only; after any change to them
# the bench reports traffic as null until the counters are taken again.
ATTN_TRAFFIC = {"source_sha256": "e67f8a86712c139e65774a47ccd39a255ca36915d7cfd4b552ca4f56cf707282",
                "bytes_per_launch": 45371011,
                # the bench's algorithmic bytes per launch at the counter run's contexts
                "algorithmic_bytes_per_launch": 41804027}


def source_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hbm_probes(torch, dev) -> dict:
    """Streaming references on the same GPU: a 4 GiB fp32 sum (read-only) and a 1 GiB copy
    (the known-size kernel that calibrates the HBM byte counters)."""
    out = {}
    x = torch.ones(1 << 30, dtype=torch.float32, device=dev)          # 4 GiB
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        x.sum()
    torch.cuda.synchronize()
    s0.record()
    for _ in range(5):
        x.sum()
    s1.record()
    torch.cuda.synchronize()
    out["sum_4GiB_GBps"] = round(5 * x.numel() * 4 / (s0.elapsed_time(s1) * 1e-3) / 1e9, 1)
    src = x[: 1 << 28]                                                  # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s0.record()
    for _ in range(5):
        dst.copy_(src)
    s1.record()
    torch.cuda.synchronize()
    out["copy_1GiB_GBps"] = round(5 * 2 * src.numel() * 4 / (s0.elapsed_time(s1) * 1e-3) / 1e9, 1)
    del x, dst
    torch.cuda.empty_cache()
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen14b_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=0, help="layers in the oracle's sample (0 = all)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="oracle steps timed per sampled layer")
    ap.add_argument("--pages-per-split", type=int, default=0)
    ap.add_argument("--unfused", action="store_true",
                    help="write and attend with two launches per layer instead of kv_decode_step")
    ap.add_argument("--fused", action="store_true",
                    help="use kv_decode_step also for more than 16 new tokens per sequence")
    ap.add_argument("--also", default="llama70b_128k",
                    help="a second workload measured after the first and reported under 'also' "
                         "('' to skip)")
    ap.add_argument("--asymmetric", action="store_true",
                    help="run the workload with the asymmetric cache format (zero point + scale)")
    ap.add_argument("--no-asym-leg", action="store_true",
                    help="skip the 'asymmetric_format' leg (the workload again, asymmetric format)")
    return ap.parse_args()


def attn_bytes(w, ctx: int, bits: int, asym: bool = False) -> int:
    """effective cache bytes one attention launch must read for one sequence of length ctx: the
    valid tokens' K and V codes and V scales, one K-scale vector per page and kv head, and the
    block-table entries (queries, outputs and workspace are not counted); the asymmetric format
    adds a zero point beside every scale"""
    D, H = w.head_dim, w.num_kv_heads
    pages = (ctx + 15) // 16
    par = 4 if asym else 2                           # bytes of a group's fp16 parameters
    per_kv = ctx * (D * bits // 4 + par) + pages * par * D
    return H * per_kv + 4 * pages


def write_bytes(w, pos: int, n: int, bits: int, asym: bool = False) -> int:
    """bytes the write of n tokens at pos must move for one sequence: the touched pages' present
    keys (ring or input) and the new values in, the pages' K codes and scales, the new tokens' V
    codes and scales, and the new keys into the ring out"""
    D, H, P = w.head_dim, w.num_kv_heads, 16
    lo = pos // P * P
    present = pos + n - lo                           # keys the touched pages hold afterwards
    pages = (pos + n - 1) // P - pos // P + 1
    par = 4 if asym else 2                           # bytes of a group's fp16 parameters
    per_kv = (present * D * 2 + n * D * 2 +          # keys and new values in
              pages * (P * D * bits // 8 + par * D) +  # K codes and scales out
              n * (D * bits // 8 + par) + n * D * 2)   # V codes and scales, ring out
    return H * per_kv


class Model:
    """All layers of one workload: pools, block tables (from the library's allocator), rings."""

    def __init__(self, w, steps_total: int, torch, kvq, synth, dev, asym=False):
        self.w = w
        self.asym = asym
        self.torch = torch
        L, B = w.num_layers, w.batch
        self.lens0 = synth.seq_lengths(w)                 # tokens at the first decode step
        self.max_ctx = int(self.lens0.max()) + steps_total * w.new_tokens
        self.max_pages = (self.max_ctx + 15) // 16 + 1
        self.bits = synth.layer_bits(w)
        self.g = kvq.geometry(L, w.num_q_heads, w.num_kv_heads, w.head_dim, B, self.max_pages,
                              asymmetric=asym)
        need = int(sum((int(n) + steps_total * w.new_tokens + 15) // 16 + 1 for n in self.lens0))
        cap = np.zeros((L, 3), dtype=np.uint32)
        for l, b in enumerate(self.bits):
            cap[l, synth.TIER_OF_BITS[b]] = need
        self.alloc = kvq.KVAlloc(self.g, cap, self.bits, shuffle_seed=12345)
        for s in range(B):                               # reserve every page the run will use
            self.alloc.kv_alloc_extend(s, int(self.lens0[s]) - 1 + steps_total * w.new_tokens)
        self.alloc.kv_check_block_table()
        self.bt = [torch.from_numpy(self.alloc.bt[l].view(np.int32).copy()).to(dev) for l in range(L)]
        self.pools_t, self.pools = [], []
        for l, b in enumerate(self.bits):
            tiers = []
            for t in range(3):
                n = int(cap[l, t])
                tiers.append(torch.empty(max(n * kvq.kv_block_bytes(self.g, kvq.TIER_BITS[t]), 256),
                                         dtype=torch.uint8, device=dev))
            self.pools_t.append(tiers)
            self.pools.append(kvq.layer_pools([x if c else 0 for x, c in zip(tiers, cap[l])], cap[l]))
        self.ring = [torch.zeros((B, w.ring_size, w.num_kv_heads, w.head_dim), dtype=torch.float16,
                                 device=dev) for _ in range(L)]


def gen_normal_f16(torch, shape, seed, dev, mult=None):
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    if mult is not None:
        x = x * mult
    return x.half()


def prefill(m: Model, kvq, synth, dev):
    """write the first len0 - 1 tokens of every sequence, layer by layer"""
    torch, w = m.torch, m.w
    for l in range(w.num_layers):
        mult = torch.from_numpy(synth.outlier_mask(w, l)).to(dev)
        for s in range(w.batch):
            n = int(m.lens0[s]) - 1
            if n <= 0:
                continue
            seed = (w.config_id * 1000 + l) * 100000 + s
            k = gen_normal_f16(torch, (1, n, w.num_kv_heads, w.head_dim), 2 * seed, dev, mult)
            v = gen_normal_f16(torch, (1, n, w.num_kv_heads, w.head_dim), 2 * seed + 1, dev)
            pos = torch.zeros(1, dtype=torch.int32, device=dev)
            kvq.kv_quant_write(m.g, m.pools[l], m.bt[l][s:s + 1], pos, 1, n, k, v, m.ring[l][s:s + 1])
    torch.cuda.synchronize()


def measure(w, steps: int, warmup: int, pages_per_split: int, unfused_flag: bool, fused_flag: bool,
            torch, kvq, synth, dev, asym: bool = False) -> dict:
    """GPU timings of one workload: the steps window, the attention launches, the canary firing"""
    L, B, nn = w.num_layers, w.batch, w.new_tokens
    # the fused step takes up to 64 new tokens, but with more than 16 (over two pages, written
    # two at a time by the last split's workgroup) the separate write launch measures faster
    unfused = unfused_flag or (nn > 16 and not fused_flag)
    steps_total = warmup + steps
    t0 = time.time()
    m = Model(w, steps_total, torch, kvq, synth, dev, asym)
    prefill(m, kvq, synth, dev)
    t_setup = time.time() - t0

    # per-step inputs, resident before timing
    gen_seed = w.config_id * 7919 + 1
    q_all = gen_normal_f16(torch, (steps_total, L, B, w.num_q_heads, w.head_dim), gen_seed, dev)
    k_all = gen_normal_f16(torch, (steps_total, L, B, nn, w.num_kv_heads, w.head_dim), gen_seed + 1, dev)
    v_all = gen_normal_f16(torch, (steps_total, L, B, nn, w.num_kv_heads, w.head_dim), gen_seed + 2, dev)
    lens0 = torch.from_numpy(m.lens0.astype(np.int32)).to(dev)
    pos_all = torch.stack([lens0 - 1 + i * nn for i in range(steps_total)]).contiguous()
    ctx_all = (pos_all + nn).contiguous()
    scale = 1.0 / math.sqrt(w.head_dim)
    # the split plan for the batch's lengths at the first timed step (the library's plan for
    # known lengths: one round for equal lengths, smaller balanced splits for a ragged batch; the
    # fused step's plan also keeps the last split, which writes, shorter)
    if pages_per_split:
        pps = pages_per_split
    elif unfused:
        pps = kvq.kv_decode_pages_per_split_for(m.g, (m.lens0 + warmup * nn).astype(np.int32))
    else:
        pps = kvq.kv_decode_step_pages_per_split_for(
            m.g, (m.lens0 - 1 + warmup * nn).astype(np.int32), nn)
    wsb = kvq.kv_decode_workspace_bytes(m.g, B, m.max_ctx, pps)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    cwsb = kvq.kv_canary_layers_workspace_bytes(m.g, L, B)
    cws = torch.zeros(cwsb, dtype=torch.uint8, device=dev)
    kl = torch.zeros((L, 3), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def writes_and_attention(i, sp_):
        for l in range(L):
            if unfused:
                kvq.kv_quant_write(m.g, m.pools[l], m.bt[l], pos_all[i], B, nn, k_all[i, l],
                                   v_all[i, l], m.ring[l], stream=sp_)
                kvq.kv_decode_attn(m.g, m.pools[l], m.bt[l], ctx_all[i], B, m.max_ctx, q_all[i, l],
                                   scale, out, ws, wsb, pps, stream=sp_)
            else:                                        # one launch: write, then attention
                kvq.kv_decode_step(m.g, m.pools[l], m.bt[l], pos_all[i], B, nn, k_all[i, l],
                                   v_all[i, l], m.ring[l], m.max_ctx, q_all[i, l], scale, out, ws,
                                   wsb, pps, stream=sp_)

    def attention_only(i, sp_):
        for l in range(L):
            if unfused:
                kvq.kv_decode_attn(m.g, m.pools[l], m.bt[l], ctx_all[i], B, m.max_ctx, q_all[i, l],
                                   scale, out, ws, wsb, pps, stream=sp_)
            else:          # the step's own kernel; replaying its write stores the same bytes again
                kvq.kv_decode_step(m.g, m.pools[l], m.bt[l], pos_all[i], B, nn, k_all[i, l],
                                   v_all[i, l], m.ring[l], m.max_ctx, q_all[i, l], scale, out, ws,
                                   wsb, pps, stream=sp_)

    def canary_all(i, sp_):                              # one firing: every layer, one launch
        kvq.kv_canary_kl_layers(m.g, m.ring, ctx_all[i], B, [q_all[i, l] for l in range(L)], scale,
                                kl, None, cws, cwsb, stream=sp_)

    for i in range(warmup):                              # eager warm-up steps
        writes_and_attention(i, sp)
        if i % CANARY_EVERY == 0:
            canary_all(i, sp)
    torch.cuda.synchronize()

    # Each timed step is replayed from a HIP graph captured once (one launch per step from the
    # host instead of ~L+1): a decode step is a chain of short kernels, and launching them one
    # by one from Python would time the interpreter, not the GPU. A step's graph holds the same
    # launches, with the same arguments, as the eager step.
    def capture(fn, i):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(i, torch.cuda.current_stream().cuda_stream)
        return g

    steps_idx = [warmup + j for j in range(steps)]
    n_fire = min(CANARY_FIRINGS_TIMED, steps)
    g_step = [capture(writes_and_attention, i) for i in steps_idx]
    g_attn = [capture(attention_only, i) for i in steps_idx]
    g_canary = [capture(canary_all, steps_idx[j]) for j in range(n_fire)]
    torch.cuda.synchronize()

    # timed window: exactly K steps, writes and attention for every layer
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for j in range(steps):
        g_step[j].replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step_nocanary = t_start.elapsed_time(t_end) / steps

    # attention launch durations: events on the launch stream around each step's L attention
    # launches, replayed back to back (the caches already hold the step's tokens, and each
    # layer's attention reads only its own layer's cache); the per-launch time is the group's / L
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for j in range(steps):
        evs[j][0].record(stream)
        g_attn[j].replay()
        evs[j][1].record(stream)
    torch.cuda.synchronize()
    attn_group_ms = np.array([a.elapsed_time(b) for (a, b) in evs])          # [K], L launches each

    # canary firings, each in its own event window right after a step (as it fires in a run):
    # the cost of one firing for all layers, charged to the step at the page's 1-in-64 rate
    cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_fire)]
    torch.cuda.synchronize()
    for j in range(n_fire):
        g_step[j].replay()
        cevs[j][0].record(stream)
        g_canary[j].replay()
        cevs[j][1].record(stream)
    torch.cuda.synchronize()
    canary_ms = float(np.mean([a.elapsed_time(b) for (a, b) in cevs]))
    del g_step, g_attn, g_canary
    ms_step = ms_step_nocanary + canary_ms / CANARY_EVERY

    # algorithmic bytes
    lens = m.lens0.astype(np.int64)
    step_bytes = []
    per_launch_bytes = np.zeros((steps, L))
    for j in range(steps):
        ctx = lens + (warmup + j) * nn
        for l, b in enumerate(m.bits):
            per_launch_bytes[j, l] = sum(attn_bytes(w, int(c), b, asym) for c in ctx)
            if not unfused:
                per_launch_bytes[j, l] += sum(write_bytes(w, int(c) - nn, nn, b, asym) for c in ctx)
        step_bytes.append(sum(attn_bytes(w, int(c), b, asym) for c in ctx for b in m.bits))
    step_bytes = float(np.mean(step_bytes))
    avg_launch_bytes = float(per_launch_bytes.mean())
    avg_attn_ms = float(attn_group_ms.mean()) / L
    achieved = avg_launch_bytes / (avg_attn_ms * 1e-3) / 1e9
    res = {"m": m, "unfused": unfused, "pps": pps, "setup_s": t_setup, "ms_step": ms_step,
           "ms_step_nocanary": ms_step_nocanary, "canary_ms": canary_ms, "n_fire": n_fire,
           "step_bytes": step_bytes, "avg_launch_bytes": avg_launch_bytes,
           "avg_attn_ms": avg_attn_ms, "achieved": achieved}
    return res


def run(args):
    import torch

    import mixed_precision_quantized_kv_amd as kvq
    from mixed_precision_quantized_kv_amd import synth

    dev = "cuda:0"
    w = synth.WORKLOADS[args.workload]
    L, B = w.num_layers, w.batch
    r = measure(w, args.steps, args.warmup, args.pages_per_split, args.unfused, args.fused,
                torch, kvq, synth, dev, args.asymmetric)
    m, unfused, pps = r["m"], r["unfused"], r["pps"]
    ms_step, step_bytes, achieved = r["ms_step"], r["step_bytes"], r["achieved"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    bits = list(m.bits)
    del r["m"], m
    torch.cuda.empty_cache()
    probes = hbm_probes(torch, dev)
    traffic = None
    if (ATTN_TRAFFIC["source_sha256"] == source_digest(ATTN_SRC) and not unfused
            and args.workload == "qwen14b_32k" and not args.pages_per_split and not args.asymmetric):
        traffic = ATTN_TRAFFIC["bytes_per_launch"]      # taken on the fused kernel, default workload
    tiers = {b: bits.count(b) for b in (2, 4, 8)}
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "steps_per_s": round(1000.0 / ms_step, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "layers": L, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "batch": B, "context": int(synth.seq_lengths(w).max()),
            "page": 16, "ring": w.ring_size, "layer_bits": {f"int{b}": n for b, n in tiers.items()},
            "pages_per_split": pps, "canary_every": CANARY_EVERY,
        },
        "storage": ("packed int2/int4/int8 codes + fp16 zero points and scales (asymmetric format)"
                    if args.asymmetric else "packed int2/int4/int8 codes + fp16 scales")
                   + "; f16 MFMA, f32 accumulate",
        "step_time": "ms_per_step = the window of K steps (every layer's write and attention) / K "
                     "+ one canary firing (every layer, one launch, own event window) / 64",
        "attn_bytes_per_step": int(step_bytes),
        "attn_kernel_us": round(r["avg_attn_ms"] * 1e3, 3),
        "ms_per_step_no_canary": round(r["ms_step_nocanary"], 5),
        "canary_ms_per_firing": round(r["canary_ms"], 5),
        "canary_firings_timed": r["n_fire"],
        "canary_overhead": round(r["canary_ms"] / CANARY_EVERY / r["ms_step_nocanary"], 5),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": f"decode_attn_kernel<{w.head_dim}> (unfused)" if unfused else
                      f"decode_attn_kernel<{w.head_dim}> fused with the write (kv_decode_step)",
            "bytes_per_launch": int(r["avg_launch_bytes"]),
            "traffic_over_algorithmic": (round(traffic / ATTN_TRAFFIC["algorithmic_bytes_per_launch"], 4)
                                         if traffic else None),
        },
        "hbm_probes": probes,
        # the same achieved rate against what a plain streaming sum over 4 GiB reaches on this GPU
        "frac_of_sum_probe": round(achieved / probes["sum_4GiB_GBps"], 4),
        "attn_source_sha256": source_digest(ATTN_SRC),
        "setup_s": round(r["setup_s"], 1),
    }
    if args.also and args.workload != args.also:
        wa = synth.WORKLOADS[args.also]
        ra = measure(wa, min(args.steps, 64), min(args.warmup, 4), 0, False, False, torch, kvq,
                     synth, dev)
        del ra["m"]
        torch.cuda.empty_cache()
        ms_a = ra["ms_step"]
        res["also"] = {
            "workload": wa.name, "layers": wa.num_layers, "q_heads": wa.num_q_heads,
            "kv_heads": wa.num_kv_heads, "batch": wa.batch,
            "context": int(synth.seq_lengths(wa).max()), "pages_per_split": ra["pps"],
            "steps": min(args.steps, 64), "value": round(ra["step_bytes"] / (ms_a * 1e-3) / 1e9, 2),
            "unit": "GB/s", "ms_per_step": round(ms_a, 5), "steps_per_s": round(1000.0 / ms_a, 2),
            "attn_kernel_us": round(ra["avg_attn_ms"] * 1e3, 3),
            "canary_ms_per_firing": round(ra["canary_ms"], 5),
            "roofline_frac": round(ra["achieved"] / HBM_PEAK_GBS, 4),
        }
    if not args.no_asym_leg and not args.asymmetric:
        rs = measure(w, min(args.steps, 64), min(args.warmup, 4), 0, args.unfused, args.fused,
                     torch, kvq, synth, dev, True)
        del rs["m"]
        torch.cuda.empty_cache()
        res["asymmetric_format"] = {
            "workload": w.name, "storage": "zero point + scale per group (KIVI-style)",
            "steps": min(args.steps, 64), "value": round(rs["step_bytes"] / (rs["ms_step"] * 1e-3) / 1e9, 2),
            "unit": "GB/s", "ms_per_step": round(rs["ms_step"], 5),
            "steps_per_s": round(1000.0 / rs["ms_step"], 2),
            "attn_kernel_us": round(rs["avg_attn_ms"] * 1e3, 3),
            "roofline_frac": round(rs["achieved"] / HBM_PEAK_GBS, 4),
        }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, bits, args.cpu_layers, args.cpu_reps, step_bytes)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, bits, n_layers: int, reps: int, step_bytes: float) -> dict:
    """The oracle (plain C, fp64) on a bounded sample of the same decode step. All cores: for
    each sampled layer, quantize-on-write of the new token plus decode attention at full context,
    repeated `reps` times, scaled to all layers; the canary of every layer timed on its own and
    charged at its 1-in-64 rate. One thread: one layer of each width once (write + attention) and
    one canary, weighted by the workload's layer mix."""
    import oracle
    from mixed_precision_quantized_kv_amd import synth

    oracle.lib()
    all_threads = oracle.num_threads()
    g = oracle.geom(w.num_q_heads, w.num_kv_heads, w.head_dim, 16, w.ring_size)
    N = int(synth.seq_lengths(w).max())
    layers = list(range(n_layers if n_layers > 0 else w.num_layers))
    B = w.batch
    # one seeded draw of keys and values serves every sampled layer (the oracle's time does not
    # depend on the values); each layer keeps its own bit-width
    K, V = synth.keys_values(w, 0, N, synth.S_PREFILL_K, synth.S_PREFILL_V)
    scale = np.float32(1.0 / math.sqrt(w.head_dim))
    prepared = {}                   # one prefilled cache per bit-width, shared by its layers
    for b in sorted(set(bits[l] for l in layers) | set(bits)):
        tier = synth.TIER_OF_BITS[b]
        pages = (N + 15) // 16
        cap = [pages * B if t == tier else 1 for t in range(3)]
        bt = synth.block_table([[tier] * pages] * B, pages, cap, synth.rng(w, b, synth.S_SHUFFLE))
        pools = oracle.Pools(g, cap)
        ring = np.zeros((B, w.ring_size, w.num_kv_heads, w.head_dim), dtype=np.uint16)
        oracle.quant_write(g, pools, bt, np.zeros(B, np.int32), K[:, :N - 1], V[:, :N - 1], ring)
        prepared[b] = (bt, pools, ring)

    def one_layer_step(b, q):
        bt, pools, ring = prepared[b]
        t0 = time.perf_counter()
        oracle.quant_write(g, pools, bt, np.full(B, N - 1, np.int32), K[:, N - 1:], V[:, N - 1:], ring)
        oracle.decode_attn(g, pools, bt, np.full(B, N, np.int32), q, scale)
        return time.perf_counter() - t0

    def one_canary(b, q):
        _, _, ring = prepared[b]
        t0 = time.perf_counter()
        oracle.canary_kl(g, ring, np.full(B, N, np.int32), q, scale)
        return time.perf_counter() - t0

    oracle.set_num_threads(all_threads)
    t_step_sum = 0.0
    for l in layers:
        q = synth.queries(w, l)
        for _ in range(reps):
            t_step_sum += one_layer_step(bits[l], q)
    t_canary_firing = sum(one_canary(bits[l], synth.queries(w, l)) for l in range(w.num_layers))
    t_step_nocanary = t_step_sum / (len(layers) * reps) * w.num_layers
    t_step = t_step_nocanary + t_canary_firing / CANARY_EVERY

    # one thread: a layer of each width, weighted by how many layers have that width
    oracle.set_num_threads(1)
    t1 = 0.0
    t1_canary = 0.0
    t1_measured = 0.0
    for b in sorted(set(bits)):
        q = synth.queries(w, bits.index(b))
        ts, tc = one_layer_step(b, q), one_canary(b, q)
        t1 += ts * bits.count(b)
        t1_canary += tc * bits.count(b)
        t1_measured += ts + tc
    oracle.set_num_threads(all_threads)
    t1_step = t1 + t1_canary / CANARY_EVERY

    # the oracle's parallel loop runs over (sequence, KV head) items
    cores = min(all_threads, B * w.num_kv_heads)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(step_bytes / t_step / 1e9, 4), "unit": "GB/s", "cores": cores,
            "cores_counted": f"threads with work: the oracle's parallel loop has batch x KV heads "
                             f"= {B * w.num_kv_heads} items, run on {all_threads} threads",
            "kind": "oracle", "steps_per_s": round(1.0 / t_step, 5),
            "s_per_step_no_canary": round(t_step_nocanary, 4),
            "canary_s_per_firing": round(t_canary_firing, 4),
            "one_thread": {"value": round(step_bytes / t1_step / 1e9, 4), "unit": "GB/s",
                           "steps_per_s": round(1.0 / t1_step, 5),
                           "canary_s_per_firing": round(t1_canary, 4),
                           "sample": f"one layer of each width ({sorted(set(bits))}) once, "
                                     f"weighted by the layer mix"},
            "host_cpus": os.cpu_count(), "cpu_model": model, "oracle_threads": all_threads,
            "sample": f"{len(layers)} of {w.num_layers} layers, each {reps}x one decode step "
                      f"(write of the new token + attention at context {N}, batch {B}), scaled to "
                      f"{w.num_layers} layers; the canary of all {w.num_layers} layers timed once, "
                      f"charged at 1/{CANARY_EVERY}",
            "seconds_measured": round(t_step_sum + t_canary_firing + t1_measured, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus above 1 is not supported "
                                   "(sharding over GPUs is not implemented)", "n_gpus": args.gpus}))
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
