"""GPU parity: libkvq (HIP, gfx950) against the CPU oracle, element by element.

Bar: packed codes, scales and the ring bit-exact; attention rows within 2e-3 of the oracle's
fp64 result (per row: max |err| / max |ref|); canary KL within 1e-4 absolute, mean and rows.
"""
import math

import numpy as np
import pytest
import torch

from mixed_precision_quantized_kv_amd import synth

import mixed_precision_quantized_kv_amd as kvq

from gpu_cases import LayerPair, rowwise_rel_err, to_dev_f16, to_dev_i32

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3
KL_TOL = 1e-4
TINY = synth.WORKLOADS["tiny"]


def case_banner(msg):
    print(f"\n[case] {msg}", flush=True)


def tiny_layer(layer: int, N: int = 512, chunks=(100, 16, 200, 195), seed=0):
    """tiny workload layer: prefill N-1 tokens in chunks, then the decode-step token"""
    bits = synth.layer_bits(TINY)[layer]
    tier = synth.TIER_OF_BITS[bits]
    pages = synth.pages_for(N)
    L = LayerPair(8, 2, 64, 1, pages + 2, [[tier] * pages], seed=seed + layer)
    K, V = synth.keys_values(TINY, layer, N, synth.S_PREFILL_K, synth.S_PREFILL_V)
    p = 0
    for n in list(chunks) + [N - 1 - sum(chunks)]:
        if n > 0:
            L.write(K[:, p:p + n], V[:, p:p + n])
            p += n
    L.write(K[:, p:p + 1], V[:, p:p + 1])          # the decode step's own token
    return L


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_tiny_write_attention_canary(layer):
    case_banner(f"tiny layer {layer}")
    L = tiny_layer(layer)
    bad, ring_ok = L.compare_bytes()
    assert not bad, f"blocks differ: {bad[:5]}"
    assert ring_ok
    q = synth.queries(TINY, layer)
    ref = L.oracle_attn(q)
    for pps in (0, 16, 32):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}")
        assert err.max() <= ATTN_TOL, (pps, err.max())
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    print(f"  canary {okl} max abs err {np.abs(rows - orows).max():.3e}")
    assert np.abs(kl - okl).max() <= KL_TOL, (kl, okl)
    assert np.abs(rows - orows).max() <= KL_TOL


@pytest.mark.parametrize("tier", [0, 1, 2])
def test_token_by_token_writes(tier):
    case_banner(f"token-by-token tier {tier}")
    L = LayerPair(8, 2, 64, 2, 8, [[tier] * 6] * 2, seed=tier)
    g = np.random.default_rng(tier)
    K = synth.normal_f16(g, (2, 90, 2, 64), np.where(np.arange(64) % 7 == 0, 10, 1).astype(np.float32))
    V = synth.normal_f16(g, (2, 90, 2, 64))
    for p in range(90):
        L.write(K[:, p:p + 1], V[:, p:p + 1])
        if p in (0, 1, 15, 16, 17, 63, 64, 65, 89):
            bad, ring_ok = L.compare_bytes()
            assert not bad and ring_ok, (p, bad[:3])


def test_large_chunk_overwrites_ring():
    """n_new > R - P: new keys overwrite ring slots that hold the open page's earlier keys"""
    case_banner("large chunk")
    L = LayerPair(8, 2, 128, 2, 16, [[1, 2, 0, 1, 2, 0, 1, 2, 0, 1]] * 2, seed=3)
    g = np.random.default_rng(3)
    K = synth.normal_f16(g, (2, 150, 2, 128))
    V = synth.normal_f16(g, (2, 150, 2, 128))
    L.write(K[:, :9], V[:, :9])
    L.write(K[:, 9:140], V[:, 9:140])
    L.write(K[:, 140:150], V[:, 140:150])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok


def test_striped_layer_and_short_context():
    """a layer whose first 256 tokens are INT2 and the rest INT8; and N = 40 < R"""
    case_banner("striped + short")
    tiers = [0] * 16 + [2] * 16
    L = LayerPair(8, 2, 64, 1, 34, [tiers], seed=5)
    K, V = synth.keys_values(TINY, 1, 512, synth.S_PREFILL_K, synth.S_PREFILL_V)
    L.write(K[:, :300], V[:, :300])
    L.write(K[:, 300:512], V[:, 300:512])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.queries(TINY, 1)
    for ctx in (512, 256, 257, 40, 1):
        got, _ = L.attn(q, ctx=[ctx])
        assert rowwise_rel_err(got, L.oracle_attn(q, ctx=[ctx])).max() <= ATTN_TOL, ctx
    S = LayerPair(8, 2, 64, 1, 4, [[1, 1, 1]], seed=6)
    S.write(K[:, :40], V[:, :40])
    got, _ = S.attn(q)
    assert rowwise_rel_err(got, S.oracle_attn(q)).max() <= ATTN_TOL
    kl, rows = S.canary(q)
    okl, orows = S.oracle_canary(q)
    assert np.abs(kl - okl).max() <= KL_TOL and np.abs(rows - orows).max() <= KL_TOL


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (40, 8, 128), (28, 4, 128), (64, 8, 128),
                                      (16, 16, 64), (16, 1, 64)])
def test_ragged_batch_gqa_shapes(hq, hkv, d):
    """group sizes 1, 4, 5, 7, 8, 16; lengths 0, 1, 15, 16, 17, ragged; mixed tiers per page"""
    case_banner(f"ragged hq={hq} hkv={hkv} d={d}")
    lens = [0, 1, 15, 16, 17, 300, 1000, 777]
    B = len(lens)
    g = np.random.default_rng(hq * 100 + d)
    tiers = [list(g.integers(0, 3, size=64)) for _ in range(B)]
    L = LayerPair(hq, hkv, d, B, 64, tiers, seed=hq)
    for s, n in enumerate(lens):
        if n:
            K = synth.normal_f16(g, (1, n, hkv, d), np.where(np.arange(d) % 11 == 0, 8, 1).astype(np.float32))
            V = synth.normal_f16(g, (1, n, hkv, d))
            L.write(K, V, rows=[s])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok
    q = synth.normal_f16(g, (B, hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 16):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}")
        assert err.max() <= ATTN_TOL, (pps, err.max(), np.argmax(err.max(-1)))
    assert not got[0].any()                       # the empty sequence gives a zero row
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    assert np.abs(kl - okl).max() <= KL_TOL and np.abs(rows - orows).max() <= KL_TOL


@pytest.mark.parametrize("hq,hkv,d", [(40, 8, 128), (8, 2, 64)])
@pytest.mark.parametrize("mix", ["int8", "int4", "int2", "mixed"])
def test_many_page_pairs_per_wave(hq, hkv, d, mix):
    """long splits: each wave walks up to 8 page pairs (ctx 2048 and 1500, up to 128 pages per
    split), so the loaded-ahead page buffers are refilled many times inside the loop"""
    case_banner(f"many pairs hq={hq} hkv={hkv} d={d} {mix}")
    g = np.random.default_rng(d * 10 + len(mix))
    lens = [2048, 1500]
    if mix == "mixed":
        tiers = [list(g.integers(0, 3, size=130)) for _ in lens]
    else:
        tiers = [[{"int2": 0, "int4": 1, "int8": 2}[mix]] * 130 for _ in lens]
    L = LayerPair(hq, hkv, d, len(lens), 130, tiers, seed=d)
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, hkv, d))
        V = synth.normal_f16(g, (1, n, hkv, d))
        L.write(K, V, rows=[s])
    q = synth.normal_f16(g, (len(lens), hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 32, 64, 128):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}")
        assert err.max() <= ATTN_TOL, (pps, err.max())


@pytest.mark.parametrize("tier", [0, 1, 2, "mix"])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_logits_rising_or_falling_across_pages(tier, direction):
    """the running maximum of the page loop: keys whose logit climbs by ~6 (log2 units) every
    page, so the maximum is raised in every round, and the reverse order, where it never is.
    One key channel is hundreds of times larger than the rest, so every logit is a large term
    plus small ones: products of very different sizes meet in each MFMA. "mix" cycles the page
    widths INT2, INT4, INT8, FP16 (the general loops)."""
    case_banner(f"{direction} logits, tier {tier}")
    tiers = [p % 4 for p in range(44)] if tier == "mix" else [tier] * 44
    seed = 3 if tier == "mix" else tier
    N = 700
    g = np.random.default_rng(31 + seed)
    ramp = np.arange(N, dtype=np.float32)           # logit +0.25 a token: ~5.8 log2 units a page
    if direction == "falling":
        ramp = ramp[::-1].copy()
    K = (g.standard_normal((1, N, 2, 64), dtype=np.float32) * 0.1)
    K[:, :, :, 0] += ramp[None, :, None]
    K = K.astype(np.float16).view(np.uint16)
    V = synth.normal_f16(g, (1, N, 2, 64))
    L = LayerPair(8, 2, 64, 1, 46, [tiers], seed=seed)
    L.write(K, V)
    qf = np.zeros((1, 8, 64), dtype=np.float32)
    qf[:, :, 0] = 2.0
    qf[:, :, 1:] = g.standard_normal((1, 8, 63), dtype=np.float32) * 0.1
    q = qf.astype(np.float16).view(np.uint16)
    ref = L.oracle_attn(q)
    for pps in (0, 4, 16, 44):
        got, _ = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}")
        assert err.max() <= ATTN_TOL, (pps, err.max())


def test_deterministic_and_workspace_reuse():
    case_banner("determinism")
    L = tiny_layer(2)
    q = synth.queries(TINY, 2)
    a, ws = L.attn(q, pages_per_split=16)
    b, _ = L.attn(q, pages_per_split=16)
    assert np.array_equal(a, b)
    assert L.tickets_zero(ws)                      # every ticket counter is left at zero


def test_workspace_reused_across_batch_sizes():
    """one workspace for calls over 2, 8, 2 and 8 sequences of one geometry: each call finds its
    split counters where the previous call left them at zero (their place does not move with
    the batch), and its outputs equal those of a fresh workspace bit for bit"""
    case_banner("workspace reuse across batch sizes")
    lens = [3000, 1000, 2500, 17, 4000, 800, 1600, 3333]
    B, hq, hkv, d = len(lens), 40, 8, 128
    g = np.random.default_rng(5)
    L = LayerPair(hq, hkv, d, B, 256, [[1] * 256 for _ in range(B)], seed=5)
    for s, n in enumerate(lens):
        L.write(synth.normal_f16(g, (1, n, hkv, d)), synth.normal_f16(g, (1, n, hkv, d)), rows=[s])
    q = synth.normal_f16(g, (B, hq, d))
    ctx = np.array(lens, dtype=np.int32)
    wsb = max(kvq.kv_decode_workspace_bytes(L.g, b, int(ctx.max()), 16) for b in (2, B))

    def call(batch, ws):
        out = torch.empty((batch, hq, d), dtype=torch.float32, device="cuda")
        kvq.kv_decode_attn(L.g, L.pools, L.bt_dev, to_dev_i32(ctx[:batch]), batch,
                           int(ctx[:batch].max()), to_dev_f16(q[:batch]), 1.0 / math.sqrt(d), out,
                           ws, wsb, 16)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    fresh = {b: call(b, torch.zeros(wsb, dtype=torch.uint8, device="cuda")) for b in (2, B)}
    ref = L.oracle_attn(q)
    assert rowwise_rel_err(fresh[B].astype(np.float64), ref).max() <= ATTN_TOL
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    for b in (2, B, 2, B):
        assert np.array_equal(call(b, ws), fresh[b]), b
    assert L.tickets_zero(ws)                       # every ticket counter is left at zero


def test_softmax_scale_zero_and_identical_keys():
    case_banner("closed forms")
    key = synth.normal_f16(np.random.default_rng(1), (1, 1, 2, 64))
    K = np.repeat(key, 200, axis=1)
    V = synth.normal_f16(np.random.default_rng(2), (1, 200, 2, 64))
    L = LayerPair(8, 2, 64, 1, 14, [[1] * 13], seed=9)
    L.write(K, V)
    q = synth.queries(TINY, 0)
    for scale in (0.0, 0.125, 3.0):
        got, _ = L.attn(q, scale=scale)
        assert rowwise_rel_err(got, L.oracle_attn(q, scale=scale)).max() <= ATTN_TOL


def test_negative_softmax_scale():
    """a scale of either sign is a valid softmax temperature: with a negative one the weights
    favour the smallest logits; attention over mixed widths and the canary against the oracle"""
    case_banner("negative softmax scale")
    g = np.random.default_rng(4)
    tiers = [[0, 1, 2, 3, 1, 0, 2, 1, 2, 0]]
    L = LayerPair(16, 4, 128, 1, 10, tiers, seed=4)
    K = synth.normal_f16(g, (1, 150, 4, 128))
    V = synth.normal_f16(g, (1, 150, 4, 128))
    L.write(K, V)
    q = synth.normal_f16(g, (1, 16, 128))
    for scale in (-0.088, -1.0):
        for pps in (0, 2):
            got, _ = L.attn(q, scale=scale, pages_per_split=pps)
            assert rowwise_rel_err(got, L.oracle_attn(q, scale=scale)).max() <= ATTN_TOL
        kl, rows = L.canary(q, scale=scale)
        okl, orows = L.oracle_canary(q, scale=scale)
        assert np.abs(kl - okl).max() <= 1e-4 and np.abs(rows - orows).max() <= 1e-4


@pytest.mark.parametrize("zero_values", [True, False])
def test_split_partials_that_are_exactly_zero(zero_values):
    """split partials whose running maximum is exactly +0.0 (every logit -3 in log2 units, the
    lazy maximum's margin above it) and, with zero values, whose accumulators are +0.0 too, at
    32 and 8 splits: the merge takes them like any other (zero rows, or the mean of the values).
    INT2 keys [-1, 0, ..., 0] quantize exactly (scale 1), so q . k = -1 exactly."""
    case_banner(f"exactly-zero split partials, zero values {zero_values}")
    N, hq, hkv, d = 2000, 8, 2, 64
    pages = synth.pages_for(N)
    K = np.zeros((1, N, hkv, d), dtype=np.float16)
    K[..., 0] = -1.0
    g = np.random.default_rng(77)
    V = np.zeros((1, N, hkv, d), dtype=np.float16) if zero_values else \
        g.standard_normal((1, N, hkv, d)).astype(np.float16)
    L = LayerPair(hq, hkv, d, 1, pages + 2, [[0] * pages], seed=77)
    L.write(K.view(np.uint16), V.view(np.uint16))
    qf = np.zeros((1, hq, d), dtype=np.float16)
    qf[..., 0] = 1.0
    q = qf.view(np.uint16)
    scale = float(np.float32(3 / 1.4426950408889634))
    assert np.float32(scale) * np.float32(1.4426950408889634) == np.float32(3.0)
    ref = L.oracle_attn(q, scale=scale)
    for pps in (4, 16):
        got, ws = L.attn(q, scale=scale, pages_per_split=pps)
        assert np.isfinite(got).all(), pps
        if zero_values:
            assert not got.any(), pps
        else:
            assert rowwise_rel_err(got, ref).max() <= ATTN_TOL, pps
        assert L.tickets_zero(ws), pps


@pytest.mark.parametrize("hq,hkv,d", [(40, 8, 128), (8, 2, 64)])
@pytest.mark.parametrize("mix", ["int4", "mixed"])
def test_split_counts_up_to_the_limit(hq, hkv, d, mix):
    """the merge at its widest: 512 pages of one sequence at 2 pages per split give the limit of
    256 splits (the (max, sum) pairs take four lanes' rounds, the partials several batches of a
    lane's run), 4 give 128, and 6 give 86 (a ragged last batch)"""
    case_banner(f"split-count limit hq={hq} hkv={hkv} d={d} {mix}")
    g = np.random.default_rng(d + len(mix))
    N = 512 * 16
    pages = synth.pages_for(N)
    tiers = [list(g.integers(0, 4, size=pages))] if mix == "mixed" else [[1] * pages]
    L = LayerPair(hq, hkv, d, 1, pages, tiers, seed=d + 7)
    L.write(synth.normal_f16(g, (1, N, hkv, d)), synth.normal_f16(g, (1, N, hkv, d)))
    q = synth.normal_f16(g, (1, hq, d))
    ref = L.oracle_attn(q)
    for pps in (2, 4, 6):
        got, ws = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} splits={-(-pages // pps)} max rel err {err.max():.3e}")
        assert err.max() <= ATTN_TOL, (pps, err.max())
        assert L.tickets_zero(ws), pps


@pytest.mark.parametrize("hq,hkv,d", [(40, 8, 128), (8, 2, 64)])
@pytest.mark.parametrize("mix", ["int2", "mixed"])
def test_splits_longer_than_a_wave_chunk_of_64_pages(hq, hkv, d, mix):
    """a caller's plan of more than 512 pages per split gives each of the eight waves more than
    64 pages, which the register-held handle chunk cannot hold: the wave then walks its pages
    through the general loop, reading handles from the table as it goes. 1100 pages (a ragged
    last page) at 1100 pages per split (one split, about 137 pages a wave) and at 520 (three
    splits), through the attention and through a fused step of three tokens"""
    case_banner(f"splits beyond 512 pages hq={hq} hkv={hkv} d={d} {mix}")
    g = np.random.default_rng(d + 3 * len(mix))
    N = 1100 * 16 - 5
    pages = synth.pages_for(N + 3)
    tiers = [list(g.integers(0, 4, size=pages))] if mix == "mixed" else [[0] * pages]
    L = LayerPair(hq, hkv, d, 1, pages, tiers, seed=d + 11)
    L.write(synth.normal_f16(g, (1, N, hkv, d)), synth.normal_f16(g, (1, N, hkv, d)))
    q = synth.normal_f16(g, (1, hq, d))
    ref = L.oracle_attn(q)
    for pps in (1100, 520):
        got, ws = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL, (pps, err.max())
        assert L.tickets_zero(ws), pps
    got, ws = L.step(synth.normal_f16(g, (1, 3, hkv, d)), synth.normal_f16(g, (1, 3, hkv, d)), q,
                     pages_per_split=1100)
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    err = rowwise_rel_err(got, L.oracle_attn(q))
    print(f"  fused step pps=1100 max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL
    assert L.tickets_zero(ws)


def test_many_short_sequences():
    """a wide batch of short, ragged sequences: 300 sequences of 0..120 tokens and 8 KV heads
    give 2400 (sequence, head) groups, one split each under the library's plan (and up to four
    at two pages a split), widths mixed per page; attention, a fused step and the canary against
    the oracle"""
    case_banner("300 short sequences")
    g = np.random.default_rng(300)
    B, hq, hkv, d = 300, 32, 8, 128
    lens = g.integers(0, 121, size=B)
    lens[:3] = (0, 1, 16)
    max_pages = 10
    tiers = [list(g.integers(0, 4, size=max_pages)) for _ in range(B)]
    L = LayerPair(hq, hkv, d, B, max_pages, tiers, seed=300)
    for s_, n in enumerate(lens):
        if n:
            L.write(synth.normal_f16(g, (1, int(n), hkv, d)), synth.normal_f16(g, (1, int(n), hkv, d)),
                    rows=[s_])
    q = synth.normal_f16(g, (B, hq, d))
    ref = L.oracle_attn(q)
    for pps in (0, 2):
        got, ws = L.attn(q, pages_per_split=pps)
        err = rowwise_rel_err(got, ref)
        print(f"  attn pps={pps} max rel err {err.max():.3e}", flush=True)
        assert err.max() <= ATTN_TOL and not got[lens == 0].any()
        assert L.tickets_zero(ws)
    got, ws = L.step(synth.normal_f16(g, (B, 3, hkv, d)), synth.normal_f16(g, (B, 3, hkv, d)), q)
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    err = rowwise_rel_err(got, L.oracle_attn(q))
    print(f"  fused step max rel err {err.max():.3e}", flush=True)
    assert err.max() <= ATTN_TOL and L.tickets_zero(ws)
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    assert np.abs(kl - okl).max() <= 1e-4 and np.abs(rows - orows).max() <= 1e-4


@pytest.mark.parametrize("R", [16, 48, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_ring_sizes(R, d):
    """the ring at the sizes the geometry allows besides 64: the write reads an open page's
    earlier keys from it (token by token, and in chunks longer than the ring), the canary
    quantizes its newest min(N, R) keys (the oldest fragment of a page included); bytes, ring,
    attention and canary against the oracle"""
    case_banner(f"ring R={R} d={d}")
    g = np.random.default_rng(R + d)
    lens = [3, 37, 150]
    max_pages = synth.pages_for(max(lens)) + 1
    tiers = [list(g.integers(0, 3, size=max_pages)) for _ in lens]
    L = LayerPair(8, 2, d, len(lens), max_pages, tiers, seed=R + d, R=R)
    for s, n in enumerate(lens):
        K = synth.normal_f16(g, (1, n, 2, d), np.where(np.arange(d) % 5 == 0, 8, 1).astype(np.float32))
        V = synth.normal_f16(g, (1, n, 2, d))
        p = 0
        for step in (1, 1, 1, 17, R + 5, 2 * R + 1):        # single tokens, then chunks past R
            m = min(step, n - p)
            if m <= 0:
                break
            L.write(K[:, p:p + m], V[:, p:p + m], rows=[s])
            p += m
        if p < n:
            L.write(K[:, p:n], V[:, p:n], rows=[s])
    bad, ring_ok = L.compare_bytes()
    assert not bad and ring_ok, bad[:3]
    q = synth.normal_f16(g, (len(lens), 8, d))
    got, _ = L.attn(q)
    assert rowwise_rel_err(got, L.oracle_attn(q)).max() <= ATTN_TOL
    kl, rows = L.canary(q)
    okl, orows = L.oracle_canary(q)
    print(f"  canary {kl} oracle {okl}")
    assert np.abs(kl - okl).max() <= KL_TOL and np.abs(rows - orows).max() <= KL_TOL
