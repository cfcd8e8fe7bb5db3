"""Host-side tests of the C ABI (no GPU work): exported symbols, argument validation, byte sizes,
and the block allocator (forward-only tiers, all-or-nothing growth, seeded shuffle).

EchoKV, "How EchoKV works": the tier vector routes future blocks to the right pool; "What
happens to old blocks...": already-allocated blocks keep their admit-time width.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

import mixed_precision_quantized_kv_amd as kvq

LIB = kvq.LIB_PATH


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(LIB):
        pytest.skip("libkvq.so not built (run __graft_entry__.build())")


def test_exports_every_header_symbol():
    names = kvq.header_symbols()
    assert len(names) >= 20
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = kvq.lib()
    for n in names:
        assert getattr(L, n) is not None
    assert kvq.kv_abi_version() == 3                  # the geometry carries the storage format


def geom(**kw):
    base = dict(num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=64, max_seqs=4,
                max_pages_per_seq=8)
    base.update(kw)
    return kvq.geometry(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), kvq.KV_EUNSUPPORTED),
    (dict(num_q_heads=9), kvq.KV_EINVAL),
    (dict(num_q_heads=34, num_kv_heads=2), kvq.KV_EUNSUPPORTED),
    (dict(ring_size=24), kvq.KV_EINVAL),
    (dict(ring_size=256), kvq.KV_EINVAL),
    (dict(page_size=32), kvq.KV_EUNSUPPORTED),
    (dict(max_seqs=0), kvq.KV_EINVAL),
])
def test_geometry_validation(kw, status):
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_validate(geom(**kw))
    assert e.value.status == status
    assert kvq.lib().kv_last_error().decode()


def test_format_flag_validation():
    g = geom()
    g.asymmetric = 2                      # the C struct field, past the binding's normalisation
    with pytest.raises(kvq.KVError) as e:
        kvq.kv_validate(g)
    assert e.value.status == kvq.KV_EINVAL and "asymmetric" in kvq.lib().kv_last_error().decode()
    assert kvq.kv_block_bytes(g, 4) == 0


def test_sizes_match_format():
    g = geom(head_dim=128, num_q_heads=40, num_kv_heads=8)
    # S_b = P*D*b/4 + 2D + 2P per KV head; the FP16 tier 4*P*D (keys and values, no scales)
    assert [kvq.kv_block_bytes(g, b) for b in (2, 4, 8)] == [8 * 1312, 8 * 2336, 8 * 4384]
    assert kvq.kv_block_bytes(g, 16) == 8 * 4 * 16 * 128
    assert kvq.kv_block_bytes(g, 3) == 0
    assert kvq.kv_ring_bytes(g) == 4 * 64 * 8 * 128 * 2
    assert kvq.kv_cache_bytes_per_token(g, [16, 16]) == 2 * 2 * 8 * 128 * 2
    assert kvq.kv_cache_bytes_per_token(g, [2, 8]) == 8 * (82 + 274)
    assert kvq.kv_handle(4, 7) == (1 << 30) | 7
    assert kvq.kv_handle(3, 7) == kvq.KV_NO_BLOCK
    assert kvq.kv_handle(16, 7) == (3 << 30) | 7
    # a layer at FP16 costs what the page's FP16 accounting says: 2 (K, V) * H_kv * D * 2 bytes
    assert kvq.kv_cache_bytes_per_token(g, [16, 16]) == 2 * kvq.kv_block_bytes(g, 16) / 16


def test_sizes_asymmetric_format():
    g = geom(head_dim=128, num_q_heads=40, num_kv_heads=8, asymmetric=True)
    # S_b = P*D*b/4 + 4D + 4P: a zero point beside every scale; the FP16 tier unchanged
    assert [kvq.kv_block_bytes(g, b) for b in (2, 4, 8)] == [8 * 1600, 8 * 2624, 8 * 4672]
    assert kvq.kv_block_bytes(g, 16) == 8 * 4 * 16 * 128
    assert kvq.kv_cache_bytes_per_token(g, [2, 8]) == 8 * (1600 + 4672) / 16


@pytest.mark.parametrize("asym", [False, True])
def test_sizes_agree_with_oracle(orc, asym):
    for hq, hkv, d in ((8, 2, 64), (40, 8, 128), (28, 4, 128)):
        g = geom(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, asymmetric=asym)
        og = orc.geom(hq, hkv, d, asymmetric=asym)
        for b in (2, 4, 8, 16):
            assert kvq.kv_block_bytes(g, b) == orc.block_bytes(og, b)
        bits = [2, 16]
        assert kvq.kv_cache_bytes_per_token(g, bits) == orc.cache_bytes_per_token(og, bits)


def test_kernel_calls_reject_bad_arguments_without_launching():
    g = geom()
    pools = kvq.layer_pools([0, 0, 0], [0, 0, 0])
    with pytest.raises(kvq.KVError) as e:           # NULL device pointers
        kvq.kv_quant_write(g, pools, 0, 0, 1, 1, 0, 0, 0, stream=0)
    assert e.value.status == kvq.KV_EINVAL
    with pytest.raises(kvq.KVError):                # batch beyond max_seqs
        kvq.kv_quant_write(g, pools, 16, 16, 5, 1, 16, 16, 16, stream=0)
    bad = kvq.layer_pools([8, 0, 0], [1, 0, 0])     # misaligned pool
    with pytest.raises(kvq.KVError):
        kvq.kv_decode_attn(g, bad, 256, 256, 1, 16, 256, 0.1, 256, 256, 1 << 20, 0, stream=0)
    need = kvq.kv_decode_workspace_bytes(g, 1, 100)
    assert need > 0
    with pytest.raises(kvq.KVError) as e:           # workspace too small
        kvq.kv_decode_attn(g, pools, 256, 256, 1, 100, 256, 0.1, 256, 256, need - 1, 0, stream=0)
    assert "workspace" in str(e.value)
    with pytest.raises(kvq.KVError):                # pages_per_split odd
        kvq.kv_decode_attn(g, pools, 256, 256, 1, 100, 256, 0.1, 256, 256, 1 << 20, 25, stream=0)
    with pytest.raises(kvq.KVError):                # context beyond the table
        kvq.kv_decode_attn(g, pools, 256, 256, 1, 8 * 16 + 1, 256, 0.1, 256, 256, 1 << 20, 0, stream=0)
    with pytest.raises(kvq.KVError):
        kvq.kv_canary_kl(g, 256, 256, 1, 256, 0.1, 256, None, 256, 4, stream=0)
    kvq.kv_quant_write(g, pools, 0, 0, 1, 0, 0, 0, 0, stream=0)   # n_new == 0: a no-op
    kvq.kv_quant_write(g, pools, 0, 0, 0, 1, 0, 0, 0, stream=0)   # batch == 0: a no-op
    for call in (lambda: kvq.kv_decode_attn(g, pools, 256, 256, 0, 16, 256, 0.1, 256, 256, 1 << 20, 0, stream=0),
                 lambda: kvq.kv_decode_step(g, pools, 256, 256, 0, 1, 256, 256, 256, 16, 256, 0.1, 256, 256,
                                            1 << 20, 0, stream=0),
                 lambda: kvq.kv_canary_kl(g, 256, 256, 0, 256, 0.1, 256, None, 256, 1 << 16, stream=0)):
        with pytest.raises(kvq.KVError) as e:       # attention and canary take 1..max_seqs rows
            call()
        assert e.value.status == kvq.KV_EINVAL and "batch 0" in str(e.value)
    need = kvq.kv_decode_workspace_bytes(g, 1, 16)
    cneed = kvq.kv_canary_workspace_bytes(g, 1)
    for bad_scale in (math.inf, -math.inf, math.nan):   # the scale must be finite, of either sign
        for call in (lambda: kvq.kv_decode_attn(g, pools, 256, 256, 1, 16, 256, bad_scale, 256, 256,
                                                need, 0, stream=0),
                     lambda: kvq.kv_decode_step(g, pools, 256, 256, 1, 1, 256, 256, 256, 16, 256,
                                                bad_scale, 256, 256, need, 0, stream=0),
                     lambda: kvq.kv_decode_step_noalloc(g, pools, 256, 256, 1, 1, 256, 256, 256, 16,
                                                        256, bad_scale, 256, 0, stream=0),
                     lambda: kvq.kv_canary_kl(g, 256, 256, 1, 256, bad_scale, 256, None, 256, cneed,
                                              stream=0),
                     lambda: kvq.kv_canary_kl_layers(g, [256], 256, 1, [256], bad_scale, 256, None,
                                                     256, kvq.kv_canary_layers_workspace_bytes(g, 1, 1),
                                                     stream=0)):
            with pytest.raises(kvq.KVError) as e:
                call()
            assert e.value.status == kvq.KV_EINVAL and "softmax_scale" in str(e.value)
    g600 = kvq.geometry(1, 8, 2, 64, 1, 600)
    ctx = 513 * 16                                  # 513 pages at 2 per split: 257 splits
    wsb = kvq.kv_decode_workspace_bytes(g600, 1, ctx, 2)
    with pytest.raises(kvq.KVError) as e:           # past the limit of 256 splits
        kvq.kv_decode_attn(g600, pools, 256, 256, 1, ctx, 256, 0.1, 256, 256, wsb, 2, stream=0)
    assert e.value.status == kvq.KV_EINVAL and "257 splits" in str(e.value)


def test_canary_layers_validation_and_workspace():
    """kv_canary_kl_layers: every layer's pointers are checked before anything is launched"""
    g = geom(num_layers=3)
    rows = 2 * 8 * 3 * 4                                          # batch 2 x 8 q heads x 3 widths
    assert kvq.kv_canary_workspace_bytes(g, 2) == 3 * 256 + rows
    # ticket lines for all three layers of the geometry, then the call's rows
    assert kvq.kv_canary_layers_workspace_bytes(g, 1, 2) == 3 * 3 * 256 + rows
    assert kvq.kv_canary_layers_workspace_bytes(g, 3, 2) == 3 * 3 * 256 + 3 * rows
    assert kvq.kv_canary_layers_workspace_bytes(g, 4, 2) == 0      # beyond the geometry's layers
    assert kvq.kv_canary_layers_workspace_bytes(g, 0, 2) == 0
    need = kvq.kv_canary_layers_workspace_bytes(g, 3, 2)
    ok = [256, 512, 768]
    for rings, qs, n, wsb in (
            (ok, ok, 4, need),                  # more layers than the geometry has
            (ok[:2], ok[:2], 0, need),          # no layers
            ([256, 0, 768], ok, 3, need),       # a NULL ring
            (ok, [256, 520, 768], 3, need),     # a misaligned q
            (ok, ok, 3, need - 1)):             # workspace too small
        with pytest.raises(kvq.KVError) as e:
            kvq.kv_canary_kl_layers(g, (rings * 2)[:n], 256, 2, (qs * 2)[:n], 0.1, 256, None, 256,
                                    wsb, stream=0)
        assert e.value.status == kvq.KV_EINVAL


def test_split_plan():
    g = geom(head_dim=128, num_q_heads=40, num_kv_heads=8, max_seqs=1, max_pages_per_seq=2100)
    pps = kvq.kv_decode_pages_per_split(g, 1, 32768)
    assert pps % 2 == 0 and pps >= 2
    assert -(-2048 // pps) * 8 >= 248            # about one workgroup per CU
    g4 = geom(max_seqs=1, max_pages_per_seq=9000)
    assert kvq.kv_decode_pages_per_split(g4, 1, 131072) * 256 >= 8192
    # many groups: one split each, capped so that a wave holds at most 64 pages
    g5 = geom(head_dim=128, num_q_heads=28, num_kv_heads=4, max_seqs=64, max_pages_per_seq=2100)
    assert kvq.kv_decode_pages_per_split(g5, 64, 32768) == 512


def test_split_plan_for_lengths():
    g = geom(head_dim=128, num_q_heads=40, num_kv_heads=8, max_seqs=1, max_pages_per_seq=2100)
    # equal (here: one) lengths: the plan for the longest length
    assert kvq.kv_decode_pages_per_split_for(g, [32768]) == kvq.kv_decode_pages_per_split(g, 1, 32768)
    g5 = geom(head_dim=128, num_q_heads=28, num_kv_heads=4, max_seqs=64, max_pages_per_seq=2100)
    lens = np.full(64, 20000, dtype=np.int32)
    lens[:3] = 20100
    assert kvq.kv_decode_pages_per_split_for(g5, lens) == kvq.kv_decode_pages_per_split(g5, 64, 20100)
    # ragged lengths: splits small enough that the batch makes about two workgroups per CU
    rng = np.random.default_rng(0)
    lens = np.round(np.exp(rng.uniform(np.log(1024), np.log(32768), 64))).astype(np.int32)
    pps = kvq.kv_decode_pages_per_split_for(g5, lens)
    pages = (lens + 15) // 16
    assert pps % 2 == 0 and 2 <= pps < kvq.kv_decode_pages_per_split(g5, 64, int(lens.max()))
    wgs = int(((pages + pps - 1) // pps).sum()) * 4
    assert 450 <= wgs <= 800, wgs
    assert -(-int(pages.max()) // pps) <= 256
    # invalid lengths
    assert kvq.kv_decode_pages_per_split_for(g5, np.array([-1] * 64, np.int32)) == 0
    assert kvq.kv_decode_pages_per_split_for(g5, np.array([2100 * 16 + 1] + [5] * 63, np.int32)) == 0
    assert kvq.kv_decode_pages_per_split_for(g5, np.zeros(65, np.int32)) == 0   # batch > max_seqs


def test_split_plan_for_fused_step():
    def splits(pages, pps):
        return -(-pages // pps)
    # 8 sequences at 8K + 1: the uniform plan leaves the writing (last) split nearly full
    g2 = geom(head_dim=128, num_q_heads=32, num_kv_heads=8, max_seqs=8, max_pages_per_seq=600)
    pos = np.full(8, 8192, dtype=np.int32)
    base = kvq.kv_decode_pages_per_split_for(g2, pos + 1)
    pps = kvq.kv_decode_step_pages_per_split_for(g2, pos, 1)
    pages = (8192 + 1 + 15) // 16
    assert pps % 2 == 0 and pps > base
    assert splits(pages, pps) == splits(pages, base)             # same grid
    last = pages - (splits(pages, pps) - 1) * pps
    assert 1 <= last <= pps - min(40, base // 2)
    # a step that writes nothing, or a last split already short, keeps the attention plan
    assert kvq.kv_decode_step_pages_per_split_for(g2, pos, 0) == kvq.kv_decode_pages_per_split_for(g2, pos)
    g3 = geom(head_dim=128, num_q_heads=40, num_kv_heads=8, max_seqs=1, max_pages_per_seq=2100)
    assert (kvq.kv_decode_step_pages_per_split_for(g3, [32768], 1)
            == kvq.kv_decode_pages_per_split_for(g3, [32769]))
    # sequences ending in different splits keep the plan for their lengths
    pos2 = np.array([8192, 2000, 8192, 8192, 8192, 8192, 8192, 8192], dtype=np.int32)
    assert (kvq.kv_decode_step_pages_per_split_for(g2, pos2, 1)
            == kvq.kv_decode_pages_per_split_for(g2, pos2 + 1))
    # the workspace for the plan of max_ctx_len covers the step's plan (same split count)
    assert (kvq.kv_decode_workspace_bytes(g2, 8, 8193, pps)
            <= kvq.kv_decode_workspace_bytes(g2, 8, 8193, 0))
    # invalid arguments
    assert kvq.kv_decode_step_pages_per_split_for(g2, pos, 65) == 0
    # 64 new tokens touch up to five pages, written in three rounds: a larger reserve
    pps64 = kvq.kv_decode_step_pages_per_split_for(g2, pos - 63, 64)
    assert pps64 >= pps and splits(pages, pps64) == splits(pages, base)
    assert kvq.kv_decode_step_pages_per_split_for(g2, pos, -1) == 0
    assert kvq.kv_decode_step_pages_per_split_for(g2, np.full(8, -2, np.int32), 1) == 0


# ------------------------------------------------------------------ allocator
def make_alloc(bits=(4, 8), cap=16, seed=1, **kw):
    g = geom(num_layers=len(bits), **kw)
    capacity = np.full((len(bits), 3), cap, dtype=np.uint32)
    return kvq.KVAlloc(g, capacity, list(bits), seed)


def test_extend_assigns_current_tier_and_checks():
    a = make_alloc()
    a.kv_alloc_extend(0, 40)                   # 3 pages per layer
    assert a.kv_alloc_seq_len(0) == 40
    for l, b in enumerate((4, 8)):
        row = a.bt[l, 0]
        assert all(int(h) >> 30 == {2: 0, 4: 1, 8: 2}[b] for h in row[:3])
        assert np.all(row[3:] == kvq.KV_NO_BLOCK)
        assert a.kv_alloc_free_blocks(l, b) == 13
    a.kv_check_block_table()


def test_fp16_layers_start_in_their_own_pool():
    g = geom(num_layers=2)
    capacity = np.full((2, 4), 8, dtype=np.uint32)          # INT2, INT4, INT8, FP16 pools
    a = kvq.KVAlloc(g, capacity, [16, 8], 3)
    a.kv_alloc_extend(0, 20)                                 # two pages per layer
    assert [int(h) >> 30 for h in a.bt[0, 0, :2]] == [3, 3]
    assert [int(h) >> 30 for h in a.bt[1, 0, :2]] == [2, 2]
    assert a.kv_alloc_free_blocks(0, 16) == 6
    a.kv_alloc_set_layer_bits(0, 4)                          # the canary has fired
    a.kv_alloc_extend(0, 50)
    assert [int(h) >> 30 for h in a.bt[0, 0, :4]] == [3, 3, 1, 1]
    a.kv_check_block_table()
    a.kv_alloc_free_seq(0)
    assert a.kv_alloc_free_blocks(0, 16) == 8 and a.kv_alloc_free_blocks(0, 4) == 8
    # [L][3] capacities (no FP16 pool): an FP16 layer has no blocks to give
    b = make_alloc(bits=(16, 4))
    with pytest.raises(kvq.KVError) as e:
        b.kv_alloc_extend(0, 1)
    assert e.value.status == kvq.KV_ENOBLOCKS


def test_tier_switch_is_forward_only():
    a = make_alloc()
    a.kv_alloc_extend(0, 20)                   # pages 0, 1 at INT4 (page 1 open)
    before = a.bt.copy()
    a.kv_alloc_set_layer_bits(0, 2)
    assert a.kv_alloc_layer_bits(0) == 2
    a.kv_alloc_extend(0, 32)                   # still page 1: nothing new
    assert np.array_equal(a.bt, before)
    a.kv_alloc_extend(0, 70)                   # pages 2..4 come from the INT2 pool
    assert np.array_equal(a.bt[0, 0, :2], before[0, 0, :2])
    assert all(int(h) >> 30 == 0 for h in a.bt[0, 0, 2:5])
    assert all(int(h) >> 30 == 2 for h in a.bt[1, 0, :5])
    a.kv_check_block_table()


def test_exhaustion_is_all_or_nothing():
    a = make_alloc(cap=4)
    a.kv_alloc_extend(0, 48)                   # 3 of 4 blocks
    snap = a.bt.copy()
    with pytest.raises(kvq.KVError) as e:
        a.kv_alloc_extend(1, 40)               # needs 3, only 1 left
    assert e.value.status == kvq.KV_ENOBLOCKS
    assert np.array_equal(a.bt, snap)
    assert a.kv_alloc_seq_len(1) == 0
    assert a.kv_alloc_free_blocks(0, 4) == 1
    a.kv_alloc_extend(1, 16)
    a.kv_alloc_free_seq(0)
    assert np.all(a.bt[:, 0] == kvq.KV_NO_BLOCK)
    assert a.kv_alloc_free_blocks(0, 4) == 3
    a.kv_alloc_extend(0, 48)                   # freed blocks are reused
    a.kv_check_block_table()


def test_shuffle_is_seeded_and_a_permutation():
    a1, a2, a3 = (make_alloc(seed=sd, max_pages_per_seq=16) for sd in (7, 7, 8))
    for a in (a1, a2, a3):
        a.kv_alloc_extend(0, 256)              # all 16 blocks
    assert np.array_equal(a1.bt, a2.bt)
    assert not np.array_equal(a1.bt, a3.bt)
    idx = sorted(int(h) & 0x3FFFFFFF for h in a1.bt[0, 0, :16])
    assert idx == list(range(16))


def test_check_block_table_catches_corruption():
    a = make_alloc()
    a.kv_alloc_extend(0, 40)
    a.kv_alloc_extend(1, 40)
    bad = a.bt.copy()
    bad[0, 1, 0] = bad[0, 0, 0]                # one block used twice
    with pytest.raises(kvq.KVError):
        a.kv_check_block_table(bad)
    bad = a.bt.copy()
    bad[0, 0, 5] = 3                           # handle past the sequence length
    with pytest.raises(kvq.KVError):
        a.kv_check_block_table(bad)
    bad = a.bt.copy()
    bad[1, 0, 0] = (2 << 30) | 99              # index beyond capacity
    with pytest.raises(kvq.KVError):
        a.kv_check_block_table(bad)


def test_check_block_table_catches_swapped_handles():
    """two sequences' valid, distinct handles exchanged: every handle is still valid and used
    once, but neither is the one handed out for that page"""
    a = make_alloc()
    a.kv_alloc_extend(0, 40)
    a.kv_alloc_extend(1, 40)
    bad = a.bt.copy()
    bad[1, 0, 2], bad[1, 1, 2] = a.bt[1, 1, 2], a.bt[1, 0, 2]
    with pytest.raises(kvq.KVError) as e:
        a.kv_check_block_table(bad)
    assert "handed out" in str(e.value)


def test_free_returns_the_allocators_own_blocks_whatever_the_table_holds():
    """a table edited after the blocks were handed out (here: one handle copied over another)
    cannot make the free return a block twice: the pools come back to their capacity and later
    sequences still get distinct blocks"""
    a = make_alloc(cap=8)
    a.kv_alloc_extend(0, 48)
    a.kv_alloc_extend(1, 32)
    a.bt[0, 0, 1] = a.bt[0, 0, 0]               # corrupt seq 0's row in layer 0
    a.kv_alloc_free_seq(0)
    assert np.all(a.bt[:, 0] == kvq.KV_NO_BLOCK)
    assert a.kv_alloc_free_blocks(0, 4) == 6 and a.kv_alloc_free_blocks(1, 8) == 6
    a.kv_alloc_free_seq(1)
    assert a.kv_alloc_free_blocks(0, 4) == 8 and a.kv_alloc_free_blocks(1, 8) == 8
    a.kv_alloc_extend(0, 64)
    a.kv_alloc_extend(1, 64)                    # all 8 blocks of each pool
    a.kv_check_block_table()
    for l in range(2):
        idx = sorted(int(h) & 0x3FFFFFFF for h in a.bt[l, :2, :4].ravel())
        assert idx == list(range(8))


def test_extend_argument_errors():
    a = make_alloc()
    with pytest.raises(kvq.KVError):
        a.kv_alloc_extend(9, 10)
    a.kv_alloc_extend(0, 30)
    with pytest.raises(kvq.KVError):
        a.kv_alloc_extend(0, 10)               # shrinking
    with pytest.raises(kvq.KVError):
        a.kv_alloc_extend(0, 8 * 16 + 1)       # beyond max_pages_per_seq
    with pytest.raises(kvq.KVError):
        a.kv_alloc_set_layer_bits(0, 3)
