"""Python loader for the plain CPU oracle (kvq_oracle.c).

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package. The product library never does; the two share no code.

Every wrapper takes and returns numpy arrays; fp16 values travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")

TIER_BITS = (2, 4, 8, 16)


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class Geom(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("page_size", ctypes.c_int),
                ("ring_size", ctypes.c_int), ("asymmetric", ctypes.c_int)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i, f, d, sz = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
        sigs = {
            "orc_f16_to_f64": (d, [ctypes.c_uint16]),
            "orc_f64_to_f16_rne": (ctypes.c_uint16, [d]),
            "orc_f64_to_f16_ru": (ctypes.c_uint16, [d]),
            "orc_quantize_group": (None, [P, i, ctypes.c_ssize_t, i, P, P]),
            "orc_quantize_group_asym": (None, [P, i, ctypes.c_ssize_t, i, P, P, P]),
            "orc_pack": (None, [P, i, i, P]),
            "orc_unpack": (None, [P, i, i, P]),
            "orc_bits_of_tier": (i, [i]),
            "orc_section_bytes": (sz, [P, i]),
            "orc_block_bytes": (sz, [P, i]),
            "orc_k_code": (i, [P, P, i, i, i]),
            "orc_v_code": (i, [P, P, i, i, i]),
            "orc_k_scale": (d, [P, P, i, i]),
            "orc_v_scale": (d, [P, P, i, i]),
            "orc_k_zero": (d, [P, P, i, i]),
            "orc_v_zero": (d, [P, P, i, i]),
            "orc_quant_write": (i, [P, P, P, i, P, i, i, P, P, P]),
            "orc_dequant_kv": (i, [P, P, P, i, i, P, P]),
            "orc_decode_attn": (i, [P, P, P, i, P, i, P, f, P]),
            "orc_decode_attn_row": (i, [P, P, P, i, P, i, f, P]),
            "orc_canary_kl": (None, [P, P, P, i, P, f, P, P]),
            "orc_canary_kl_mode": (None, [P, P, P, i, P, f, i, P, P]),
            "orc_kl_logits": (d, [P, P, i]),
            "orc_cache_bytes_per_token": (d, [P, i, P]),
            "orc_ring_bytes": (d, [P, i]),
            "orc_num_threads": (i, []),
            "orc_set_num_threads": (None, [i]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def geom(num_q_heads, num_kv_heads, head_dim, page_size=16, ring_size=64,
         asymmetric=False) -> Geom:
    """asymmetric: the cache's INT tiers hold zero point + scale per group (the asymmetric
    storage format); the default is the symmetric format"""
    return Geom(num_q_heads, num_kv_heads, head_dim, page_size, ring_size, int(bool(asymmetric)))


class Pools:
    """Host byte arrays for the four tier pools of one layer (INT2, INT4, INT8, FP16); a
    capacity list of three leaves the FP16 pool empty."""

    def __init__(self, g: Geom, capacity):
        cap = [int(c) for c in capacity] + [0] * (4 - len(capacity))
        self.capacity = cap
        self.arrays = [np.zeros(max(1, cap[t] * block_bytes(g, TIER_BITS[t])), dtype=np.uint8)
                       for t in range(4)]
        self._ptrs = (ctypes.c_void_p * 4)(*[a.ctypes.data for a in self.arrays])

    @property
    def ptr(self):
        return self._ptrs


# ---- fp16 ----
def f16_to_f64(h: int) -> float:
    return lib().orc_f16_to_f64(int(h))


def f64_to_f16_rne(x: float) -> int:
    return lib().orc_f64_to_f16_rne(float(x))


def f64_to_f16_ru(x: float) -> int:
    return lib().orc_f64_to_f16_ru(float(x))


# ---- quantizer / packing ----
def quantize_group(x_bits: np.ndarray, bits: int):
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.zeros(x.size, dtype=np.int32)
    scale = np.zeros(1, dtype=np.uint16)
    lib().orc_quantize_group(_ptr(x), x.size, 1, bits, _ptr(scale), _ptr(codes))
    return int(scale[0]), codes


def quantize_group_asym(x_bits: np.ndarray, bits: int):
    """asymmetric quantizer over one group: (scale bits, zero-point bits, codes in [0, 2^b-1])"""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.zeros(x.size, dtype=np.int32)
    scale = np.zeros(1, dtype=np.uint16)
    zero = np.zeros(1, dtype=np.uint16)
    lib().orc_quantize_group_asym(_ptr(x), x.size, 1, bits, _ptr(scale), _ptr(zero), _ptr(codes))
    return int(scale[0]), int(zero[0]), codes


def _whole_words(n: int, bits: int) -> None:
    # the format packs codes into 32-bit words (32 / bits codes a word)
    if n % (32 // bits):
        raise ValueError(f"{n} codes of {bits} bits do not fill whole 32-bit words")


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int32)
    _whole_words(q.size, bits)
    out = np.zeros(q.size * bits // 8, dtype=np.uint8)
    lib().orc_pack(_ptr(q), q.size, bits, _ptr(out))
    return out


def unpack(b: np.ndarray, n: int, bits: int) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    _whole_words(n, bits)
    if b.size < n * bits // 8:
        raise ValueError(f"{b.size} bytes hold fewer than {n} codes of {bits} bits")
    q = np.zeros(n, dtype=np.int32)
    lib().orc_unpack(_ptr(b), n, bits, _ptr(q))
    return q


def section_bytes(g: Geom, bits: int) -> int:
    return lib().orc_section_bytes(ctypes.byref(g), bits)


def block_bytes(g: Geom, bits: int) -> int:
    return lib().orc_block_bytes(ctypes.byref(g), bits)


def k_code(g, sec: np.ndarray, bits, t, c):
    return lib().orc_k_code(ctypes.byref(g), _ptr(sec), bits, t, c)


def v_code(g, sec: np.ndarray, bits, t, c):
    return lib().orc_v_code(ctypes.byref(g), _ptr(sec), bits, t, c)


def k_scale(g, sec: np.ndarray, bits, c):
    return lib().orc_k_scale(ctypes.byref(g), _ptr(sec), bits, c)


def v_scale(g, sec: np.ndarray, bits, t):
    return lib().orc_v_scale(ctypes.byref(g), _ptr(sec), bits, t)


def k_zero(g, sec: np.ndarray, bits, c):
    return lib().orc_k_zero(ctypes.byref(g), _ptr(sec), bits, c)


def v_zero(g, sec: np.ndarray, bits, t):
    return lib().orc_v_zero(ctypes.byref(g), _ptr(sec), bits, t)


# ---- the three path operations ----
def _check_pages(g: Geom, pools: Pools, bt: np.ndarray, first: np.ndarray, end: np.ndarray,
                 what: str) -> None:
    """every page p in [first[s], end[s]) of row s lies in the table and holds a handle of a
    block its pool has, so that the C code never reaches outside the host arrays"""
    for s in range(bt.shape[0]):
        if end[s] <= first[s]:
            continue
        if first[s] < 0 or end[s] > bt.shape[1]:
            raise ValueError(f"{what}: row {s} pages {first[s]}..{end[s] - 1} outside the table")
        h = bt[s, first[s]:end[s]].astype(np.int64)
        tier, idx = h >> 30, h & 0x3FFFFFFF
        cap = np.array(pools.capacity, dtype=np.int64)[tier]
        if (h == 0xFFFFFFFF).any() or (idx >= cap).any():
            raise ValueError(f"{what}: row {s} has a page without a block of its pool")


def quant_write(g: Geom, pools: Pools, bt: np.ndarray, pos: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, ring: np.ndarray) -> None:
    """In place on pools and ring. bt [B][max_pages] uint32; k_new/v_new [B][n][Hkv][D] uint16."""
    bt = np.ascontiguousarray(bt, dtype=np.uint32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    assert ring.dtype == np.uint16 and ring.flags["C_CONTIGUOUS"]
    B, n = k_new.shape[0], k_new.shape[1]
    hd = (g.num_kv_heads, g.head_dim)
    if k_new.shape[2:] != hd or v_new.shape != k_new.shape or pos.shape != (B,) or \
            bt.shape[0] < B or ring.shape[0] < B or ring.shape[1:] != (g.ring_size,) + hd:
        raise ValueError("oracle write: shapes do not match the geometry")
    P = g.page_size
    _check_pages(g, pools, bt[:B], pos // P, (pos + n + P - 1) // P if n else pos // P,
                 "oracle write")
    rc = lib().orc_quant_write(ctypes.byref(g), pools.ptr, _ptr(bt), bt.shape[1], _ptr(pos), B, n,
                               _ptr(k_new), _ptr(v_new), _ptr(ring))
    if rc != 0:
        raise ValueError("oracle write: invalid block handle or page out of range")


def dequant_kv(g: Geom, pools: Pools, bt_row: np.ndarray, n: int, kv: int):
    bt_row = np.ascontiguousarray(bt_row, dtype=np.uint32)
    K = np.zeros((n, g.head_dim), dtype=np.float64)
    V = np.zeros((n, g.head_dim), dtype=np.float64)
    rc = lib().orc_dequant_kv(ctypes.byref(g), pools.ptr, _ptr(bt_row), n, kv, _ptr(K), _ptr(V))
    if rc != 0:
        raise ValueError("oracle dequant: invalid block handle")
    return K, V


def decode_attn(g: Geom, pools: Pools, bt: np.ndarray, ctx_len: np.ndarray, q: np.ndarray,
                softmax_scale: float) -> np.ndarray:
    bt = np.ascontiguousarray(bt, dtype=np.uint32)
    ctx_len = np.ascontiguousarray(ctx_len, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B = q.shape[0]
    if q.shape[1:] != (g.num_q_heads, g.head_dim) or ctx_len.shape != (B,) or bt.shape[0] < B:
        raise ValueError("oracle attention: shapes do not match the geometry")
    _check_pages(g, pools, bt[:B], np.zeros(B, np.int64), (ctx_len + g.page_size - 1) // g.page_size,
                 "oracle attention")
    out = np.zeros((B, g.num_q_heads, g.head_dim), dtype=np.float64)
    rc = lib().orc_decode_attn(ctypes.byref(g), pools.ptr, _ptr(bt), bt.shape[1], _ptr(ctx_len), B,
                               _ptr(q), float(softmax_scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attention: invalid block handle")
    return out


def decode_attn_row(g: Geom, pools: Pools, bt_row: np.ndarray, ctx_len: int, q_row: np.ndarray,
                    h: int, softmax_scale: float) -> np.ndarray:
    bt_row = np.ascontiguousarray(bt_row, dtype=np.uint32)
    q_row = np.ascontiguousarray(q_row, dtype=np.uint16)
    out = np.zeros(g.head_dim, dtype=np.float64)
    rc = lib().orc_decode_attn_row(ctypes.byref(g), pools.ptr, _ptr(bt_row), int(ctx_len),
                                   _ptr(q_row), int(h), float(softmax_scale), _ptr(out))
    if rc != 0:
        raise ValueError("oracle attention row: invalid block handle")
    return out


def canary_kl(g: Geom, ring: np.ndarray, seq_len: np.ndarray, q: np.ndarray,
              softmax_scale: float, asymmetric=None):
    """asymmetric None: the cache's own quantizer (the geometry's format); True / False force
    the asymmetric or the symmetric copies"""
    if asymmetric is None:
        asymmetric = bool(g.asymmetric)
    ring = np.ascontiguousarray(ring, dtype=np.uint16)
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int32)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    B = q.shape[0]
    kl3 = np.zeros(3, dtype=np.float64)
    rows = np.zeros((B, g.num_q_heads, 3), dtype=np.float64)
    lib().orc_canary_kl_mode(ctypes.byref(g), _ptr(ring), _ptr(seq_len), B, _ptr(q),
                             float(softmax_scale), int(bool(asymmetric)), _ptr(kl3), _ptr(rows))
    return kl3, rows


def kl_logits(l: np.ndarray, m: np.ndarray) -> float:
    l = np.ascontiguousarray(l, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float64)
    return lib().orc_kl_logits(_ptr(l), _ptr(m), l.size)


def cache_bytes_per_token(g: Geom, bits_per_layer) -> float:
    b = np.ascontiguousarray(bits_per_layer, dtype=np.int32)
    return lib().orc_cache_bytes_per_token(ctypes.byref(g), b.size, _ptr(b))


def ring_bytes(g: Geom, num_layers: int) -> float:
    return lib().orc_ring_bytes(ctypes.byref(g), num_layers)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))
