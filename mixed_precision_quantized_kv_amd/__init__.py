"""Thin ctypes binding of libkvq (include/kv_quant.h), the MI355X mixed-precision quantized
KV-cache decode path. Names match the C ABI; this module only marshals arguments.

Device buffers are passed as torch tensors (their data_ptr()) or raw integer addresses; the
stream defaults to torch's current stream. Every nonzero status raises KVError with the
library's own message. The library is loaded on first use and its absence is an error: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "kv_quant.h")

KV_OK, KV_EINVAL, KV_ENOBLOCKS, KV_EUNSUPPORTED, KV_EHIP = range(5)
KV_NO_BLOCK = 0xFFFFFFFF
TIER_BITS = (2, 4, 8, 16)       # tier index -> bits (16 = plain FP16)
NUM_TIERS = 4


class KVError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class Geometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "ring_size",
        "max_seqs", "max_pages_per_seq", "asymmetric")]


class LayerPools(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p * NUM_TIERS), ("capacity", ctypes.c_uint32 * NUM_TIERS)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mixed_precision_quantized_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, u32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t
        G = ctypes.POINTER(Geometry)
        sigs = {
            "kv_abi_version": (i32, []),
            "kv_strerror": (ctypes.c_char_p, [i32]),
            "kv_last_error": (ctypes.c_char_p, []),
            "kv_validate": (i32, [G]),
            "kv_handle": (u32, [i32, u32]),
            "kv_block_bytes": (sz, [G, i32]),
            "kv_ring_bytes": (sz, [G]),
            "kv_cache_bytes_per_token": (ctypes.c_double, [G, P]),
            "kv_alloc_create": (i32, [G, P, P, ctypes.c_uint64, ctypes.POINTER(P)]),
            "kv_alloc_set_layer_bits": (i32, [P, i32, i32]),
            "kv_alloc_extend": (i32, [P, i32, ctypes.c_int32, P]),
            "kv_alloc_free_seq": (i32, [P, i32, P]),
            "kv_alloc_seq_len": (ctypes.c_int32, [P, i32]),
            "kv_alloc_free_blocks": (ctypes.c_int64, [P, i32, i32]),
            "kv_alloc_layer_bits": (i32, [P, i32]),
            "kv_alloc_destroy": (None, [P]),
            "kv_check_block_table": (i32, [P, P]),
            "kv_controller_tau": (ctypes.c_double, [ctypes.c_double] * 3),
            "kv_controller_create": (i32, [i32, P, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, ctypes.POINTER(P)]),
            "kv_controller_observe": (i32, [P, P, ctypes.c_double, P]),
            "kv_controller_set_frozen": (i32, [P, i32]),
            "kv_controller_state": (i32, [P, P, P, P]),
            "kv_controller_apply": (i32, [P, P]),
            "kv_controller_destroy": (None, [P]),
            "kv_quant_write": (i32, [G, ctypes.POINTER(LayerPools), P, P, i32, i32, P, P, P, P]),
            "kv_decode_workspace_bytes": (sz, [G, i32, i32, i32]),
            "kv_decode_pages_per_split": (i32, [G, i32, i32]),
            "kv_decode_pages_per_split_for": (i32, [G, i32, P]),
            "kv_decode_step_pages_per_split_for": (i32, [G, i32, P, i32]),
            "kv_decode_attn": (i32, [G, ctypes.POINTER(LayerPools), P, P, i32, i32, P,
                                     ctypes.c_float, P, P, sz, i32, P]),
            "kv_decode_step": (i32, [G, ctypes.POINTER(LayerPools), P, P, i32, i32, P, P, P, i32,
                                     P, ctypes.c_float, P, P, sz, i32, P]),
            "kv_canary_workspace_bytes": (sz, [G, i32]),
            "kv_canary_kl": (i32, [G, P, P, i32, P, ctypes.c_float, P, P, P, sz, P]),
            "kv_canary_kl_asym": (i32, [G, P, P, i32, P, ctypes.c_float, P, P, P, sz, P]),
            "kv_canary_layers_workspace_bytes": (sz, [G, i32, i32]),
            "kv_decode_step_noalloc": (i32, [G, ctypes.POINTER(LayerPools), P, P, i32, i32, P, P,
                                             P, i32, P, ctypes.c_float, P, i32, P]),
            "kv_canary_kl_layers": (i32, [G, i32, P, P, i32, P, ctypes.c_float, P, P, P, sz, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list:
    """Every function the public header declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(kv_[a-z_0-9]+)\s*\(", text)) - {"kv_alloc"})


def _check(status: int) -> None:
    if status != KV_OK:
        raise KVError(status, lib().kv_last_error().decode() or lib().kv_strerror(status).decode())


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):                    # numpy (host arrays)
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def geometry(num_layers, num_q_heads, num_kv_heads, head_dim, max_seqs, max_pages_per_seq,
             page_size=16, ring_size=64, asymmetric=False) -> Geometry:
    """asymmetric: the INT tiers hold a zero point and a scale per group (the asymmetric
    storage format of the header); the default is the symmetric format"""
    return Geometry(num_layers, num_q_heads, num_kv_heads, head_dim, page_size, ring_size,
                    max_seqs, max_pages_per_seq, int(bool(asymmetric)))


def layer_pools(bases, capacities) -> LayerPools:
    """pools of one layer; lists of three leave the FP16 pool empty"""
    p = LayerPools()
    for t in range(NUM_TIERS):
        p.base[t] = (_addr(bases[t]) or None) if t < len(bases) else None
        p.capacity[t] = int(capacities[t]) if t < len(capacities) else 0
    return p


# ------------------------------------------------------------------ sizes and validation
def kv_abi_version() -> int:
    return lib().kv_abi_version()


def kv_validate(g: Geometry) -> None:
    _check(lib().kv_validate(ctypes.byref(g)))


def kv_handle(bits: int, index: int) -> int:
    return lib().kv_handle(bits, index)


def kv_block_bytes(g: Geometry, bits: int) -> int:
    return lib().kv_block_bytes(ctypes.byref(g), bits)


def kv_ring_bytes(g: Geometry) -> int:
    return lib().kv_ring_bytes(ctypes.byref(g))


def kv_cache_bytes_per_token(g: Geometry, bits_per_layer) -> float:
    arr = (ctypes.c_int * len(bits_per_layer))(*bits_per_layer)
    return lib().kv_cache_bytes_per_token(ctypes.byref(g), arr)


def kv_decode_workspace_bytes(g: Geometry, batch: int, max_ctx_len: int, pages_per_split=0) -> int:
    return lib().kv_decode_workspace_bytes(ctypes.byref(g), batch, max_ctx_len, pages_per_split)


def kv_decode_pages_per_split(g: Geometry, batch: int, max_ctx_len: int) -> int:
    return lib().kv_decode_pages_per_split(ctypes.byref(g), batch, max_ctx_len)


def kv_decode_pages_per_split_for(g: Geometry, ctx_len_host) -> int:
    """split plan for known lengths (host int32 array, one per sequence)"""
    import numpy as np
    a = np.ascontiguousarray(ctx_len_host, dtype=np.int32)
    return lib().kv_decode_pages_per_split_for(ctypes.byref(g), int(a.size), a.ctypes.data)


def kv_decode_step_pages_per_split_for(g: Geometry, pos_host, n_new: int) -> int:
    """split plan of a fused step for known positions (host int32 array, one per sequence)"""
    import numpy as np
    a = np.ascontiguousarray(pos_host, dtype=np.int32)
    return lib().kv_decode_step_pages_per_split_for(ctypes.byref(g), int(a.size), a.ctypes.data,
                                                    int(n_new))


def kv_canary_workspace_bytes(g: Geometry, batch: int) -> int:
    return lib().kv_canary_workspace_bytes(ctypes.byref(g), batch)


# ------------------------------------------------------------------ allocator
class KVAlloc:
    """kv_alloc_* on a host block table bt_host [L][max_seqs][max_pages] (numpy uint32)."""

    def __init__(self, g: Geometry, capacity, bits, shuffle_seed: int = 0):
        import numpy as np
        self.g = g
        cap = np.asarray(capacity, dtype=np.uint32).reshape(g.num_layers, -1)
        if cap.shape[1] < NUM_TIERS:                # [L][3]: no FP16 pool
            cap = np.concatenate([cap, np.zeros((g.num_layers, NUM_TIERS - cap.shape[1]),
                                                dtype=np.uint32)], axis=1)
        cap = np.ascontiguousarray(cap).reshape(-1)
        b = np.ascontiguousarray(bits, dtype=np.int32)
        h = ctypes.c_void_p()
        _check(lib().kv_alloc_create(ctypes.byref(g), cap.ctypes.data, b.ctypes.data,
                                     shuffle_seed, ctypes.byref(h)))
        self.handle = h.value
        self.bt = np.full((g.num_layers, g.max_seqs, g.max_pages_per_seq), KV_NO_BLOCK,
                          dtype=np.uint32)

    def kv_alloc_set_layer_bits(self, layer: int, bits: int) -> None:
        _check(lib().kv_alloc_set_layer_bits(self.handle, layer, bits))

    def kv_alloc_extend(self, seq: int, new_len: int) -> None:
        _check(lib().kv_alloc_extend(self.handle, seq, new_len, self.bt.ctypes.data))

    def kv_alloc_free_seq(self, seq: int) -> None:
        _check(lib().kv_alloc_free_seq(self.handle, seq, self.bt.ctypes.data))

    def kv_alloc_seq_len(self, seq: int) -> int:
        return lib().kv_alloc_seq_len(self.handle, seq)

    def kv_alloc_free_blocks(self, layer: int, bits: int) -> int:
        return lib().kv_alloc_free_blocks(self.handle, layer, bits)

    def kv_alloc_layer_bits(self, layer: int) -> int:
        return lib().kv_alloc_layer_bits(self.handle, layer)

    def kv_check_block_table(self, bt=None) -> None:
        bt = self.bt if bt is None else bt
        _check(lib().kv_check_block_table(self.handle, bt.ctypes.data))

    def kv_alloc_destroy(self) -> None:
        if self.handle:
            lib().kv_alloc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.kv_alloc_destroy()
        except Exception:
            pass


# ------------------------------------------------------------------ controller (host)
def kv_controller_tau(tau0: float, l0: float, context_len: float) -> float:
    return lib().kv_controller_tau(tau0, l0, context_len)


class KVController:
    """kv_controller_*: canary readings [L][3] in, one width per layer out (host only)."""

    def __init__(self, initial_bits, alpha: float = 0.1, tau0: float = 0.022, l0: float = 4096.0):
        import numpy as np
        b = np.ascontiguousarray(initial_bits, dtype=np.int32)
        self.layers = int(b.size)
        h = ctypes.c_void_p()
        _check(lib().kv_controller_create(self.layers, b.ctypes.data, alpha, tau0, l0,
                                          ctypes.byref(h)))
        self.handle = h.value

    def kv_controller_observe(self, kl, context_len: float):
        import numpy as np
        k = np.ascontiguousarray(kl, dtype=np.float32).reshape(self.layers, 3)
        out = np.zeros(self.layers, dtype=np.int32)
        _check(lib().kv_controller_observe(self.handle, k.ctypes.data, float(context_len),
                                           out.ctypes.data))
        return out

    def kv_controller_set_frozen(self, frozen: bool) -> None:
        _check(lib().kv_controller_set_frozen(self.handle, int(bool(frozen))))

    def kv_controller_state(self):
        import numpy as np
        ema = np.zeros((self.layers, 3), dtype=np.float64)
        bits = np.zeros(self.layers, dtype=np.int32)
        n = ctypes.c_int64()
        _check(lib().kv_controller_state(self.handle, ema.ctypes.data, bits.ctypes.data,
                                         ctypes.byref(n)))
        return ema, bits, n.value

    def kv_controller_apply(self, alloc: "KVAlloc") -> None:
        _check(lib().kv_controller_apply(self.handle, alloc.handle))

    def kv_controller_destroy(self) -> None:
        if self.handle:
            lib().kv_controller_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.kv_controller_destroy()
        except Exception:
            pass


# ------------------------------------------------------------------ the three kernels
def kv_quant_write(g: Geometry, pools: LayerPools, bt, pos, batch: int, n_new: int, k_new, v_new,
                   ring, stream=None) -> None:
    _check(lib().kv_quant_write(ctypes.byref(g), ctypes.byref(pools), _addr(bt), _addr(pos), batch,
                                n_new, _addr(k_new), _addr(v_new), _addr(ring), _stream(stream)))


def kv_decode_attn(g: Geometry, pools: LayerPools, bt, ctx_len, batch: int, max_ctx_len: int, q,
                   softmax_scale: float, out, workspace, workspace_bytes=None,
                   pages_per_split: int = 0, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().kv_decode_attn(ctypes.byref(g), ctypes.byref(pools), _addr(bt), _addr(ctx_len),
                                batch, max_ctx_len, _addr(q), softmax_scale, _addr(out),
                                _addr(workspace), workspace_bytes, pages_per_split,
                                _stream(stream)))


def kv_decode_step(g: Geometry, pools: LayerPools, bt, pos, batch: int, n_new: int, k_new, v_new,
                   ring, max_ctx_len: int, q, softmax_scale: float, out, workspace,
                   workspace_bytes=None, pages_per_split: int = 0, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().kv_decode_step(ctypes.byref(g), ctypes.byref(pools), _addr(bt), _addr(pos), batch,
                                n_new, _addr(k_new), _addr(v_new), _addr(ring), max_ctx_len,
                                _addr(q), softmax_scale, _addr(out), _addr(workspace),
                                workspace_bytes, pages_per_split, _stream(stream)))


def kv_canary_kl(g: Geometry, ring, seq_len, batch: int, q, softmax_scale: float, kl_out,
                 kl_rows, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().kv_canary_kl(ctypes.byref(g), _addr(ring), _addr(seq_len), batch, _addr(q),
                              softmax_scale, _addr(kl_out), _addr(kl_rows), _addr(workspace),
                              workspace_bytes, _stream(stream)))


def kv_canary_kl_asym(g: Geometry, ring, seq_len, batch: int, q, softmax_scale: float, kl_out,
                      kl_rows, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().kv_canary_kl_asym(ctypes.byref(g), _addr(ring), _addr(seq_len), batch, _addr(q),
                                   softmax_scale, _addr(kl_out), _addr(kl_rows), _addr(workspace),
                                   workspace_bytes, _stream(stream)))


def kv_canary_layers_workspace_bytes(g: Geometry, num_layers: int, batch: int) -> int:
    return lib().kv_canary_layers_workspace_bytes(ctypes.byref(g), num_layers, batch)


def kv_canary_kl_layers(g: Geometry, rings, seq_len, batch: int, qs, softmax_scale: float, kl_out,
                        kl_rows, workspace, workspace_bytes=None, stream=None) -> None:
    """rings, qs: sequences of per-layer device tensors (or addresses); their addresses are passed
    as host arrays of device pointers"""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    n = len(rings)
    if len(qs) != n:
        raise ValueError("one q per ring")
    ring_ptrs = (ctypes.c_void_p * max(n, 1))(*[_addr(r) for r in rings])
    q_ptrs = (ctypes.c_void_p * max(n, 1))(*[_addr(q) for q in qs])
    _check(lib().kv_canary_kl_layers(ctypes.byref(g), n, ring_ptrs, _addr(seq_len), batch, q_ptrs,
                                     softmax_scale, _addr(kl_out), _addr(kl_rows), _addr(workspace),
                                     workspace_bytes, _stream(stream)))


def kv_decode_step_noalloc(g: Geometry, pools: LayerPools, bt, pos, batch: int, n_new: int, k_new,
                           v_new, ring, max_ctx_len: int, q, softmax_scale: float, out,
                           pages_per_split: int = 0, stream=None) -> None:
    _check(lib().kv_decode_step_noalloc(ctypes.byref(g), ctypes.byref(pools), _addr(bt), _addr(pos),
                                        batch, n_new, _addr(k_new), _addr(v_new), _addr(ring),
                                        max_ctx_len, _addr(q), softmax_scale, _addr(out),
                                        pages_per_split, _stream(stream)))
