"""Thin ctypes binding over libpa.so (include/pa.h).  Argument marshalling only.

Every function keeps the C name.  Device arguments are torch tensors on the GPU
(PyTorch supplies device memory and streams); pool arguments are host values.
If libpa.so is missing or fails to load, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_OOM, PA_ERR_HIP = range(6)
PA_F32, PA_F16, PA_BF16, PA_I8, PA_FP8 = 0, 1, 2, 3, 4
PA_KERNEL_AUTO, PA_KERNEL_VALU, PA_KERNEL_MFMA = 0, 1, 2
PA_PARTITION_BALANCED = -1      # partition_tokens value: the balanced split
KERNELS = {"auto": PA_KERNEL_AUTO, "valu": PA_KERNEL_VALU, "mfma": PA_KERNEL_MFMA}
BLOCK_SIZE = 16
PA_NOALLOC_WORKSPACE_BYTES = 64 << 20   # the per-device workspace of pa_decode_noalloc

_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[pa status {status}] {msg}")
        self.status = status


class PaOutOfBlocks(PaError):
    pass


class pa_decode_params(ctypes.Structure):
    _fields_ = [("out", _P), ("q", _P), ("k_cache", _P), ("v_cache", _P),
                ("block_tables", _P), ("context_lens", _P),
                ("num_seqs", _I32), ("num_q_heads", _I32), ("num_kv_heads", _I32),
                ("head_dim", _I32), ("max_blocks_per_seq", _I32), ("num_blocks", _I32),
                ("max_context_len", _I32), ("scale", ctypes.c_float), ("kv_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("partition_tokens", _I32), ("kernel", ctypes.c_int),
                ("k_new", _P), ("v_new", _P), ("slot_mapping", _P),
                ("q_dtype", ctypes.c_int),
                ("start_event", _P), ("stop_event", _P), ("sliding_window", _I32),
                ("shared_prefix_blocks", _I32)]


class pa_extend_params(ctypes.Structure):
    _fields_ = [("out", _P), ("q", _P), ("k_cache", _P), ("v_cache", _P),
                ("block_tables", _P), ("context_lens", _P), ("query_start", _P),
                ("num_seqs", _I32), ("num_query_rows", _I32), ("num_q_heads", _I32),
                ("num_kv_heads", _I32), ("head_dim", _I32), ("max_blocks_per_seq", _I32),
                ("num_blocks", _I32), ("max_context_len", _I32), ("max_query_len", _I32),
                ("scale", ctypes.c_float), ("kv_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("partition_tokens", _I32), ("start_event", _P), ("stop_event", _P)]


_lib = None


def use_library(path: str) -> None:
    """Loads the library from `path` instead of libpa.so (the traced build,
    libpa_trace.so, for a per-wave timeline); call before anything else here."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("the library is already loaded")
    LIB_PATH = path


def lib():
    """Loads libpa.so once; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m paged_kv_cache_65_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "pa_version": (ctypes.c_char_p, []),
            "pa_last_error": (ctypes.c_char_p, []),
            "pa_decode_partition_tokens": (_I32, [ctypes.POINTER(pa_decode_params)]),
            "pa_decode_workspace_bytes": (_SZ, [ctypes.POINTER(pa_decode_params)]),
            "pa_decode": (ctypes.c_int, [ctypes.POINTER(pa_decode_params), _P, _SZ, _P]),
            "pa_decode_partitions": (ctypes.c_int, [ctypes.POINTER(pa_decode_params), _P, _SZ, _P]),
            "pa_decode_merge": (ctypes.c_int, [ctypes.POINTER(pa_decode_params), _P, _SZ, _P]),
            "pa_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(pa_decode_params), _P]),
            "pa_extend_partition_tokens": (_I32, [ctypes.POINTER(pa_extend_params)]),
            "pa_extend_workspace_bytes": (_SZ, [ctypes.POINTER(pa_extend_params)]),
            "pa_extend": (ctypes.c_int, [ctypes.POINTER(pa_extend_params), _P, _SZ, _P]),
            "pa_reshape_and_cache": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                    ctypes.c_int, _P]),
            "pa_copy_blocks": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, ctypes.c_int, _P]),
            "pa_reshape_and_cache_int8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                         ctypes.c_int, _P]),
            "pa_copy_blocks_int8": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P]),
            "pa_reshape_and_cache_fp8": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                        ctypes.c_int, _P]),
            "pa_swap_blocks": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32,
                                              ctypes.c_int, _P]),
            "pa_swap_blocks_int8": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _P, _I32, _I32, _I32, _P]),
            "pa_seq_swap_out": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32]),
            "pa_seq_swap_in": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32]),
            "pa_seq_swapped_blocks": (_I32, [_P, _I32]),
            "pa_block_pool_create": (ctypes.c_int, [_I32, _I32, _PI32, ctypes.POINTER(_P)]),
            "pa_block_pool_destroy": (None, [_P]),
            "pa_block_pool_num_blocks": (_I32, [_P]),
            "pa_block_pool_num_free": (_I32, [_P]),
            "pa_block_pool_refcount": (_I32, [_P, _I32]),
            "pa_block_pool_free_list": (_I32, [_P, _PI32, _I32]),
            "pa_block_pool_alloc": (ctypes.c_int, [_P, _PI32]),
            "pa_block_pool_incref": (ctypes.c_int, [_P, _I32]),
            "pa_block_pool_decref": (ctypes.c_int, [_P, _I32]),
            "pa_seq_create": (ctypes.c_int, [_P, _PI32]),
            "pa_seq_fork": (ctypes.c_int, [_P, _I32, _PI32]),
            "pa_seq_append": (ctypes.c_int, [_P, _I32, _I32, _PI64, _PI32, _PI32]),
            "pa_seq_append_batch": (ctypes.c_int, [_P, _PI32, _I32, _PI64, _PI32, _PI32]),
            "pa_seq_free": (ctypes.c_int, [_P, _I32]),
            "pa_seq_num_tokens": (_I32, [_P, _I32]),
            "pa_seq_export": (ctypes.c_int, [_P, _PI32, _I32, _I32, _PI32, _PI32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != PA_OK:
        msg = lib().pa_last_error().decode()
        raise (PaOutOfBlocks if status == PA_ERR_OOM else PaError)(status, msg)


def pa_version() -> str:
    return lib().pa_version().decode()


# ---------------------------------------------------------------- device calls
def _dtype_code(t) -> int:
    import torch
    # an FP8 (E4M3) cache holds its codes in uint8 (or float8_e4m3fn) tensors
    codes = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.int8: PA_I8,
             torch.uint8: PA_FP8}
    if hasattr(torch, "float8_e4m3fn"):
        codes[torch.float8_e4m3fn] = PA_FP8
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dev(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _gpu_addressable(t):
    """A device tensor, or a pinned host tensor (the GPU addresses it directly)."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError("expected a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def block_elems(cache, num_kv_heads, head_dim) -> int:
    """Elements of one block of a cache tensor: a byte cache (int8 / uint8 /
    float8 codes) holds its 16 row scales in every tile (16*(D+4) bytes)."""
    return num_kv_heads * BLOCK_SIZE * (head_dim + 4 if cache.element_size() == 1 else head_dim)


def make_decode_params(out, q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                       max_context_len, scale, partition_tokens=0, kernel="auto", k_new=None,
                       v_new=None, slot_mapping=None, start_event=None, stop_event=None,
                       sliding_window=0, shared_prefix_blocks=0):
    """start_event / stop_event: raw hipEvent_t handles (ints) or None.
    sliding_window: W > 0 attends positions L-1-W .. L-1 only; 0 = the whole context."""
    S, Hq, D = q.shape
    nb = k_cache.numel() // block_elems(k_cache, num_kv_heads, D)
    return pa_decode_params(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        S, Hq, num_kv_heads, D, block_tables.shape[1] if block_tables.dim() == 2 else 0, nb,
        int(max_context_len), float(scale), _dtype_code(k_cache), _dtype_code(out),
        int(partition_tokens), KERNELS[kernel], _dev(k_new), _dev(v_new), _dev(slot_mapping),
        _dtype_code(q), _event(start_event), _event(stop_event),
        int(sliding_window), int(shared_prefix_blocks))


def _event(ev):
    if ev is None:
        return None
    return int(ev.value if isinstance(ev, ctypes.c_void_p) else ev)


def pa_decode_workspace_bytes(params: pa_decode_params) -> int:
    return lib().pa_decode_workspace_bytes(ctypes.byref(params))


def pa_decode_partition_tokens(params: pa_decode_params) -> int:
    v = lib().pa_decode_partition_tokens(ctypes.byref(params))
    if v < 0:
        _check(-v)
    return v


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
              max_context_len, scale, partition_tokens=0, kernel="auto", workspace=None,
              stream=None, k_new=None, v_new=None, slot_mapping=None, sliding_window=0,
              shared_prefix_blocks=0):
    """out <- paged decode attention (optionally appending k_new/v_new first).
    workspace: a uint8 device tensor of at least pa_decode_workspace_bytes()
    bytes (no initialization needed), or None to allocate one.  For an int8
    cache (codes and scales in its tiles) q gives the q type."""
    import torch
    params = make_decode_params(out, q, k_cache, v_cache, block_tables, context_lens,
                                num_kv_heads, max_context_len, scale, partition_tokens, kernel,
                                k_new, v_new, slot_mapping, sliding_window=sliding_window,
                                shared_prefix_blocks=shared_prefix_blocks)
    need = pa_decode_workspace_bytes(params)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pa_decode(ctypes.byref(params), ws_ptr, ws_bytes, _stream(stream)))
    return out


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                      max_context_len, scale, partition_tokens=0, kernel="auto", stream=None,
                      k_new=None, v_new=None, slot_mapping=None, sliding_window=0, shared_prefix_blocks=0):
    """pa_decode with the library's own per-device workspace: allocates nothing."""
    params = make_decode_params(out, q, k_cache, v_cache, block_tables, context_lens,
                                num_kv_heads, max_context_len, scale, partition_tokens, kernel,
                                k_new, v_new, slot_mapping, sliding_window=sliding_window,
                                shared_prefix_blocks=shared_prefix_blocks)
    _check(lib().pa_decode_noalloc(ctypes.byref(params), _stream(stream)))
    return out


def make_extend_params(out, q, k_cache, v_cache, block_tables, context_lens, query_start, num_kv_heads,
                       max_context_len, max_query_len, scale, partition_tokens=0, start_event=None,
                       stop_event=None):
    """q, out: [T][Hq][D]; query_start: int32 [S+1] device tensor (see include/pa.h)."""
    T, Hq, D = q.shape
    S = context_lens.numel()
    nb = k_cache.numel() // (num_kv_heads * BLOCK_SIZE * D)
    return pa_extend_params(
        _dev(out), _dev(q), _dev(k_cache), _dev(v_cache), _dev(block_tables), _dev(context_lens),
        _dev(query_start), S, T, Hq, num_kv_heads, D,
        block_tables.shape[1] if block_tables.dim() == 2 else 0, nb, int(max_context_len),
        int(max_query_len), float(scale), _dtype_code(k_cache), _dtype_code(out), int(partition_tokens),
        _event(start_event), _event(stop_event))


def pa_extend_workspace_bytes(params: pa_extend_params) -> int:
    return lib().pa_extend_workspace_bytes(ctypes.byref(params))


def pa_extend_partition_tokens(params: pa_extend_params) -> int:
    v = lib().pa_extend_partition_tokens(ctypes.byref(params))
    if v < 0:
        _check(-v)
    return v


def pa_extend(out, q, k_cache, v_cache, block_tables, context_lens, query_start, num_kv_heads,
              max_context_len, max_query_len, scale, partition_tokens=0, workspace=None, stream=None):
    """out <- multi-query attention of the new tokens (rows of q) over the cache."""
    import torch
    params = make_extend_params(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                                num_kv_heads, max_context_len, max_query_len, scale, partition_tokens)
    need = pa_extend_workspace_bytes(params)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ptr, n = _ws(workspace)
    _check(lib().pa_extend(ctypes.byref(params), ptr, n, _stream(stream)))
    return out


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace), workspace.numel() * workspace.element_size()


def pa_decode_partitions(params: pa_decode_params, workspace=None, stream=None):
    """Partition kernel only, on prebuilt parameters (see include/pa.h)."""
    ptr, n = _ws(workspace)
    _check(lib().pa_decode_partitions(ctypes.byref(params), ptr, n, _stream(stream)))


def pa_decode_merge(params: pa_decode_params, workspace=None, stream=None):
    """Merge kernel only, on prebuilt parameters (see include/pa.h)."""
    ptr, n = _ws(workspace)
    _check(lib().pa_decode_merge(ctypes.byref(params), ptr, n, _stream(stream)))


def pa_reshape_and_cache(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None):
    T, Hkv, D = k_new.shape
    nb = k_cache.numel() // (Hkv * BLOCK_SIZE * D)
    _check(lib().pa_reshape_and_cache(_dev(k_new), _dev(v_new), _dev(k_cache), _dev(v_cache),
                                      _dev(slot_mapping), T, Hkv, D, nb, _dtype_code(k_cache),
                                      _stream(stream)))


def pa_reshape_and_cache_int8(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None):
    """Quantize [T][Hkv][D] fp16/bf16 rows into an int8 cache (codes and scales in its tiles)."""
    T, Hkv, D = k_new.shape
    nb = k_cache.numel() // block_elems(k_cache, Hkv, D)
    _check(lib().pa_reshape_and_cache_int8(_dev(k_new), _dev(v_new), _dev(k_cache), _dev(v_cache),
                                           _dev(slot_mapping), T, Hkv, D, nb, _dtype_code(k_new),
                                           _stream(stream)))


def pa_reshape_and_cache_fp8(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None):
    """Quantize [T][Hkv][D] fp16/bf16 rows into an E4M3 cache (uint8 codes and scales in its tiles)."""
    T, Hkv, D = k_new.shape
    nb = k_cache.numel() // block_elems(k_cache, Hkv, D)
    _check(lib().pa_reshape_and_cache_fp8(_dev(k_new), _dev(v_new), _dev(k_cache), _dev(v_cache),
                                          _dev(slot_mapping), T, Hkv, D, nb, _dtype_code(k_new),
                                          _stream(stream)))


def pa_copy_blocks_int8(k_cache, v_cache, src_dst_pairs, num_kv_heads, head_dim, stream=None):
    n = src_dst_pairs.numel() // 2
    nb = k_cache.numel() // block_elems(k_cache, num_kv_heads, head_dim)
    _check(lib().pa_copy_blocks_int8(_dev(k_cache), _dev(v_cache), _dev(src_dst_pairs), n, num_kv_heads,
                                     head_dim, nb, _stream(stream)))


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, num_kv_heads, head_dim, stream=None):
    """Block copies between two pools (device or pinned host tensors of the cache
    layout); src_dst_pairs int32 [n][2] on the device or pinned."""
    n = src_dst_pairs.numel() // 2
    per = num_kv_heads * BLOCK_SIZE * head_dim
    _check(lib().pa_swap_blocks(_gpu_addressable(src_k), _gpu_addressable(src_v), src_k.numel() // per,
                                _gpu_addressable(dst_k), _gpu_addressable(dst_v), dst_k.numel() // per,
                                _gpu_addressable(src_dst_pairs), n, num_kv_heads, head_dim,
                                _dtype_code(src_k), _stream(stream)))


def pa_swap_blocks_int8(src_k, src_v, dst_k, dst_v, src_dst_pairs, num_kv_heads, head_dim, stream=None):
    """Block copies between two byte caches (codes and scales in their tiles)."""
    n = src_dst_pairs.numel() // 2
    per = block_elems(src_k, num_kv_heads, head_dim)
    g = _gpu_addressable
    _check(lib().pa_swap_blocks_int8(g(src_k), g(src_v), src_k.numel() // per, g(dst_k), g(dst_v),
                                     dst_k.numel() // per, g(src_dst_pairs), n, num_kv_heads, head_dim,
                                     _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, src_dst_pairs, num_kv_heads, head_dim, stream=None):
    n = src_dst_pairs.numel() // 2
    nb = k_cache.numel() // (num_kv_heads * BLOCK_SIZE * head_dim)
    _check(lib().pa_copy_blocks(_dev(k_cache), _dev(v_cache), _dev(src_dst_pairs), n,
                                num_kv_heads, head_dim, nb, _dtype_code(k_cache), _stream(stream)))


# ---------------------------------------------------------------- host pool
class BlockPool:
    """The pa_block_pool_* / pa_seq_* calls on one pool handle."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, initial_free_order=None):
        self._h = ctypes.c_void_p()
        order = None
        if initial_free_order is not None:
            self._order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            order = self._order.ctypes.data_as(_PI32)
        _check(lib().pa_block_pool_create(num_blocks, block_size, order, ctypes.byref(self._h)))

    def close(self):
        if self._h:
            lib().pa_block_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return lib().pa_block_pool_num_blocks(self._h)

    def num_free(self) -> int:
        return lib().pa_block_pool_num_free(self._h)

    def refcount(self, block: int) -> int:
        return lib().pa_block_pool_refcount(self._h, block)

    def free_list(self):
        n = lib().pa_block_pool_free_list(self._h, None, 0)
        buf = np.empty(max(n, 1), dtype=np.int32)
        lib().pa_block_pool_free_list(self._h, buf.ctypes.data_as(_PI32), n)
        return buf[:n].tolist()

    def alloc(self) -> int:
        b = ctypes.c_int32()
        _check(lib().pa_block_pool_alloc(self._h, ctypes.byref(b)))
        return b.value

    def incref(self, block: int):
        _check(lib().pa_block_pool_incref(self._h, block))

    def decref(self, block: int):
        _check(lib().pa_block_pool_decref(self._h, block))

    def seq_create(self) -> int:
        s = ctypes.c_int32()
        _check(lib().pa_seq_create(self._h, ctypes.byref(s)))
        return s.value

    def seq_fork(self, parent: int) -> int:
        s = ctypes.c_int32()
        _check(lib().pa_seq_fork(self._h, parent, ctypes.byref(s)))
        return s.value

    def seq_append(self, seq: int, n_tokens: int = 1):
        """Returns (slots int64 array, cow) with cow = (src, dst) or None."""
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_seq_append(self._h, seq, n_tokens, slots.ctypes.data_as(_PI64),
                                   ctypes.byref(src), ctypes.byref(dst)))
        return slots[:n_tokens], (None if src.value < 0 else (src.value, dst.value))

    def seq_append_batch(self, seq_ids, slots_out=None, cows_out=None):
        """One token for each sequence.  Returns (slots, cow_pairs [k][2])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        n = len(ids)
        slots = slots_out if slots_out is not None else np.empty(max(n, 1), dtype=np.int64)
        cows = cows_out if cows_out is not None else np.empty((max(n, 1), 2), dtype=np.int32)
        k = ctypes.c_int32()
        _check(lib().pa_seq_append_batch(self._h, ids.ctypes.data_as(_PI32), n,
                                         slots.ctypes.data_as(_PI64), cows.ctypes.data_as(_PI32),
                                         ctypes.byref(k)))
        return slots[:n], cows[:k.value]

    def seq_free(self, seq: int):
        _check(lib().pa_seq_free(self._h, seq))

    def seq_num_tokens(self, seq: int) -> int:
        return lib().pa_seq_num_tokens(self._h, seq)

    def seq_swap_out(self, seq: int) -> np.ndarray:
        """Releases the private blocks; returns their ids (table order)."""
        cap = max(1, -(-self.seq_num_tokens(seq) // BLOCK_SIZE))
        buf = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_seq_swap_out(self._h, seq, buf.ctypes.data_as(_PI32), cap, ctypes.byref(n)))
        return buf[:n.value].copy()

    def seq_swap_in(self, seq: int) -> np.ndarray:
        """Appends fresh blocks for the swapped-out ones; returns their ids."""
        cap = max(1, self.seq_swapped_blocks(seq))
        buf = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().pa_seq_swap_in(self._h, seq, buf.ctypes.data_as(_PI32), cap, ctypes.byref(n)))
        return buf[:n.value].copy()

    def seq_swapped_blocks(self, seq: int) -> int:
        return lib().pa_seq_swapped_blocks(self._h, seq)

    def seq_export(self, seq_ids, max_blocks: int, tables_out=None, lens_out=None):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        n = len(ids)
        tables = tables_out if tables_out is not None else np.empty((n, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        _check(lib().pa_seq_export(self._h, ids.ctypes.data_as(_PI32), n, max_blocks,
                                   tables.ctypes.data_as(_PI32), lens.ctypes.data_as(_PI32)))
        return tables, lens
