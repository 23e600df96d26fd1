"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it, and
it shares no code with the GPU path: ``pa_oracle.c`` re-implements the cache
layout from its written contract and does all arithmetic in IEEE double.

Contents
  * ``pa_oracle.c`` (built to ``liboracle.so`` with gcc, no fast-math): fp64
    table-walk decode, contiguous brute force, the slot-mapped KV append and
    whole-block copies.  Passages followed are cited in that file.
  * ``pool_model.py``: an independent pure-Python model of the refcounted
    block pool (allocation, fork, append with copy-on-write, free).
  * INT8 / FP8 caches: one byte array per K and V whose tiles hold the codes
    (``np.int8`` / ``np.uint8``) of 16 tokens of one (block, KV head) followed
    by their 16 float32 row scales; quantized on append, attended over the
    dequantized rows (``*_i8`` / ``*_fp8`` functions).

Data convention for the wrappers: cache-typed arrays are numpy arrays of
``np.float32`` (fp32), ``np.float16`` (fp16) or ``np.uint16`` holding raw
bfloat16 bits (bf16); ``dtype`` names the type: "f32", "f16" or "bf16".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .pool_model import PoolModel, PoolError, OutOfBlocks  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_k_offset.restype = _I64
        lib.oracle_k_offset.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.oracle_v_offset.restype = _I64
        lib.oracle_v_offset.argtypes = [_I64, _I, _I, _I, _I, _I, _I]
        lib.oracle_reshape_and_cache.restype = _I
        lib.oracle_reshape_and_cache.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I64, _I]
        lib.oracle_copy_blocks.restype = None
        lib.oracle_copy_blocks.argtypes = [_P, _P, _P, _I, _I, _I, _I]
        lib.oracle_decode.restype = _I
        lib.oracle_decode.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                      ctypes.c_float, _I, _I, _I]
        lib.oracle_k_offset_i8.restype = _I64
        lib.oracle_k_offset_i8.argtypes = [_I64, _I, _I, _I, _I, _I]
        lib.oracle_v_offset_i8.restype = _I64
        lib.oracle_v_offset_i8.argtypes = [_I64, _I, _I, _I, _I, _I]
        lib.oracle_quantize_row_i8.restype = ctypes.c_float
        lib.oracle_quantize_row_i8.argtypes = [_P, _I64, _I, _I, _P]
        lib.oracle_scale_offset_i8.restype = _I64
        lib.oracle_scale_offset_i8.argtypes = [_I64, _I, _I, _I, _I]
        lib.oracle_reshape_and_cache_i8.restype = _I
        lib.oracle_reshape_and_cache_i8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I64, _I]
        lib.oracle_copy_blocks_i8.restype = None
        lib.oracle_copy_blocks_i8.argtypes = [_P, _P, _P, _I, _I, _I]
        lib.oracle_decode_codes.restype = _I
        lib.oracle_decode_codes.argtypes = [_P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I,
                                            _I, ctypes.c_float, _I, _I, _I]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [_I]
        lib.oracle_e4m3_encode.restype = _I
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_quantize_row_fp8.restype = ctypes.c_float
        lib.oracle_quantize_row_fp8.argtypes = [_P, _I64, _I, _I, _P]
        lib.oracle_reshape_and_cache_fp8.restype = _I
        lib.oracle_reshape_and_cache_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I64, _I]
        lib.oracle_extend.restype = _I
        lib.oracle_extend.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                      ctypes.c_float, _I, _I]
        lib.oracle_bruteforce_contiguous.restype = None
        lib.oracle_bruteforce_contiguous.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                                     ctypes.c_float, _I, _I]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(a: np.ndarray, dtype: str):
    if a.dtype != _NP[dtype]:
        raise TypeError(f"expected {np.dtype(_NP[dtype])} for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def np_type(dtype: str):
    return _NP[dtype]


def k_offset(block, head, tok, dim, num_kv_heads, head_dim, dtype):
    return _load().oracle_k_offset(block, head, tok, dim, num_kv_heads, head_dim, _DTYPES[dtype])


def v_offset(block, head, tok, dim, num_kv_heads, head_dim, dtype):
    return _load().oracle_v_offset(block, head, tok, dim, num_kv_heads, head_dim, _DTYPES[dtype])


def empty_cache(num_blocks, num_kv_heads, head_dim, dtype):
    """A pool whose every element is NaN (unused slots stay poisoned)."""
    n = num_blocks * num_kv_heads * 16 * head_dim
    if dtype == "bf16":
        return np.full(n, 0x7FC0, dtype=np.uint16)
    return np.full(n, np.nan, dtype=_NP[dtype])


def reshape_and_cache(k_new, v_new, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                      num_blocks, dtype):
    """Scatter [T][Hkv][D] rows into the caches in place; returns #out-of-range slots."""
    k_new = _check(k_new, dtype)
    v_new = _check(v_new, dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]
    return _load().oracle_reshape_and_cache(_ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                            _ptr(v_cache), _ptr(slots), len(slots),
                                            num_kv_heads, head_dim, num_blocks, _DTYPES[dtype])


def copy_blocks(k_cache, v_cache, pairs, num_kv_heads, head_dim, dtype):
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _load().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), len(pairs),
                               num_kv_heads, head_dim, _DTYPES[dtype])


def swap_blocks(src, dst, pairs, per_block):
    """Whole-block copies between two pools of one array each (a K or V cache,
    or a scale array): block p of src -> block q of dst for each (p, q), with
    per_block elements per block; pairs outside either pool are skipped.  The
    swap copies of preemption ("Inference serving: the KV-cache machine",
    section "Paged KV")."""
    s = src.reshape(-1, per_block)
    d = dst.reshape(-1, per_block)
    for p, q in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= p < len(s) and 0 <= q < len(d):
            d[q] = s[p]


def decode(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads, scale, dtype,
           nthreads=0, return_threads=False, window=0):
    """fp64 paged decode; q is [S][Hq][D] in the cache type.  Returns float64 [S][Hq][D].
    window: sliding window W (0 = none): the query at position L-1 sees L-1-W .. L-1."""
    q = _check(q, dtype)
    S, Hq, D = q.shape
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty((S, Hq, D), dtype=np.float64)
    used = _load().oracle_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(tables),
                                 _ptr(lens), S, Hq, num_kv_heads, D, tables.shape[1],
                                 float(scale), _DTYPES[dtype], int(window), nthreads)
    return (out, used) if return_threads else out


def extend(q, k_cache, v_cache, block_tables, context_lens, query_start, num_kv_heads, scale, dtype,
           nthreads=0):
    """fp64 multi-query attention: q is [T][Hq][D] (rows of sequence s are
    query_start[s] .. query_start[s+1]-1, at positions L-n .. L-1); row t at
    position p attends to 0 .. p.  Returns float64 [T][Hq][D]."""
    q = _check(q, dtype)
    T, Hq, D = q.shape
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    assert qs[-1] == T and len(qs) == len(lens) + 1
    out = np.empty((T, Hq, D), dtype=np.float64)
    _load().oracle_extend(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(tables), _ptr(lens),
                          _ptr(qs), len(lens), Hq, num_kv_heads, D, tables.shape[1], float(scale),
                          _DTYPES[dtype], nthreads)
    return out


def bruteforce_contiguous(q, k_seq, v_seq, context_lens, scale, dtype, window=0):
    """fp64 attention over contiguous [S][Lmax][Hkv][D] arrays (no table)."""
    q = _check(q, dtype)
    k_seq = _check(k_seq, dtype)
    v_seq = _check(v_seq, dtype)
    S, Hq, D = q.shape
    _, Lmax, Hkv, _ = k_seq.shape
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty((S, Hq, D), dtype=np.float64)
    _load().oracle_bruteforce_contiguous(_ptr(out), _ptr(q), _ptr(k_seq), _ptr(v_seq),
                                         _ptr(lens), S, Hq, Hkv, D, Lmax, float(scale),
                                         _DTYPES[dtype], int(window))
    return out


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen cache-typed values to float64 exactly (bf16 bits are the top half of fp32)."""
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------- INT8 caches
def k_offset_i8(block, head, tok, dim, num_kv_heads, head_dim):
    return _load().oracle_k_offset_i8(block, head, tok, dim, num_kv_heads, head_dim)


def v_offset_i8(block, head, tok, dim, num_kv_heads, head_dim):
    return _load().oracle_v_offset_i8(block, head, tok, dim, num_kv_heads, head_dim)


def scale_offset_i8(block, head, tok, num_kv_heads, head_dim):
    """Byte offset of the float32 scale of row (block, head, tok) in a K or V cache."""
    return _load().oracle_scale_offset_i8(block, head, tok, num_kv_heads, head_dim)


def read_scale(cache, block, head, tok, num_kv_heads, head_dim) -> np.float32:
    o = scale_offset_i8(block, head, tok, num_kv_heads, head_dim)
    return cache[o:o + 4].view(np.float32)[0]


def cache_bytes_i8(num_blocks, num_kv_heads, head_dim) -> int:
    """Bytes of one K or V byte cache: 16 rows of head_dim codes + 4 scale bytes per tile."""
    return num_blocks * num_kv_heads * 16 * (head_dim + 4)


def quantize_row_i8(row: np.ndarray, dtype: str):
    """(codes int8 [n], scale float32) of one row in the given type."""
    row = _check(np.asarray(row), dtype)
    codes = np.empty(row.size, dtype=np.int8)
    sc = _load().oracle_quantize_row_i8(_ptr(row), 0, row.size, _DTYPES[dtype], _ptr(codes))
    return codes, np.float32(sc)


def _empty_codes(num_blocks, num_kv_heads, head_dim, np_type):
    """An unwritten byte cache: codes 0x7F, every scale NaN."""
    tiles = np.full((num_blocks * num_kv_heads, 16 * (head_dim + 4)), 0x7F, dtype=np.uint8)
    tiles[:, 16 * head_dim:].view(np.float32)[:] = np.nan
    return tiles.reshape(-1).view(np_type)


def empty_cache_i8(num_blocks, num_kv_heads, head_dim):
    """One unwritten int8 cache (K or V): codes 0x7F, scales NaN."""
    return _empty_codes(num_blocks, num_kv_heads, head_dim, np.int8)


def reshape_and_cache_i8(k_new, v_new, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                         num_blocks, src_dtype):
    """Quantize [T][Hkv][D] rows into the int8 caches in place; returns #out-of-range slots."""
    k_new = _check(k_new, src_dtype)
    v_new = _check(v_new, src_dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    for a in (k_cache, v_cache):
        assert a.dtype == np.int8 and a.flags["C_CONTIGUOUS"]
        assert a.size == cache_bytes_i8(num_blocks, num_kv_heads, head_dim)
    return _load().oracle_reshape_and_cache_i8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(slots), len(slots), num_kv_heads, head_dim, num_blocks,
                                               _DTYPES[src_dtype])


def copy_blocks_i8(k_cache, v_cache, pairs, num_kv_heads, head_dim):
    """Whole-block copies of a byte cache (int8 or E4M3): codes and scales of every head."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _load().oracle_copy_blocks_i8(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), len(pairs), num_kv_heads,
                                  head_dim)


def decode_i8(q, q_dtype, k_cache, v_cache, block_tables, context_lens, num_kv_heads, scale, nthreads=0,
              return_threads=False, window=0, fp8=False):
    """fp64 paged decode over an int8 cache (an E4M3 one with fp8=True; codes as
    uint8); q is [S][Hq][D] in q_dtype."""
    q = _check(q, q_dtype)
    S, Hq, D = q.shape
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty((S, Hq, D), dtype=np.float64)
    used = _load().oracle_decode_codes(_ptr(out), _ptr(q), _DTYPES[q_dtype], _ptr(k_cache), _ptr(v_cache),
                                       _ptr(tables), _ptr(lens), S, Hq, num_kv_heads, D, tables.shape[1],
                                       float(scale), int(window), int(fp8), nthreads)
    return (out, used) if return_threads else out


# ---------------------------------------------------------------- FP8 (E4M3) caches
def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def e4m3_encode(x: float) -> int:
    return _load().oracle_e4m3_encode(float(x))


def quantize_row_fp8(row: np.ndarray, dtype: str):
    """(codes uint8 [n], scale float32) of one row in the given type."""
    row = _check(np.asarray(row), dtype)
    codes = np.empty(row.size, dtype=np.uint8)
    sc = _load().oracle_quantize_row_fp8(_ptr(row), 0, row.size, _DTYPES[dtype], _ptr(codes))
    return codes, np.float32(sc)


def empty_cache_fp8(num_blocks, num_kv_heads, head_dim):
    """One unwritten FP8 cache (K or V): NaN codes 0x7F, NaN scales."""
    return _empty_codes(num_blocks, num_kv_heads, head_dim, np.uint8)


def reshape_and_cache_fp8(k_new, v_new, k_cache, v_cache, slot_mapping, num_kv_heads, head_dim,
                          num_blocks, src_dtype):
    """Quantize [T][Hkv][D] rows into the FP8 caches in place; returns #out-of-range slots."""
    k_new = _check(k_new, src_dtype)
    v_new = _check(v_new, src_dtype)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    for a in (k_cache, v_cache):
        assert a.dtype == np.uint8 and a.flags["C_CONTIGUOUS"]
        assert a.size == cache_bytes_i8(num_blocks, num_kv_heads, head_dim)
    return _load().oracle_reshape_and_cache_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                                _ptr(slots), len(slots), num_kv_heads, head_dim, num_blocks,
                                                _DTYPES[src_dtype])
