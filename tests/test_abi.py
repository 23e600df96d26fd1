"""The C-ABI library loads and exports every declared entry point (no GPU).

Only host-side paths run here: symbol lookup, argument validation that returns
before any launch, and the workspace / partition arithmetic.
"""
import ctypes
import os
import re

import pytest

from paged_kv_cache_65_amd import binding as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pa.LIB_PATH)
    names = _declared()
    assert len(names) >= 20
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_version_and_empty_error():
    assert "gfx950" in pa.pa_version()


def _params(**over):
    p = pa.pa_decode_params(
        ctypes.c_void_p(16), ctypes.c_void_p(32), ctypes.c_void_p(48), ctypes.c_void_p(64),
        ctypes.c_void_p(80), ctypes.c_void_p(96), 64, 64, 8, 128, 256, 20000, 4096, 0.088,
        pa.PA_BF16, pa.PA_BF16, 0, pa.PA_KERNEL_AUTO)
    for k, v in over.items():
        setattr(p, k, v)
    return p


def test_workspace_and_partition_arithmetic():
    # the partition rule of the vector-ALU path (and of the matrix-core path
    # when a batch is too large for the balanced split).  No GPU here: the
    # library assumes 256 compute units, i.e. a target of 2048 workgroups;
    # 64 sequences x 8 KV heads x ceil(4096/1024) reach it
    p = _params(kernel=pa.PA_KERNEL_VALU)
    assert pa.pa_decode_partition_tokens(p) == 1024
    # m and l plus a D-wide accumulator per (seq, q head, partition), float32
    assert pa.pa_decode_workspace_bytes(p) == 64 * 64 * 4 * (128 + 2) * 4
    p.num_seqs = 8                      # 8 x 8 x ceil(4096/256) < 2048: smallest partitions
    assert pa.pa_decode_partition_tokens(p) == 256
    p.num_seqs = 64
    p.max_context_len = 300             # 512 pairs x 1 partition < 2048: split at 256
    assert pa.pa_decode_partition_tokens(p) == 256
    assert pa.pa_decode_workspace_bytes(p) == 64 * 64 * 2 * 130 * 4
    p.num_seqs = 4096                   # a large batch of short contexts is not split
    assert pa.pa_decode_partition_tokens(p) == 304
    assert pa.pa_decode_workspace_bytes(p) == 0
    p.num_seqs = 64
    p.partition_tokens = 64
    assert pa.pa_decode_workspace_bytes(p) == 64 * 64 * 5 * 130 * 4
    p.num_seqs, p.num_kv_heads, p.num_q_heads = 3, 1, 2
    assert pa.pa_decode_workspace_bytes(p) == 3 * 2 * 5 * 130 * 4


def _r16(x):
    return (x + 15) // 16 * 16


def test_balanced_split_selection_and_workspace():
    # automatic partitioning on the matrix-core path: balanced split, reported
    # as partition size 0.  Without a GPU: one workgroup of 4 waves per CU, 256 CUs.
    nw = 256 * 4
    p = _params()
    assert pa.pa_decode_partition_tokens(p) == 0
    slots = nw + 64 * 8 - 1             # one slot per segment: NW + pairs - 1
    G, D = 8, 128
    assert pa.pa_decode_workspace_bytes(p) == _r16(65 * 4) + _r16(slots * G * 2 * 4) + slots * G * D * 4
    # explicit partitions, more than 1024 sequences, or more than 2^15 (s, g)
    # pairs go back to the partition path
    assert pa.pa_decode_partition_tokens(_params(partition_tokens=512)) == 512
    assert pa.pa_decode_partition_tokens(_params(num_seqs=1025)) == 1024
    assert pa.pa_decode_partition_tokens(_params(num_seqs=1024)) == 0
    assert pa.pa_decode_partition_tokens(_params(num_seqs=1024, num_q_heads=64, num_kv_heads=32)) == 0
    assert pa.pa_decode_partition_tokens(_params(num_seqs=1024, num_q_heads=64, num_kv_heads=64)) > 0
    # fp32 caches never take the matrix-core path
    assert pa.pa_decode_partition_tokens(_params(kv_dtype=pa.PA_F32, out_dtype=pa.PA_F32)) > 0


def test_arrays_without_elements_may_be_null():
    # every context empty: a table with no columns needs no pointer
    p = _params(num_seqs=2, max_blocks_per_seq=0, max_context_len=0, block_tables=None)
    assert pa.pa_decode_partition_tokens(p) >= 0
    # no sequences: out, q, lengths and tables need none either
    p = _params(num_seqs=0, out=None, q=None, context_lens=None, block_tables=None)
    assert pa.pa_decode_partition_tokens(p) >= 0
    # but a table with columns does
    with pytest.raises(pa.PaError) as err:
        pa.pa_decode_partition_tokens(_params(block_tables=None))
    assert err.value.status == pa.PA_ERR_INVALID_ARG
    with pytest.raises(pa.PaError):
        pa.pa_decode_partition_tokens(_params(max_blocks_per_seq=-1))


def test_small_batches_take_partitions_unless_the_balanced_split_is_asked_for():
    # fewer than 48 units per wave at the longest context (1024 waves without a
    # GPU): 8 sequences x 32 KV heads x 128 blocks = 32768 < 49152
    # ... about one workgroup per CU: with as many (sequence, KV head) pairs as
    # CUs (256 without a GPU) each pair is one partition and nothing is merged
    small = dict(num_seqs=8, num_q_heads=32, num_kv_heads=32, max_context_len=2048)
    assert pa.pa_decode_partition_tokens(_params(**small)) == 2048
    assert pa.pa_decode_workspace_bytes(_params(**small)) == 0
    assert pa.pa_decode_partition_tokens(_params(**{**small, "max_context_len": 300})) == 304
    # 64 pairs: each range cut into 256 / 64 = 4 pieces, ceil(4304 / 4) = 1076 -> 1088
    tp = dict(num_seqs=64, num_q_heads=8, num_kv_heads=1, max_context_len=4300)
    assert pa.pa_decode_partition_tokens(_params(**tp)) == 1088
    assert pa.pa_decode_workspace_bytes(_params(**tp)) == 64 * 8 * 4 * (128 + 2) * 4
    assert pa.pa_decode_partition_tokens(_params(**small, partition_tokens=pa.PA_PARTITION_BALANCED)) == 0
    # 8 sequences x 32 heads x 192 blocks = 49152: the balanced split
    assert pa.pa_decode_partition_tokens(_params(**{**small, "max_context_len": 3072})) == 0
    # a sliding window bounds the units a pair can hold: 48 x 1024 units need
    # 32 x 8 pairs of >= 192 blocks, more than a 1024-token window spans
    # (256 pairs: one partition over the window's W + 16 tokens, no merge)
    win = _params(num_seqs=32, num_q_heads=32, num_kv_heads=8, max_context_len=16384, sliding_window=1024)
    assert pa.pa_decode_partition_tokens(win) == 1040 and pa.pa_decode_workspace_bytes(win) == 0
    # with a pair for every CU a window makes one partition per pair (W + 16 tokens, no merge);
    # fewer pairs with enough units keep the balanced split
    assert pa.pa_decode_partition_tokens(_params(num_seqs=32, num_q_heads=32, num_kv_heads=8,
                                                 max_context_len=16384, sliding_window=4096)) == 4112
    assert pa.pa_decode_partition_tokens(_params(num_seqs=64, num_q_heads=16, num_kv_heads=2,
                                                 max_context_len=16384, sliding_window=8192)) == 0
    # the balanced split cannot run an fp32 cache or > 1024 sequences: asking is an error
    for bad, status in ((dict(kv_dtype=pa.PA_F32, out_dtype=pa.PA_F32, partition_tokens=pa.PA_PARTITION_BALANCED),
                         pa.PA_ERR_UNSUPPORTED),
                        (dict(num_seqs=1025, partition_tokens=pa.PA_PARTITION_BALANCED), pa.PA_ERR_UNSUPPORTED),
                        (dict(partition_tokens=-2), pa.PA_ERR_INVALID_ARG)):
        with pytest.raises(pa.PaError) as err:
            pa.pa_decode_partition_tokens(_params(**bad))
        assert err.value.status == status
        assert pa.pa_decode_workspace_bytes(_params(**bad)) == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, pa.PA_ERR_UNSUPPORTED),
    ("num_kv_heads", 7, pa.PA_ERR_INVALID_ARG),
    ("num_q_heads", 8 * 65, pa.PA_ERR_UNSUPPORTED),
    ("partition_tokens", 24, pa.PA_ERR_INVALID_ARG),
    ("out_dtype", pa.PA_F16, pa.PA_ERR_UNSUPPORTED),
    ("q", ctypes.c_void_p(33), pa.PA_ERR_INVALID_ARG),
    ("k_cache", None, pa.PA_ERR_INVALID_ARG),
    ("kernel", 9, pa.PA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_parameters_before_launch(field, value, status):
    p = _params(**{field: value})
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == status
    assert pa.lib().pa_last_error().decode().startswith("pa_decode")


def test_decode_requires_the_workspace():
    p = _params()
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == pa.PA_ERR_WORKSPACE


def test_noalloc_decode_validates_and_refuses_more_than_its_array_before_any_device_call():
    # invalid parameters: the same checks as pa_decode
    p = _params(partition_tokens=24)
    assert pa.lib().pa_decode_noalloc(ctypes.byref(p), None) == pa.PA_ERR_INVALID_ARG
    # 1024 sequences x 64 query heads x 64 partitions x (128 + 2) floats >> 64 MiB
    p = _params(kernel=pa.PA_KERNEL_VALU, num_seqs=1024, partition_tokens=64)
    assert pa.pa_decode_workspace_bytes(p) > pa.PA_NOALLOC_WORKSPACE_BYTES
    assert pa.lib().pa_decode_noalloc(ctypes.byref(p), None) == pa.PA_ERR_WORKSPACE
    assert "pa_decode_noalloc" in pa.lib().pa_last_error().decode()


def test_fused_append_fields_go_together():
    p = _params(k_new=ctypes.c_void_p(16))
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == pa.PA_ERR_INVALID_ARG


def test_mfma_kernel_rejects_fp32():
    p = _params(kv_dtype=pa.PA_F32, out_dtype=pa.PA_F32, kernel=pa.PA_KERNEL_MFMA)
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == pa.PA_ERR_UNSUPPORTED


def test_append_and_copy_reject_bad_sizes():
    L = pa.lib()
    assert L.pa_reshape_and_cache(None, None, None, None, None, 4, 8, 96, 10, pa.PA_BF16, None) \
        == pa.PA_ERR_UNSUPPORTED
    assert L.pa_reshape_and_cache(None, None, None, None, None, 4, 8, 128, 10, pa.PA_BF16, None) \
        == pa.PA_ERR_INVALID_ARG
    assert L.pa_reshape_and_cache(None, None, None, None, None, 0, 8, 128, 10, pa.PA_BF16, None) \
        == pa.PA_OK
    assert L.pa_copy_blocks(None, None, None, -1, 8, 128, 10, pa.PA_BF16, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_copy_blocks(None, None, None, 0, 8, 128, 10, pa.PA_BF16, None) == pa.PA_OK


def _i8(**over):
    base = dict(kv_dtype=pa.PA_I8, q_dtype=pa.PA_BF16, out_dtype=pa.PA_F32)
    base.update(over)
    return _params(**base)


def test_int8_cache_takes_the_balanced_split():
    assert pa.pa_decode_partition_tokens(_i8()) == 0
    assert pa.pa_decode_partition_tokens(_i8(out_dtype=pa.PA_BF16)) == 0


@pytest.mark.parametrize("over,status", [
    (dict(q_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),
    (dict(out_dtype=pa.PA_F16), pa.PA_ERR_UNSUPPORTED),
    (dict(partition_tokens=256), pa.PA_ERR_UNSUPPORTED),
    (dict(kernel=pa.PA_KERNEL_VALU), pa.PA_ERR_UNSUPPORTED),
    (dict(num_seqs=1025), pa.PA_ERR_UNSUPPORTED),
    (dict(k_new=ctypes.c_void_p(16)), pa.PA_ERR_INVALID_ARG),
    (dict(k_new=ctypes.c_void_p(16), v_new=ctypes.c_void_p(16), slot_mapping=ctypes.c_void_p(16),
          partition_tokens=256), pa.PA_ERR_UNSUPPORTED),
])
def test_int8_decode_rejects_unsupported_requests(over, status):
    p = _i8(**over)
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == status
    assert pa.pa_decode_workspace_bytes(p) == 0


def test_byte_caches_take_the_fused_append_on_the_balanced_split():
    for kv in (pa.PA_I8, pa.PA_FP8):
        p = _i8(kv_dtype=kv, k_new=ctypes.c_void_p(16), v_new=ctypes.c_void_p(16),
                slot_mapping=ctypes.c_void_p(16))
        assert pa.pa_decode_partition_tokens(p) == 0
        assert pa.pa_decode_workspace_bytes(p) > 0


def test_int8_append_and_copy_reject_bad_arguments():
    L = pa.lib()
    args = (None, None, None, None, None)       # rows, caches (codes and scales in their tiles), slots
    assert L.pa_reshape_and_cache_int8(*args, 4, 8, 128, 10, pa.PA_F32, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_reshape_and_cache_int8(*args, 4, 8, 96, 10, pa.PA_BF16, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_reshape_and_cache_int8(*args, 4, 8, 128, 10, pa.PA_BF16, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_reshape_and_cache_int8(*args, 0, 8, 128, 10, pa.PA_BF16, None) == pa.PA_OK
    assert L.pa_copy_blocks_int8(None, None, None, 0, 8, 128, 10, None) == pa.PA_OK
    assert L.pa_copy_blocks_int8(None, None, None, 2, 8, 128, 10, None) == pa.PA_ERR_INVALID_ARG


# ---------------------------------------------------------------- FP8 caches, window
def test_fp8_cache_follows_the_byte_cache_rules():
    f8 = dict(kv_dtype=pa.PA_FP8, q_dtype=pa.PA_BF16, out_dtype=pa.PA_F32)
    assert pa.pa_decode_partition_tokens(_params(**f8)) == 0
    for over, status in ((dict(q_dtype=pa.PA_F32), pa.PA_ERR_UNSUPPORTED),
                         (dict(partition_tokens=64), pa.PA_ERR_UNSUPPORTED)):
        p = _params(**{**f8, **over})
        assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == status
    L = pa.lib()
    args = (None, None, None, None, None)
    assert L.pa_reshape_and_cache_fp8(*args, 4, 8, 128, 10, pa.PA_F32, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_reshape_and_cache_fp8(*args, 4, 8, 128, 10, pa.PA_BF16, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_reshape_and_cache_fp8(*args, 0, 8, 128, 10, pa.PA_BF16, None) == pa.PA_OK


def test_negative_sliding_window_is_rejected():
    p = _params(sliding_window=-1)
    assert pa.lib().pa_decode(ctypes.byref(p), None, 0, None) == pa.PA_ERR_INVALID_ARG
    assert pa.pa_decode_workspace_bytes(p) == 0


# ---------------------------------------------------------------- extend
def _ext(**over):
    p = pa.pa_extend_params(
        ctypes.c_void_p(16), ctypes.c_void_p(32), ctypes.c_void_p(48), ctypes.c_void_p(64),
        ctypes.c_void_p(80), ctypes.c_void_p(96), ctypes.c_void_p(112),
        64, 256, 64, 8, 128, 256, 20000, 4096, 4, 0.088, pa.PA_BF16, pa.PA_BF16, 0, None, None)
    for k, v in over.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("field,value,status", [
    ("query_start", None, pa.PA_ERR_INVALID_ARG),
    ("out", ctypes.c_void_p(17), pa.PA_ERR_INVALID_ARG),
    ("kv_dtype", pa.PA_F32, pa.PA_ERR_UNSUPPORTED),
    ("kv_dtype", pa.PA_I8, pa.PA_ERR_UNSUPPORTED),
    ("num_q_heads", 8 * 65, pa.PA_ERR_UNSUPPORTED),
    ("num_kv_heads", 7, pa.PA_ERR_INVALID_ARG),
    ("head_dim", 96, pa.PA_ERR_UNSUPPORTED),
    ("out_dtype", pa.PA_F16, pa.PA_ERR_UNSUPPORTED),
    ("partition_tokens", 24, pa.PA_ERR_INVALID_ARG),
    ("max_query_len", -1, pa.PA_ERR_INVALID_ARG),
    ("num_query_rows", -1, pa.PA_ERR_INVALID_ARG),
])
def test_extend_rejects_bad_parameters_before_launch(field, value, status):
    p = _ext(**{field: value})
    assert pa.lib().pa_extend(ctypes.byref(p), None, 0, None) == status
    assert pa.lib().pa_last_error().decode().startswith("pa_extend")
    assert pa.pa_extend_workspace_bytes(p) == 0
    assert pa.lib().pa_extend_partition_tokens(ctypes.byref(p)) == -status


def test_extend_partition_and_workspace_arithmetic():
    # 64 sequences x 8 KV heads x 1 query group (4 tokens of 8 heads fit 32 columns)
    # already give two workgroups per CU: one partition, no workspace
    p = _ext()
    assert pa.pa_extend_partition_tokens(p) == 4096
    assert pa.pa_extend_workspace_bytes(p) == 0
    # one sequence: the context is split, partials need [T][Hq][P][D+2] floats
    p = _ext(num_seqs=1, num_query_rows=4)
    pt = pa.pa_extend_partition_tokens(p)
    assert pt % 16 == 0 and 64 <= pt < 4096
    np_ = -(-4096 // pt)
    assert pa.pa_extend_workspace_bytes(p) == 4 * 64 * np_ * 130 * 4
    assert pa.lib().pa_extend(ctypes.byref(p), None, 0, None) == pa.PA_ERR_WORKSPACE
    p = _ext(partition_tokens=1024)
    assert pa.pa_extend_partition_tokens(p) == 1024
    assert pa.pa_extend_workspace_bytes(p) == 256 * 64 * 4 * 130 * 4


def test_extend_without_rows_launches_nothing():
    for over in (dict(num_seqs=0), dict(num_query_rows=0)):
        p = _ext(**over)
        assert pa.lib().pa_extend(ctypes.byref(p), None, 0, None) == pa.PA_OK


# ---------------------------------------------------------------- swap copies
def test_swap_blocks_reject_bad_arguments_before_touching_memory():
    L = pa.lib()
    nul = (None, None)
    assert L.pa_swap_blocks(*nul, 10, *nul, 10, None, 0, 8, 128, pa.PA_BF16, None) == pa.PA_OK
    assert L.pa_swap_blocks(*nul, 10, *nul, 10, None, 1, 8, 96, pa.PA_BF16, None) == pa.PA_ERR_UNSUPPORTED
    assert L.pa_swap_blocks(*nul, 10, *nul, 10, None, 1, 8, 128, pa.PA_BF16, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks(*nul, 10, *nul, 10, None, 70000, 8, 128, pa.PA_BF16, None) \
        == pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks(*nul, 10, *nul, 10, None, 1, 8, 128, pa.PA_I8, None) == pa.PA_ERR_INVALID_ARG
    # pointers the runtime does not know (no device here, or pageable memory) are refused
    buf = (ctypes.c_uint8 * 4096)()
    addr = (ctypes.addressof(buf) + 15) // 16 * 16
    pairs = (ctypes.c_int32 * 2)(0, 0)
    a = ctypes.c_void_p(addr)
    assert L.pa_swap_blocks(a, a, 1, a, a, 1, pairs, 1, 1, 64, pa.PA_BF16, None) == pa.PA_ERR_INVALID_ARG
    assert L.pa_swap_blocks_int8(*nul, 10, *nul, 10, None, 0, 8, 128, None) == pa.PA_OK
    assert L.pa_swap_blocks_int8(*nul, 10, *nul, 10, None, 1, 8, 128, None) == pa.PA_ERR_INVALID_ARG
