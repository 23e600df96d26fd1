"""Byte and FLOP accounting for paged decode attention (host-side arithmetic).

KV bytes per token = 2 (K and V) x layers x KV heads x head_dim x element bytes
-- the closed form stated on several pages: "Modern AI Infrastructure and
Agentic System Design", section 9.1 "The key and value cache"; "Inference
serving: the KV-cache machine", section "The KV cache: attention's memory bill,
derived"; "KV Cache Explained Like You're an LLM Engineer", section "Why
Recomputing Attention is Inefficient".  All kernels here work on one layer.

Algorithmic bytes of one decode launch are the bytes the method must move:
every cached K/V row read once per (sequence, KV head) -- a physical block
shared by several sequences counts once -- plus q, the output, the used block
table entries and the context lengths.  Split-K workspace traffic is not
algorithmic and is reported apart.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
# An INT8 cache row is head_dim one-byte codes plus one float32 scale.
I8_SCALE_BYTES = 4


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def attended(context_lens, window: int = 0):
    """(tokens, blocks) a decode query reads per sequence: with a sliding window
    W > 0 the positions L-1-W .. L-1 (clipped at 0) and the blocks holding them."""
    lens = np.asarray(context_lens, dtype=np.int64)
    blocks = -(-lens // BLOCK_SIZE)
    if window <= 0:
        return lens, blocks
    first = np.maximum(lens - 1 - window, 0)
    return np.where(lens > 0, lens - first, 0), np.where(lens > 0, blocks - first // BLOCK_SIZE, 0)


def decode_algorithmic_bytes(context_lens, num_q_heads, num_kv_heads, head_dim, dtype,
                             out_dtype, shared_tokens: int = 0, cache: str = "", window: int = 0) -> dict:
    """Bytes one paged decode launch must move.

    shared_tokens: tokens of a prefix whose blocks every sequence maps (counted
    once in 'kv_unique' and once per sequence in 'kv_logical').
    cache: "i8" / "fp8" for an INT8 / E4M3 cache (codes + per-row scales); q and out stay in
    dtype / out_dtype.
    window: sliding window W (0 = none): only the attended rows and the table
    entries of their blocks count.
    """
    lens_all = np.asarray(context_lens, dtype=np.int64)
    lens, blocks = attended(lens_all, window)
    eb = ELEM_BYTES[dtype]
    S = len(lens)
    if cache in ("i8", "fp8"):
        per_tok = 2 * num_kv_heads * (head_dim + I8_SCALE_BYTES)
    else:
        per_tok = kv_bytes_per_token(1, num_kv_heads, head_dim, eb)
    kv_logical = int(lens.sum()) * per_tok
    kv_unique = kv_logical - max(S - 1, 0) * shared_tokens * per_tok if shared_tokens else kv_logical
    q = S * num_q_heads * head_dim * eb
    out = S * num_q_heads * head_dim * ELEM_BYTES[out_dtype]
    tables = 4 * int(blocks.sum())
    ctx = 4 * S
    small = q + out + tables + ctx
    return {"kv_unique": kv_unique, "kv_logical": kv_logical, "q": q, "out": out,
            "tables": tables, "context_lens": ctx,
            "total": kv_unique + small, "total_logical": kv_logical + small}


def decode_flops(context_lens, num_q_heads, head_dim) -> int:
    """q.k and p.v multiply-adds: 4*D flops per (query head, context token)."""
    return 4 * head_dim * num_q_heads * int(np.asarray(context_lens, dtype=np.int64).sum())


def append_bytes(num_tokens, num_kv_heads, head_dim, dtype, cache: str = "") -> int:
    """Read new K/V rows + write them into the cache + the int64 slot mapping."""
    row = 2 * num_kv_heads * head_dim * ELEM_BYTES[dtype]
    written = 2 * num_kv_heads * (head_dim + I8_SCALE_BYTES) if cache in ("i8", "fp8") else row
    return num_tokens * (row + written + 8)
