"""Seeded synthetic inputs for paged decode attention.

This module holds input generation only -- no attention, addressing or pool
arithmetic -- so that the GPU path and the CPU oracle can be fed identical
bytes.  Nothing here imports the native library or the oracle.

Every workload is described by shapes plus one ``numpy.random.default_rng``
seed.  Draws are taken in a fixed order:
  1. context lengths (where random),
  2. the initial free-block order (a permutation of the pool) -- it places the
     sequences' blocks at random physical positions,
  3. q  [S][Hq][D],
  4. K and V rows of the prompt tokens, in logical order, sequence after
     sequence ([T][Hkv][D] each; a shared prefix is drawn once),
  5. K and V rows of the tokens appended by later decode steps.
Values are standard normal float32, rounded to nearest-even into the cache type
(fp16 through numpy's conversion, bf16 by rounding the float32 bit pattern).

The five named workloads follow the paged decode configurations this library
is measured on: a tiny fp32 case; a Llama-2-7B-shaped MHA layer (fp16); a
70B-shaped GQA layer (bf16, ragged lengths, 20000-block pool); a Llama-3-8B-
shaped GQA layer where 256 sequences share a 512-token prefix; and a
long-context decode loop (4 x 32768 tokens, 128 appended steps).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass
class Spec:
    name: str
    seed: int
    dtype: str                 # cache (and q) type: "f32", "f16" or "bf16"
    out_dtype: str             # "f32" or the cache type
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    lens: Optional[list] = None          # fixed prompt lengths, or None when drawn
    len_range: Optional[tuple] = None    # (lo, hi) inclusive uniform integers
    prefix_len: int = 0                  # tokens of a prefix shared by every sequence
    suffix_lognormal: Optional[tuple] = None  # (median, sigma, clip_hi) for suffixes
    decode_steps: int = 0                # tokens appended per sequence after the prompt
    partition_tokens: int = 0            # 0 = library default
    scale: Optional[float] = None        # None = 1/sqrt(head_dim) rounded to fp32
    cache: str = ""                      # cache type when it differs from dtype: "i8", "fp8"
                                         # (int8 or E4M3 codes + per-row scales; q, rows, out in dtype)
    window: int = 0                      # sliding window W (0 = none): the query at L-1
                                         # attends to positions L-1-W .. L-1

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def fp32_scale(self) -> float:
        s = 1.0 / math.sqrt(self.head_dim) if self.scale is None else self.scale
        return float(np.float32(s))


def named(n: int) -> Spec:
    """The measured workloads (1-based; 6 and 8 are workload 3 over an INT8 and an
    FP8 cache; 7 is a Mistral-7B-shaped batch under a 4096-token sliding window;
    9 and 10 are one GPU's share of workloads 3 and 5 when they are sharded over
    eight GPUs by KV head and by context; 11 is multi-query attention, 32 query
    heads on one shared KV head)."""
    if n == 1:
        return Spec("tiny-fp32-mha-d64", 1, "f32", "f32", 4, 4, 4, 64, 64,
                    lens=[1, 17, 33, 100], scale=1.0 / 8.0)
    if n == 2:
        return Spec("llama2-7b-mha-fp16-b8-l2048", 2, "f16", "f16", 8, 32, 32, 128, 1024,
                    lens=[2048] * 8)
    if n == 3:
        return Spec("llama70b-gqa8-bf16-b64-l128to4096", 3, "bf16", "bf16", 64, 64, 8, 128,
                    20000, len_range=(128, 4096))
    if n == 4:
        return Spec("llama3-8b-gqa4-bf16-b256-prefix512", 4, "bf16", "bf16", 256, 32, 8, 128,
                    0, prefix_len=512, suffix_lognormal=(400.0, 1.0, 8192))
    if n == 5:
        return Spec("long-ctx-gqa4-bf16-b4-l32768-128steps", 5, "bf16", "bf16", 4, 32, 8, 128,
                    8192 + 64, lens=[32768] * 4, decode_steps=128, partition_tokens=512)
    if n == 6:  # workload 3 with an INT8 cache (rows quantized on append)
        return Spec("llama70b-gqa8-int8kv-b64-l128to4096", 3, "bf16", "bf16", 64, 64, 8, 128,
                    20000, len_range=(128, 4096), cache="i8")
    if n == 8:  # workload 3 with an FP8 (E4M3) cache
        return Spec("llama70b-gqa8-fp8kv-b64-l128to4096", 3, "bf16", "bf16", 64, 64, 8, 128,
                    20000, len_range=(128, 4096), cache="fp8")
    if n == 7:  # GQA 32/8 heads, D = 128, contexts past the window
        return Spec("mistral7b-gqa4-bf16-b32-l4kto16k-sw4096", 7, "bf16", "bf16", 32, 32, 8, 128,
                    0, len_range=(4096, 16384), window=4096)
    if n == 9:  # one GPU's share of workload 3 under 8-way tensor parallelism: 1 KV head, 8 q heads
        return Spec("llama70b-tp8share-gqa8-bf16-b64-l128to4096", 3, "bf16", "bf16", 64, 8, 1, 128,
                    20000, len_range=(128, 4096))
    if n == 10:  # one GPU's share of workload 5 under 8-way context parallelism: 4096 tokens each
        return Spec("long-ctx-cp8share-gqa4-bf16-b4-l4096", 5, "bf16", "bf16", 4, 32, 8, 128,
                    1024 + 64, lens=[4096] * 4)
    if n == 11:  # multi-query attention: the Llama-3-8B shape with one KV head shared by all 32 q heads
        return Spec("llama3-8b-mqa32-bf16-b256-l128to4096", 11, "bf16", "bf16", 256, 32, 1, 128,
                    0, len_range=(128, 4096))
    raise ValueError(f"no workload {n}")


@dataclasses.dataclass
class Workload:
    spec: Spec
    prompt_lens: np.ndarray      # int32 [S] tokens cached before the first decode step
    free_order: np.ndarray       # int32 [NB] initial free stack (top = last)
    q: np.ndarray                # [S][Hq][D] cache type (np.float32/np.float16/np.uint16 bf16 bits)
    prefix_k: np.ndarray         # [P][Hkv][D] shared prefix rows (P may be 0)
    prefix_v: np.ndarray
    k_tokens: np.ndarray         # [T][Hkv][D] private prompt rows, sequence after sequence
    v_tokens: np.ndarray
    token_offsets: np.ndarray    # int64 [S+1] into k_tokens / v_tokens
    step_k: np.ndarray           # [steps][S][Hkv][D] rows appended by decode steps
    step_v: np.ndarray

    @property
    def num_blocks(self) -> int:
        return len(self.free_order)

    def seq_rows(self, s: int, which: str = "k") -> np.ndarray:
        """Contiguous prompt rows of sequence s ([L][Hkv][D]), prefix included."""
        pre = self.prefix_k if which == "k" else self.prefix_v
        tok = self.k_tokens if which == "k" else self.v_tokens
        own = tok[self.token_offsets[s]:self.token_offsets[s + 1]]
        return np.concatenate([pre, own], axis=0) if len(pre) else own


def np_cache_type(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> cache type, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    # bf16: add 0x7FFF plus the lowest kept bit, keep the high half.  In
    # chunks, in uint32 (the only inputs that wrap are negative NaNs with
    # large payloads, which wrap to 0 as the uint16 conversion would).
    u = x.view(np.uint32).reshape(-1)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 22
    for i in range(0, u.size, step):
        c = u[i:i + step]
        t = c >> 16
        t &= 1
        t += 0x7FFF
        t += c
        t >>= 16
        out[i:i + step] = t
    return out.reshape(x.shape)


def _normals(rng, shape, dtype):
    return round_to(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def generate(spec: Spec) -> Workload:
    rng = np.random.default_rng(spec.seed)
    S, Hq, Hkv, D = spec.num_seqs, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    # 1. lengths
    if spec.lens is not None:
        suffix = np.asarray(spec.lens, dtype=np.int64)
    elif spec.len_range is not None:
        lo, hi = spec.len_range
        suffix = rng.integers(lo, hi + 1, size=S, dtype=np.int64)
    elif spec.suffix_lognormal is not None:
        median, sigma, clip_hi = spec.suffix_lognormal
        z = rng.standard_normal(size=S)
        suffix = np.clip(np.rint(np.exp(np.log(median) + sigma * z)), 1, clip_hi).astype(np.int64)
    else:
        raise ValueError("spec has no lengths")
    prompt = suffix + spec.prefix_len
    nb = spec.num_blocks
    if nb == 0:  # size the pool: prefix once + private blocks + decode growth + slack
        per_seq = -(-(suffix + spec.decode_steps) // BLOCK_SIZE) + 1
        nb = spec.prefix_len // BLOCK_SIZE + int(per_seq.sum()) + 64
    # 2. block placement
    free_order = rng.permutation(nb).astype(np.int32)
    # 3. q
    q = _normals(rng, (S, Hq, D), spec.dtype)
    # 4. prompt rows
    prefix_k = _normals(rng, (spec.prefix_len, Hkv, D), spec.dtype)
    prefix_v = _normals(rng, (spec.prefix_len, Hkv, D), spec.dtype)
    offsets = np.zeros(S + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(suffix)
    T = int(offsets[-1])
    k_tokens = _normals(rng, (T, Hkv, D), spec.dtype)
    v_tokens = _normals(rng, (T, Hkv, D), spec.dtype)
    # 5. decode-step rows
    step_k = _normals(rng, (spec.decode_steps, S, Hkv, D), spec.dtype)
    step_v = _normals(rng, (spec.decode_steps, S, Hkv, D), spec.dtype)
    return Workload(spec, prompt.astype(np.int32), free_order, q, prefix_k, prefix_v,
                    k_tokens, v_tokens, offsets, step_k, step_v)


def custom(name="custom", seed=0, dtype="bf16", out_dtype=None, lens=(1, 17), num_q_heads=8,
           num_kv_heads=2, head_dim=128, num_blocks=0, prefix_len=0, decode_steps=0,
           partition_tokens=0, scale=None, cache="") -> Spec:
    """A small spec for parity sweeps; num_blocks=0 sizes the pool to fit plus slack."""
    if num_blocks == 0:
        need = sum(-(-(l + decode_steps) // BLOCK_SIZE) + 1 for l in lens)
        num_blocks = prefix_len // BLOCK_SIZE + need + 16
    return Spec(name, seed, dtype, out_dtype or dtype, len(lens), num_q_heads, num_kv_heads,
                head_dim, num_blocks, lens=list(lens), prefix_len=prefix_len,
                decode_steps=decode_steps, partition_tokens=partition_tokens, scale=scale,
                cache=cache)
