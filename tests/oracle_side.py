"""Builds the oracle's view of a workload: pool model -> slots -> fp64 oracle.

The script of pool operations is fixed and mirrored by the GPU-side harness:
  (a) with a shared prefix: owner = create(); append(owner, prefix_len)
  (b) for s in 0..S-1: sid = fork(owner) if prefix else create();
      append(sid, own prompt length)
  (c) for each decode step: append_batch(all sids), then K/V of that step.
Copy-on-write pairs are applied to the oracle cache before the append writes.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from oracle.pool_model import PoolModel

BS = 16


@dataclasses.dataclass
class OracleState:
    pool: PoolModel
    seq_ids: list
    owner: int
    k_cache: np.ndarray
    v_cache: np.ndarray
    prompt_slots: list          # per sequence, list of slots of its own prompt tokens
    prefix_slots: list
    step_slots: list            # per step, slots in sequence order
    cow_log: list               # (phase, src, dst)


def max_blocks_for(wl, steps=None) -> int:
    steps = wl.spec.decode_steps if steps is None else steps
    return int(-(-(int(wl.prompt_lens.max()) + steps) // BS))


def build(wl, steps: int = 0) -> OracleState:
    spec = wl.spec
    Hkv, D, dt = spec.num_kv_heads, spec.head_dim, spec.dtype
    pool = PoolModel(wl.num_blocks, BS, wl.free_order)
    i8 = spec.cache in ("i8", "fp8")
    fp8 = spec.cache == "fp8"
    if i8:
        empty = oracle.empty_cache_fp8 if fp8 else oracle.empty_cache_i8
        kc, vc = empty(wl.num_blocks, Hkv, D), empty(wl.num_blocks, Hkv, D)
    else:
        kc = oracle.empty_cache(wl.num_blocks, Hkv, D, dt)
        vc = oracle.empty_cache(wl.num_blocks, Hkv, D, dt)

    def put(k, v, slots):
        if fp8:
            oracle.reshape_and_cache_fp8(k, v, kc, vc, slots, Hkv, D, wl.num_blocks, dt)
        elif i8:
            oracle.reshape_and_cache_i8(k, v, kc, vc, slots, Hkv, D, wl.num_blocks, dt)
        else:
            oracle.reshape_and_cache(k, v, kc, vc, slots, Hkv, D, wl.num_blocks, dt)

    def copy(pairs):
        if i8:
            oracle.copy_blocks_i8(kc, vc, pairs, Hkv, D)
        else:
            oracle.copy_blocks(kc, vc, pairs, Hkv, D, dt)
    cow_log = []
    owner = -1
    prefix_slots = []
    if spec.prefix_len:
        owner = pool.seq_create()
        prefix_slots, cow = pool.seq_append(owner, spec.prefix_len)
        assert cow is None
        put(wl.prefix_k, wl.prefix_v, prefix_slots)
    seq_ids, prompt_slots = [], []
    for s in range(spec.num_seqs):
        sid = pool.seq_fork(owner) if spec.prefix_len else pool.seq_create()
        seq_ids.append(sid)
        lo, hi = wl.token_offsets[s], wl.token_offsets[s + 1]
        slots, cow = pool.seq_append(sid, int(hi - lo))
        if cow is not None:
            copy(np.array([cow]))
            cow_log.append(("prompt", *cow))
        put(wl.k_tokens[lo:hi], wl.v_tokens[lo:hi], slots)
        prompt_slots.append(slots)
    st = OracleState(pool, seq_ids, owner, kc, vc, prompt_slots, prefix_slots, [], cow_log)
    for step in range(steps):
        advance(wl, st, step)
    return st


def advance(wl, st: OracleState, step: int):
    spec = wl.spec
    slots, cows = st.pool.seq_append_batch(st.seq_ids)
    i8 = spec.cache in ("i8", "fp8")
    if cows:
        if i8:
            oracle.copy_blocks_i8(st.k_cache, st.v_cache, np.array(cows), spec.num_kv_heads, spec.head_dim)
        else:
            oracle.copy_blocks(st.k_cache, st.v_cache, np.array(cows), spec.num_kv_heads,
                               spec.head_dim, spec.dtype)
        st.cow_log.extend(("step", *c) for c in cows)
    if i8:
        put = oracle.reshape_and_cache_fp8 if spec.cache == "fp8" else oracle.reshape_and_cache_i8
        put(wl.step_k[step], wl.step_v[step], st.k_cache, st.v_cache, slots, spec.num_kv_heads, spec.head_dim,
            wl.num_blocks, spec.dtype)
    else:
        oracle.reshape_and_cache(wl.step_k[step], wl.step_v[step], st.k_cache, st.v_cache, slots,
                                 spec.num_kv_heads, spec.head_dim, wl.num_blocks, spec.dtype)
    st.step_slots.append(slots)


def tables(st: OracleState, max_blocks: int):
    t, l = st.pool.export(st.seq_ids, max_blocks)
    return np.array(t, dtype=np.int32).reshape(len(st.seq_ids), max_blocks), np.array(l, dtype=np.int32)


def decode(wl, st: OracleState, max_blocks: int, nthreads: int = 0, seq_subset=None, window: int = 0):
    spec = wl.spec
    tab, lens = tables(st, max_blocks)
    q = wl.q
    if seq_subset is not None:
        tab, lens, q = tab[seq_subset], lens[seq_subset], np.ascontiguousarray(q[seq_subset])
    if spec.cache in ("i8", "fp8"):
        return oracle.decode_i8(q, spec.dtype, st.k_cache, st.v_cache, tab, lens, spec.num_kv_heads,
                                spec.fp32_scale(), nthreads=nthreads, window=window, fp8=spec.cache == "fp8")
    return oracle.decode(q, st.k_cache, st.v_cache, tab, lens, spec.num_kv_heads,
                         spec.fp32_scale(), spec.dtype, nthreads=nthreads, window=window)
