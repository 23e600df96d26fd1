"""Pins for the oracle's multi-query ("extend") attention (no GPU).

Sequence s brings n_s new tokens, already cached, at positions L-n_s .. L-1;
query row i of it sits at p = L - n_s + i and attends to positions 0 .. p.
The pins: a hand-worked two-row case; one new token is the decode, bitwise;
every row is the decode of the sequence cut at p+1, bitwise; numpy float64
masked attention in matrix form (scores + a causal mask, softmax, times V)
on contiguous rows; rows of a sequence with more new tokens than context are
NaN.
"""
import numpy as np
import pytest

import oracle
from paged_kv_cache_65_amd import workloads
from tests import oracle_side


@pytest.fixture(scope="module", autouse=True)
def _built(oracle_lib):
    return oracle_lib


def _fresh(dtype, k, v, seed=5):
    """One sequence's rows k/v [L][Hkv][D] in a fresh pool: (k_cache, v_cache, table row, L)."""
    L, Hkv, D = k.shape
    nb = L // 16 + 3
    pool = oracle.PoolModel(nb, 16, np.random.default_rng(seed).permutation(nb))
    sid = pool.seq_create()
    slots, _ = pool.seq_append(sid, L)
    kc = oracle.empty_cache(nb, Hkv, D, dtype)
    vc = oracle.empty_cache(nb, Hkv, D, dtype)
    oracle.reshape_and_cache(k, v, kc, vc, slots, Hkv, D, nb, dtype)
    t, l = pool.export([sid], nb)
    return kc, vc, np.array(t, np.int32), np.array(l, np.int32)


def _q_rows(rng, T, Hq, D, dtype):
    return workloads.round_to(rng.standard_normal((T, Hq, D), dtype=np.float32), dtype)


def test_hand_worked_two_new_tokens():
    # L = 3 cached tokens, the last 2 new: rows at p = 1 and p = 2.  q = 0 gives
    # equal weights, V row j = e_j: row 0 = (e0 + e1)/2, row 1 = (e0 + e1 + e2)/3.
    D = 8
    k = np.random.default_rng(1).standard_normal((3, 1, D)).astype(np.float32)
    v = np.zeros((3, 1, D), np.float32)
    for j in range(3):
        v[j, 0, j] = 1.0
    kc, vc, t, l = _fresh("f32", k, v)
    q = np.zeros((2, 1, D), np.float32)
    out = oracle.extend(q, kc, vc, t, l, [0, 2], 1, 0.5, "f32")
    assert np.allclose(out[0, 0], [0.5, 0.5, 0, 0, 0, 0, 0, 0], rtol=0, atol=1e-15)
    assert np.allclose(out[1, 0], [1 / 3] * 3 + [0] * 5, rtol=0, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_new_token_per_sequence_is_the_decode_bitwise(dtype):
    wl = workloads.generate(workloads.custom(seed=31, dtype=dtype, lens=(1, 17, 64, 100), num_q_heads=8,
                                             num_kv_heads=2, head_dim=64))
    st = oracle_side.build(wl)
    mb = oracle_side.max_blocks_for(wl)
    tab, lens = oracle_side.tables(st, mb)
    dec = oracle_side.decode(wl, st, mb)
    ext = oracle.extend(wl.q, st.k_cache, st.v_cache, tab, lens, np.arange(5, dtype=np.int32), 2,
                        wl.spec.fp32_scale(), dtype)
    assert np.array_equal(ext, dec)


def test_every_row_is_the_decode_of_the_sequence_cut_at_its_position_bitwise():
    lens = (5, 40, 33, 70)
    news = (5, 3, 17, 1)          # a whole-prompt prefill, a short verify, a chunk across a block edge
    wl = workloads.generate(workloads.custom(seed=32, dtype="bf16", lens=lens, num_q_heads=8,
                                             num_kv_heads=4, head_dim=128))
    st = oracle_side.build(wl)
    mb = oracle_side.max_blocks_for(wl)
    tab, l = oracle_side.tables(st, mb)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    q = _q_rows(np.random.default_rng(33), int(qs[-1]), 8, 128, "bf16")
    ext = oracle.extend(q, st.k_cache, st.v_cache, tab, l, qs, 4, wl.spec.fp32_scale(), "bf16")
    for s, (L, n) in enumerate(zip(lens, news)):
        for i in range(n):
            t = qs[s] + i
            cut = np.array([L - n + i + 1], np.int32)
            ref = oracle.decode(np.ascontiguousarray(q[t:t + 1]), st.k_cache, st.v_cache,
                                np.ascontiguousarray(tab[s:s + 1]), cut, 4, wl.spec.fp32_scale(), "bf16")
            assert np.array_equal(ext[t], ref[0]), (s, i)


def test_matches_numpy_masked_attention_in_matrix_form():
    rng = np.random.default_rng(34)
    Hq, Hkv, D = 4, 2, 64
    for L, n in ((50, 50), (40, 7), (16, 16), (33, 2)):
        k = workloads.round_to(rng.standard_normal((L, Hkv, D), dtype=np.float32), "f16")
        v = workloads.round_to(rng.standard_normal((L, Hkv, D), dtype=np.float32), "f16")
        kc, vc, t, l = _fresh("f16", k, v, seed=L)
        q = _q_rows(rng, n, Hq, D, "f16")
        scale = float(np.float32(1 / 8))
        out = oracle.extend(q, kc, vc, t, l, [0, n], Hkv, scale, "f16")
        k64, v64, q64 = (oracle.to_float64(x, "f16") for x in (k, v, q))
        pos = np.arange(L - n, L)[:, None]                     # query positions
        mask = np.where(np.arange(L)[None, :] <= pos, 0.0, -np.inf)
        for h in range(Hq):
            sc = q64[:, h] @ k64[:, h // 2].T * scale + mask    # [n][L]
            w = np.exp(sc - sc.max(axis=1, keepdims=True))
            ref = (w / w.sum(axis=1, keepdims=True)) @ v64[:, h // 2]
            assert np.max(np.abs(out[:, h] - ref)) <= 1e-12, (L, n, h)


def test_more_new_tokens_than_context_gives_nan_rows():
    rng = np.random.default_rng(35)
    k = rng.standard_normal((10, 1, 64)).astype(np.float32)
    kc, vc, t, l = _fresh("f32", k, k)
    q = _q_rows(rng, 11, 2, 64, "f32")
    out = oracle.extend(q, kc, vc, t, l, [0, 11], 1, 0.125, "f32")
    assert np.all(np.isnan(out))
