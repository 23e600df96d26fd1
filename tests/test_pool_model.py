"""Pins for the pool model (no GPU): the pages' worked examples plus invariants."""
import numpy as np
import pytest

from oracle.pool_model import PoolModel, PoolError, OutOfBlocks


def _order_popping(seq, n):
    """Initial free order whose pops yield `seq` first, then the rest ascending."""
    rest = [b for b in range(n) if b not in seq]
    return rest[::-1] + list(seq)[::-1]


def test_shared_prefix_diagram_refcount_three():
    """'Modern AI Infrastructure and Agentic System Design', section 9.1 diagram:
    A [b0,b1,b2,b3,b7], B [b0,b1,b2,b4,b8], C [b0,b1,b2,b5]; the 48-token
    system prompt (3 blocks) is shared with refcount 3."""
    pool = PoolModel(10, 16, _order_popping([0, 1, 2, 3, 4, 5, 7, 8, 6, 9], 10))
    a = pool.seq_create()
    pool.seq_append(a, 48)
    b = pool.seq_fork(a)
    c = pool.seq_fork(a)
    pool.seq_append(a, 16)
    pool.seq_append(b, 16)
    pool.seq_append(c, 16)
    pool.seq_append(a, 1)
    pool.seq_append(b, 1)
    assert pool.seq_table(a) == [0, 1, 2, 3, 7]
    assert pool.seq_table(b) == [0, 1, 2, 4, 8]
    assert pool.seq_table(c) == [0, 1, 2, 5]
    assert [pool.refcount[x] for x in (0, 1, 2)] == [3, 3, 3]
    assert pool.num_free() == 10 - 8
    for s in (a, b, c):
        pool.seq_free(s)
    assert pool.num_free() == 10 and sum(pool.refcount) == 0


def test_four_beam_fork_refcount_five_to_one():
    """'Inference serving: the KV-cache machine', Lab B tweak: a 4-beam fork
    aliasing one parent's table takes refcount 5 -> 1 as the beams finish."""
    pool = PoolModel(64)
    parent = pool.seq_create()
    pool.seq_append(parent, 40)
    beams = [pool.seq_fork(parent) for _ in range(4)]
    tab = pool.seq_table(parent)
    assert all(pool.refcount[b] == 5 for b in tab)
    for s in beams:
        pool.seq_free(s)
    assert all(pool.refcount[b] == 1 for b in tab)


def test_first_divergent_token_copies_the_shared_block():
    """Fork then append: the partly filled shared last block is copied once."""
    pool = PoolModel(16)
    parent = pool.seq_create()
    pool.seq_append(parent, 20)              # blocks: full + 4 tokens
    child = pool.seq_fork(parent)
    last = pool.seq_table(parent)[-1]
    slots, cow = pool.seq_append(child, 3)
    assert cow is not None and cow[0] == last
    dst = cow[1]
    assert pool.seq_table(child) == pool.seq_table(parent)[:-1] + [dst]
    assert slots == [dst * 16 + 4, dst * 16 + 5, dst * 16 + 6]
    assert pool.refcount[last] == 1 and pool.refcount[dst] == 1
    # parent's own append now finds its block private: no copy
    _, cow2 = pool.seq_append(parent, 1)
    assert cow2 is None


def test_fork_at_block_boundary_needs_no_copy():
    pool = PoolModel(16)
    p = pool.seq_create()
    pool.seq_append(p, 32)
    c = pool.seq_fork(p)
    _, cow = pool.seq_append(c, 1)
    assert cow is None
    assert pool.seq_table(c)[:2] == pool.seq_table(p)


def test_500_tokens_use_32_blocks():
    """'LLM Inference Optimization ...', section 'PagedAttention: OS Concepts Meet
    GPU Memory': a 500-token response uses ceil(500/16) = 32 blocks."""
    pool = PoolModel(100)
    s = pool.seq_create()
    pool.seq_append(s, 500)
    assert len(pool.seq_table(s)) == 32 and pool.num_free() == 68


def test_hundred_requests_pay_the_prefix_once():
    """'Inference serving ...', section 'Paged KV: virtual memory for tokens':
    100 requests behind the same ~512-token prompt map the same 32 blocks."""
    pool = PoolModel(4000)
    owner = pool.seq_create()
    pool.seq_append(owner, 512)
    reqs = [pool.seq_fork(owner) for _ in range(100)]
    assert 4000 - pool.num_free() == 32
    assert pool.refcount[pool.seq_table(owner)[0]] == 101
    for r in reqs:
        pool.seq_free(r)
    pool.seq_free(owner)
    assert pool.num_free() == 4000


def test_out_of_blocks_leaves_state_unchanged():
    pool = PoolModel(4)
    s = pool.seq_create()
    pool.seq_append(s, 40)                    # 3 blocks
    snap = (list(pool.free), list(pool.refcount), pool.seq_table(s), pool.seq_num_tokens(s))
    with pytest.raises(OutOfBlocks):
        pool.seq_append(s, 30)                # needs 2 more, 1 free
    assert snap == (list(pool.free), list(pool.refcount), pool.seq_table(s), pool.seq_num_tokens(s))
    t = pool.seq_create()
    pool.seq_append(t, 16)
    with pytest.raises(OutOfBlocks):
        pool.seq_append_batch([s, t])         # s fits in its block, t needs one, none free
    with pytest.raises(OutOfBlocks):
        pool.alloc()
    pool.seq_free(t)                          # recovery: free and retry
    pool.seq_append(s, 8)


def test_errors_on_bad_ids_and_underflow():
    pool = PoolModel(4)
    with pytest.raises(PoolError):
        pool.decref(0)
    with pytest.raises(PoolError):
        pool.incref(7)
    with pytest.raises(PoolError):
        pool.seq_append(3, 1)
    with pytest.raises(PoolError):
        PoolModel(4, 16, [0, 1, 1, 3])


def test_lifo_reuse_and_lowest_free_sequence_id():
    pool = PoolModel(8)
    a = pool.seq_create()
    b = pool.seq_create()
    pool.seq_append(a, 17)                    # pops 7, 6
    assert pool.seq_table(a) == [7, 6]
    pool.seq_free(a)                          # pushes 7 then 6 -> 6 on top
    assert pool.free[-2:] == [7, 6]
    c = pool.seq_create()
    assert c == a and b == 1
    pool.seq_append(c, 1)
    assert pool.seq_table(c) == [6]


def test_randomized_scripts_keep_invariants():
    rng = np.random.default_rng(0)
    for trial in range(20):
        n = int(rng.integers(8, 64))
        pool = PoolModel(n, 16, rng.permutation(n))
        live = []
        for _ in range(300):
            op = rng.integers(0, 5)
            try:
                if op == 0 or not live:
                    live.append(pool.seq_create())
                elif op == 1:
                    live.append(pool.seq_fork(live[rng.integers(len(live))]))
                elif op == 2:
                    pool.seq_append(live[rng.integers(len(live))], int(rng.integers(0, 40)))
                elif op == 3:
                    pool.seq_free(live.pop(rng.integers(len(live))))
                else:
                    k = int(rng.integers(1, len(live) + 1))
                    pool.seq_append_batch(list(rng.choice(live, size=k, replace=False)))
            except OutOfBlocks:
                pass
            held = sum(len(pool.seq_table(s)) for s in live)
            assert sum(pool.refcount) == held
            assert pool.num_free() == sum(1 for r in pool.refcount if r == 0)
            assert sorted(pool.free) == [b for b in range(n) if pool.refcount[b] == 0]
            for s in live:
                assert len(pool.seq_table(s)) == -(-pool.seq_num_tokens(s) // 16)
        for s in live:
            pool.seq_free(s)
        assert pool.num_free() == n


# ---------------------------------------------------------------- swap (preemption)
def test_swap_out_releases_the_private_suffix_and_swap_in_refills_from_the_stack():
    # Identity order: the stack top is block 9.  The owner of a 32-token shared
    # prefix takes 9, 8; A forks it and grows by 40 tokens into 7, 6, 5.
    # Swap-out pushes 7, 6, 5 (front to back) and keeps 9, 8; swap-in pops
    # 5, 6, 7 back into the table: [9, 8, 5, 6, 7].
    pool = PoolModel(10)
    owner = pool.seq_create()
    pool.seq_append(owner, 32)
    a = pool.seq_fork(owner)
    pool.seq_append(a, 40)
    assert pool.seq_table(a) == [9, 8, 7, 6, 5] and pool.num_free() == 5
    out = pool.seq_swap_out(a)
    assert out == [7, 6, 5]
    assert pool.seq_table(a) == [9, 8] and pool.seq_num_tokens(a) == 72
    assert pool.free == [0, 1, 2, 3, 4, 7, 6, 5] and pool.seq_swapped_blocks(a) == 3
    assert pool.refcount[9] == pool.refcount[8] == 2      # the prefix stays shared
    new = pool.seq_swap_in(a)
    assert new == [5, 6, 7] and pool.seq_table(a) == [9, 8, 5, 6, 7]
    assert pool.seq_swapped_blocks(a) == -1 and pool.free == [0, 1, 2, 3, 4]


def test_swapped_out_sequence_is_frozen_until_swapped_in():
    pool = PoolModel(8)
    a = pool.seq_create()
    pool.seq_append(a, 20)
    pool.seq_swap_out(a)
    for call in (lambda: pool.seq_append(a, 1), lambda: pool.seq_append_batch([a]),
                 lambda: pool.seq_fork(a), lambda: pool.export([a], 4), lambda: pool.seq_swap_out(a)):
        with pytest.raises(PoolError):
            call()
    b = pool.seq_create()
    with pytest.raises(PoolError):
        pool.seq_swap_in(b)                                # resident
    pool.seq_append(b, 16 * 7)                             # takes all 7 free blocks but one
    before = (list(pool.free), list(pool.refcount), pool.seq_table(a))
    with pytest.raises(OutOfBlocks):
        pool.seq_swap_in(a)                                # needs 2, 1 free
    assert (list(pool.free), list(pool.refcount), pool.seq_table(a)) == before
    pool.seq_free(b)
    assert pool.seq_swap_in(a) and pool.seq_num_tokens(a) == 20
    pool.seq_swap_out(a)
    pool.seq_free(a)                                       # frees what is resident
    assert pool.num_free() == 8


def test_swap_out_keeps_a_shared_last_block():
    # a fork shares every block, including the partly filled last one: nothing
    # is private, so swap-out releases nothing and swap-in takes nothing
    pool = PoolModel(6)
    a = pool.seq_create()
    pool.seq_append(a, 20)
    b = pool.seq_fork(a)
    assert pool.seq_swap_out(a) == [] and pool.seq_swapped_blocks(a) == 0
    assert pool.seq_table(a) == pool.seq_table(b) and pool.refcount[5] == 2
    assert pool.seq_swap_in(a) == [] and pool.seq_swapped_blocks(a) == -1


def test_a_batch_of_every_holder_of_a_shared_block_fits_a_tight_pool():
    """Worked by hand: a parent with 20 tokens (a full block and one with 4
    tokens) and its fork share both blocks; one block is free.  Appending one
    token to both copies the shared partly filled block once: the first in the
    batch takes the free block, and the second, now its only holder, writes
    in place.  The batch fits; so would the same appends one after another."""
    for first_parent in (True, False):
        pool = PoolModel(3, 16, [2, 1, 0])            # pops 0, 1, 2
        p = pool.seq_create()
        pool.seq_append(p, 20)
        assert pool.seq_table(p) == [0, 1]
        c = pool.seq_fork(p)
        assert pool.refcount[1] == 2 and pool.num_free() == 1
        batch = [p, c] if first_parent else [c, p]
        slots, cows = pool.seq_append_batch(batch)
        assert cows == [(1, 2)]
        copier, stayer = batch
        assert pool.seq_table(copier) == [0, 2] and pool.seq_table(stayer) == [0, 1]
        assert slots == [2 * 16 + 4, 1 * 16 + 4]
        assert pool.refcount[1] == 1 and pool.refcount[2] == 1 and pool.num_free() == 0
        # a third sequence needing a block of its own does not fit: nothing changes
        snap = (list(pool.free), list(pool.refcount), pool.seq_table(p), pool.seq_table(c))
        q = pool.seq_create()
        with pytest.raises(OutOfBlocks):
            pool.seq_append_batch([p, c, q])
        assert snap == (list(pool.free), list(pool.refcount), pool.seq_table(p), pool.seq_table(c))
