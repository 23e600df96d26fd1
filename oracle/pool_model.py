"""Independent model of the refcounted KV block pool -- TEST INFRASTRUCTURE ONLY.

Plain Python, written from the pages, used to check the native pool bit for bit
(block tables, slots, copy-on-write pairs, refcounts, free-stack order).

What the pages fix, and the readings taken where they leave a choice:
  * Fixed-size blocks of 16 tokens, allocated on demand: nothing at arrival, a
    new block when the last one is full, blocks returned at completion --
    "PagedAttention vs Traditional KV Cache ...", section 4 "PagedAttention:
    How It Works" (allocation lifecycle and the block-manager snippet).
  * Free blocks form a stack: allocation pops the top, a freed block is pushed
    back (same snippet).  The "Inference serving: the KV-cache machine" Lab B
    simulator instead takes the lowest free index.  Reading taken: the stack,
    seeded with a caller-given initial order (top = last element, identity =
    0..N-1), which also lets a seeded permutation place blocks at random.
  * Blocks are refcounted; a finisher decrements, a block returns to the pool
    at refcount zero ("Inference serving ...", section "Paged KV: virtual memory
    for tokens" and Lab B; "Modern AI Infrastructure ...", section 9.1 diagram,
    refcount 3 for a prefix shared by three sequences).
  * Fork aliases the parent's table and increments every block; the first
    divergent write copies the shared block ("Inference serving ...", fork
    paragraph).  Reading taken: on append, a full (or absent) last block gets a
    fresh block and no copy; a partly filled last block with refcount > 1 is
    copied whole into a fresh block, the old one is decremented, and the table
    entry is replaced.
  * Pool exhaustion is signalled, not fatal ("PagedAttention vs Traditional KV
    Cache ...", the allocator returns "no block" to trigger preemption).
    Reading taken: every operation is all-or-nothing; on any error the state is
    unchanged.
  * Freeing a sequence decrements its blocks in table order (front to back).
  * Sequence ids: the lowest id not currently in use.
  * Preemption by swapping ("Inference serving ...", section "Paged KV" -- a
    block table lets the private blocks be swapped out and reloaded anywhere --
    and the Lab B loop): swap-out returns the victim's private blocks to the
    pool, front to back, and keeps the shared ones; swap-in takes that many
    fresh blocks from the free stack and appends them to the table.  Readings
    taken: the private blocks are the longest suffix of the table whose
    blocks have refcount 1 (blocks are shared only through forks, which share
    a prefix); swap-in is all-or-nothing; a swapped-out sequence keeps its
    token count and cannot be appended to, forked or exported until swapped
    back in; freeing it releases its resident blocks.
"""
from __future__ import annotations

BLOCK_SIZE = 16


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class PoolModel:
    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, initial_free_order=None):
        if block_size != BLOCK_SIZE:
            raise PoolError("block size must be 16")
        if num_blocks <= 0:
            raise PoolError("num_blocks must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("initial free order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = order                  # top of the stack = last element
        self.refcount = [0] * num_blocks
        self.seqs = {}                     # id -> [table(list), num_tokens, swapped blocks or None]

    # ---- blocks -----------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks("pool exhausted")
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def _check_live(self, b: int):
        if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
            raise PoolError(f"block {b} is not allocated")

    def incref(self, b: int):
        self._check_live(b)
        self.refcount[b] += 1

    def decref(self, b: int):
        self._check_live(b)
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    # ---- sequences ----------------------------------------------------------
    def _new_id(self) -> int:
        i = 0
        while i in self.seqs:
            i += 1
        return i

    def _seq(self, sid: int):
        if sid not in self.seqs:
            raise PoolError(f"no sequence {sid}")
        return self.seqs[sid]

    def _resident(self, sid: int):
        s = self._seq(sid)
        if s[2] is not None:
            raise PoolError(f"sequence {sid} is swapped out")
        return s

    def seq_create(self) -> int:
        sid = self._new_id()
        self.seqs[sid] = [[], 0, None]
        return sid

    def seq_fork(self, parent: int) -> int:
        table, ntok, _ = self._resident(parent)
        sid = self._new_id()
        for b in table:
            self.refcount[b] += 1
        self.seqs[sid] = [list(table), ntok, None]
        return sid

    def _blocks_needed(self, sid: int, n: int) -> int:
        table, ntok, _ = self.seqs[sid]
        if n == 0:
            return 0
        need = 0
        pos = ntok
        if pos % self.block_size != 0 and self.refcount[table[-1]] > 1:
            need += 1                      # copy-on-write of the shared last block
        new_total = ntok + n
        have = len(table)
        need += -(-new_total // self.block_size) - have
        return need

    def seq_append(self, sid: int, n: int = 1):
        """Append n tokens.  Returns (slots, cow) with cow = (src, dst) or None."""
        if n < 0:
            raise PoolError("negative token count")
        self._resident(sid)
        if self._blocks_needed(sid, n) > len(self.free):
            raise OutOfBlocks("pool exhausted")
        table, ntok, _ = self.seqs[sid]
        cow = None
        slots = []
        for _ in range(n):
            if ntok % self.block_size == 0:
                table.append(self.alloc())
            elif self.refcount[table[-1]] > 1:
                src = table[-1]
                dst = self.alloc()
                self.decref(src)
                table[-1] = dst
                cow = (src, dst)
            slots.append(table[ntok // self.block_size] * self.block_size + ntok % self.block_size)
            ntok += 1
        self.seqs[sid][1] = ntok
        return slots, cow

    def seq_append_batch(self, sids):
        """One token for each listed sequence, all-or-nothing.
        Returns (slots, cows) with cows a list of (src, dst) in sequence order."""
        if len(set(sids)) != len(sids):
            raise PoolError("duplicate sequence in batch")
        # blocks taken in batch order: a shared, partly filled last block is
        # copied and loses one holder, so the last of its holders in the batch
        # writes in place
        need = 0
        holders = {}
        for sid in sids:
            table, ntok, _ = self._resident(sid)
            if ntok % self.block_size == 0:
                need += 1
            else:
                last = table[-1]
                holders.setdefault(last, self.refcount[last])
                if holders[last] > 1:
                    need += 1
                    holders[last] -= 1
        if need > len(self.free):
            raise OutOfBlocks("pool exhausted")
        slots, cows = [], []
        for sid in sids:
            s, cow = self.seq_append(sid, 1)
            slots.extend(s)
            if cow is not None:
                cows.append(cow)
        return slots, cows

    def seq_free(self, sid: int):
        table = self._seq(sid)[0]
        for b in table:
            self.decref(b)
        del self.seqs[sid]

    def seq_swap_out(self, sid: int):
        """Releases the private blocks (table order) and returns their ids; the
        caller copies their contents out before the pool hands them again."""
        table = self._resident(sid)[0]
        k = 0
        while k < len(table) and self.refcount[table[len(table) - 1 - k]] == 1:
            k += 1
        out = table[len(table) - k:]
        for b in out:
            self.decref(b)
        del table[len(table) - k:]
        self.seqs[sid][2] = k
        return out

    def seq_swap_in(self, sid: int):
        """Appends fresh blocks for the swapped-out ones and returns their ids
        (table order); the caller copies the contents back into them."""
        s = self._seq(sid)
        if s[2] is None:
            raise PoolError(f"sequence {sid} is not swapped out")
        if s[2] > len(self.free):
            raise OutOfBlocks("pool exhausted")
        new = [self.alloc() for _ in range(s[2])]
        s[0].extend(new)
        s[2] = None
        return new

    def seq_swapped_blocks(self, sid: int) -> int:
        """Blocks held on the host for a swapped-out sequence, else -1."""
        s = self._seq(sid)
        return -1 if s[2] is None else s[2]

    def seq_num_tokens(self, sid: int) -> int:
        return self._seq(sid)[1]

    def seq_table(self, sid: int):
        return list(self._seq(sid)[0])

    def export(self, sids, max_blocks: int):
        """Tables padded with -1 to max_blocks, and context lengths."""
        tables, lens = [], []
        for sid in sids:
            table, ntok, _ = self._resident(sid)
            if len(table) > max_blocks:
                raise PoolError("table longer than max_blocks")
            tables.append(list(table) + [-1] * (max_blocks - len(table)))
            lens.append(ntok)
        return tables, lens
