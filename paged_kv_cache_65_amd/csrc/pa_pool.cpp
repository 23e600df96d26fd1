// Host-side refcounted KV block pool (see include/pa.h for the contract).
//
// Blocks are handed out on demand from a free stack and returned at refcount
// zero ("PagedAttention vs Traditional KV Cache", section 4 "PagedAttention:
// How It Works"; "Inference serving: the KV-cache machine", section "Paged KV:
// virtual memory for tokens").  Sequences own block tables; a fork shares the
// parent's blocks, and the first write into a shared, partly filled block is
// redirected to a fresh copy ("Modern AI Infrastructure and Agentic System
// Design", section 9.1).  Every operation checks first and mutates second, so
// a failure leaves the pool exactly as it was.  Preemption by swapping
// ("Inference serving: the KV-cache machine", section "Paged KV": the private
// blocks of a block table can be swapped out and reloaded anywhere) releases a
// sequence's private suffix and later refills it with fresh blocks.
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_error.h"

struct pa_block_pool {
  struct Seq {
    std::vector<int32_t> table;
    int64_t tokens = 0;
    bool live = false;
    int32_t swapped = -1;  // blocks held elsewhere while swapped out, else -1
  };
  int32_t num_blocks = 0;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> refcount;
  std::vector<Seq> seqs;            // index = sequence id

  bool valid_block(int32_t b) const { return b >= 0 && b < num_blocks; }
  bool valid_seq(int32_t s) const {
    return s >= 0 && s < (int32_t)seqs.size() && seqs[s].live;
  }
  bool resident(int32_t s) const { return valid_seq(s) && seqs[s].swapped < 0; }

  int32_t pop() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) free_stack.push_back(b);
  }
  int32_t new_seq_id() {
    for (size_t i = 0; i < seqs.size(); ++i)
      if (!seqs[i].live) return (int32_t)i;
    seqs.emplace_back();
    return (int32_t)seqs.size() - 1;
  }
  // Blocks one sequence needs to grow by n tokens (including a copy-on-write).
  int64_t blocks_needed(const Seq &s, int64_t n) const {
    if (n == 0) return 0;
    int64_t need = 0;
    if (s.tokens % PA_BLOCK_SIZE != 0 && refcount[s.table.back()] > 1) need += 1;
    int64_t total = s.tokens + n;
    need += (total + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE - (int64_t)s.table.size();
    return need;
  }
  // Appends n tokens; the caller has checked capacity.
  void append(Seq &s, int64_t n, int64_t *slots, int32_t *cow_src, int32_t *cow_dst) {
    *cow_src = -1;
    *cow_dst = -1;
    for (int64_t k = 0; k < n; ++k) {
      if (s.tokens % PA_BLOCK_SIZE == 0) {
        s.table.push_back(pop());
      } else if (refcount[s.table.back()] > 1) {
        int32_t src = s.table.back();
        int32_t dst = pop();
        release(src);
        s.table.back() = dst;
        *cow_src = src;
        *cow_dst = dst;
      }
      slots[k] = (int64_t)s.table[s.tokens / PA_BLOCK_SIZE] * PA_BLOCK_SIZE +
                 s.tokens % PA_BLOCK_SIZE;
      ++s.tokens;
    }
  }
};

extern "C" {

pa_status pa_block_pool_create(int32_t num_blocks, int32_t block_size,
                               const int32_t *initial_free_order, pa_block_pool **out) {
  if (!out) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_create: out is NULL");
  if (block_size != PA_BLOCK_SIZE)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_block_pool_create: block_size must be %d",
                    PA_BLOCK_SIZE);
  if (num_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_create: num_blocks must be positive");
  std::vector<int32_t> order(num_blocks);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return pa::fail(PA_ERR_INVALID_ARG,
                        "pa_block_pool_create: initial_free_order is not a permutation");
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  auto *p = new (std::nothrow) pa_block_pool;
  if (!p) return pa::fail(PA_ERR_OOM, "pa_block_pool_create: host allocation failed");
  p->num_blocks = num_blocks;
  p->free_stack = std::move(order);
  p->refcount.assign(num_blocks, 0);
  *out = p;
  return PA_OK;
}

void pa_block_pool_destroy(pa_block_pool *pool) { delete pool; }

int32_t pa_block_pool_num_blocks(const pa_block_pool *pool) {
  return pool ? pool->num_blocks : -1;
}

int32_t pa_block_pool_num_free(const pa_block_pool *pool) {
  return pool ? (int32_t)pool->free_stack.size() : -1;
}

int32_t pa_block_pool_refcount(const pa_block_pool *pool, int32_t block) {
  if (!pool || !pool->valid_block(block)) return -1;
  return pool->refcount[block];
}

int32_t pa_block_pool_free_list(const pa_block_pool *pool, int32_t *out, int32_t capacity) {
  if (!pool) return -1;
  int32_t n = (int32_t)pool->free_stack.size();
  if (out)
    for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = pool->free_stack[i];
  return n;
}

pa_status pa_block_pool_alloc(pa_block_pool *pool, int32_t *block) {
  if (!pool || !block) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_alloc: NULL argument");
  if (pool->free_stack.empty()) return pa::fail(PA_ERR_OOM, "pa_block_pool_alloc: pool exhausted");
  *block = pool->pop();
  return PA_OK;
}

pa_status pa_block_pool_incref(pa_block_pool *pool, int32_t block) {
  if (!pool) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_incref: NULL pool");
  if (!pool->valid_block(block) || pool->refcount[block] == 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_incref: block %d is not allocated", block);
  ++pool->refcount[block];
  return PA_OK;
}

pa_status pa_block_pool_decref(pa_block_pool *pool, int32_t block) {
  if (!pool) return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_decref: NULL pool");
  if (!pool->valid_block(block) || pool->refcount[block] == 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_block_pool_decref: block %d is not allocated", block);
  pool->release(block);
  return PA_OK;
}

pa_status pa_seq_create(pa_block_pool *pool, int32_t *seq_id) {
  if (!pool || !seq_id) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_create: NULL argument");
  int32_t id = pool->new_seq_id();
  pool->seqs[id] = pa_block_pool::Seq();
  pool->seqs[id].live = true;
  *seq_id = id;
  return PA_OK;
}

pa_status pa_seq_fork(pa_block_pool *pool, int32_t parent, int32_t *child) {
  if (!pool || !child) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: NULL argument");
  if (!pool->valid_seq(parent))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: no sequence %d", parent);
  if (!pool->resident(parent))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_fork: sequence %d is swapped out", parent);
  int32_t id = pool->new_seq_id();  // may grow seqs: index, do not hold references
  pa_block_pool::Seq s;
  s.table = pool->seqs[parent].table;
  s.tokens = pool->seqs[parent].tokens;
  s.live = true;
  for (int32_t b : s.table) ++pool->refcount[b];
  pool->seqs[id] = std::move(s);
  *child = id;
  return PA_OK;
}

pa_status pa_seq_append(pa_block_pool *pool, int32_t seq, int32_t n_tokens, int64_t *slots,
                        int32_t *cow_src, int32_t *cow_dst) {
  if (!pool || !cow_src || !cow_dst || (n_tokens > 0 && !slots))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: NULL argument");
  if (n_tokens < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: negative n_tokens");
  if (!pool->valid_seq(seq)) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: no sequence %d", seq);
  if (!pool->resident(seq))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: sequence %d is swapped out", seq);
  auto &s = pool->seqs[seq];
  if (s.tokens + n_tokens > (int64_t)INT32_MAX)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append: sequence would exceed 2^31-1 tokens");
  if (pool->blocks_needed(s, n_tokens) > (int64_t)pool->free_stack.size())
    return pa::fail(PA_ERR_OOM, "pa_seq_append: pool exhausted");
  pool->append(s, n_tokens, slots, cow_src, cow_dst);
  return PA_OK;
}

pa_status pa_seq_append_batch(pa_block_pool *pool, const int32_t *seq_ids, int32_t n,
                              int64_t *slots, int32_t *cow_pairs, int32_t *num_cow) {
  if (!pool || !num_cow || (n > 0 && (!seq_ids || !slots || !cow_pairs)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: NULL argument");
  if (n < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: negative n");
  std::vector<char> seen(pool->seqs.size(), 0);
  // Blocks the batch takes, counted as the appends below will take them: a
  // partly filled last block shared with others is copied, and its refcount
  // drops, so when every holder is in the batch the last one in batch order
  // finds itself alone and writes in place.
  std::unordered_map<int32_t, int32_t> shared_left;  // block -> refcount as the batch goes
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t sid = seq_ids[i];
    if (!pool->valid_seq(sid))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: no sequence %d", sid);
    if (!pool->resident(sid))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: sequence %d is swapped out", sid);
    if (seen[sid]) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: duplicate sequence %d", sid);
    seen[sid] = 1;
    const auto &sq = pool->seqs[sid];
    if (sq.tokens >= (int64_t)INT32_MAX)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_append_batch: sequence %d is full", sid);
    if (sq.tokens % PA_BLOCK_SIZE == 0) {
      need += 1;  // a fresh block
    } else {
      const int32_t last = sq.table.back();
      auto it = shared_left.find(last);
      if (it == shared_left.end()) it = shared_left.emplace(last, pool->refcount[last]).first;
      if (it->second > 1) {  // copy-on-write into a fresh block, one holder fewer
        need += 1;
        --it->second;
      }
    }
  }
  if (need > (int64_t)pool->free_stack.size())
    return pa::fail(PA_ERR_OOM, "pa_seq_append_batch: pool exhausted");
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    pool->append(pool->seqs[seq_ids[i]], 1, slots + i, &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * k] = src;
      cow_pairs[2 * k + 1] = dst;
      ++k;
    }
  }
  *num_cow = k;
  return PA_OK;
}

pa_status pa_seq_free(pa_block_pool *pool, int32_t seq) {
  if (!pool) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_free: NULL pool");
  if (!pool->valid_seq(seq)) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_free: no sequence %d", seq);
  auto &s = pool->seqs[seq];
  for (int32_t b : s.table) pool->release(b);
  s = pa_block_pool::Seq();
  return PA_OK;
}

pa_status pa_seq_swap_out(pa_block_pool *pool, int32_t seq, int32_t *blocks_out, int32_t capacity,
                          int32_t *n_out) {
  if (!pool || !n_out) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_out: NULL argument");
  if (!pool->valid_seq(seq)) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_out: no sequence %d", seq);
  if (!pool->resident(seq))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_out: sequence %d is already swapped out", seq);
  auto &s = pool->seqs[seq];
  // the private blocks: the longest suffix of the table held by this sequence alone
  int32_t k = 0;
  const int32_t nb = (int32_t)s.table.size();
  while (k < nb && pool->refcount[s.table[nb - 1 - k]] == 1) ++k;
  if (k > 0 && (!blocks_out || capacity < k))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_out: %d private blocks, capacity %d", k, capacity);
  for (int32_t i = 0; i < k; ++i) {
    const int32_t b = s.table[nb - k + i];
    blocks_out[i] = b;
    pool->release(b);  // front to back, as a finished sequence frees its blocks
  }
  s.table.resize(nb - k);
  s.swapped = k;
  *n_out = k;
  return PA_OK;
}

pa_status pa_seq_swap_in(pa_block_pool *pool, int32_t seq, int32_t *blocks_out, int32_t capacity,
                         int32_t *n_out) {
  if (!pool || !n_out) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_in: NULL argument");
  if (!pool->valid_seq(seq)) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_in: no sequence %d", seq);
  auto &s = pool->seqs[seq];
  if (s.swapped < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_in: sequence %d is not swapped out", seq);
  const int32_t k = s.swapped;
  if (k > 0 && (!blocks_out || capacity < k))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_swap_in: %d blocks to restore, capacity %d", k, capacity);
  if ((size_t)k > pool->free_stack.size()) return pa::fail(PA_ERR_OOM, "pa_seq_swap_in: pool exhausted");
  for (int32_t i = 0; i < k; ++i) {
    blocks_out[i] = pool->pop();
    s.table.push_back(blocks_out[i]);
  }
  s.swapped = -1;
  *n_out = k;
  return PA_OK;
}

int32_t pa_seq_swapped_blocks(const pa_block_pool *pool, int32_t seq) {
  if (!pool || !pool->valid_seq(seq)) return -1;
  return pool->seqs[seq].swapped;
}

int32_t pa_seq_num_tokens(const pa_block_pool *pool, int32_t seq) {
  if (!pool || !pool->valid_seq(seq)) return -1;
  return (int32_t)pool->seqs[seq].tokens;
}

pa_status pa_seq_export(const pa_block_pool *pool, const int32_t *seq_ids, int32_t n,
                        int32_t max_blocks, int32_t *tables_out, int32_t *context_lens_out) {
  if (!pool || (n > 0 && (!seq_ids || !tables_out || !context_lens_out)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_export: NULL argument");
  if (n < 0 || max_blocks < 0) return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_export: negative size");
  for (int32_t i = 0; i < n; ++i) {
    if (!pool->valid_seq(seq_ids[i]))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_export: no sequence %d", seq_ids[i]);
    if (!pool->resident(seq_ids[i]))
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_export: sequence %d is swapped out", seq_ids[i]);
    if ((int64_t)pool->seqs[seq_ids[i]].table.size() > max_blocks)
      return pa::fail(PA_ERR_INVALID_ARG, "pa_seq_export: sequence %d needs %zu > %d blocks",
                      seq_ids[i], pool->seqs[seq_ids[i]].table.size(), max_blocks);
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto &s = pool->seqs[seq_ids[i]];
    int32_t *row = tables_out + (int64_t)i * max_blocks;
    size_t nb = s.table.size();
    if (nb) std::memcpy(row, s.table.data(), nb * sizeof(int32_t));
    for (int32_t j = (int32_t)nb; j < max_blocks; ++j) row[j] = -1;
    context_lens_out[i] = (int32_t)s.tokens;
  }
  return PA_OK;
}

}  // extern "C"
