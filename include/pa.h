/*
 * pa.h -- C ABI of libpa: paged decode attention on AMD MI355X (gfx950).
 *
 * The library exports these groups of calls:
 *   1. pa_decode            paged decode attention (one new query per sequence;
 *                           optional sliding window, shared prefix, fused
 *                           append); pa_decode_partitions + pa_decode_merge
 *                           run it as two launches
 *   2. pa_extend            the same attention for several new tokens per
 *                           sequence (chunked prefill, speculative verify)
 *   3. pa_reshape_and_cache append new tokens' K/V into the block pool through
 *      pa_copy_blocks       a slot mapping; whole-block copies for copy-on-write
 *                           (_int8 / _fp8 variants quantize into byte caches)
 *   4. pa_swap_blocks       block copies between a device cache and a pinned
 *                           host pool (preemption)
 *   5. pa_block_pool_* /    a host-side refcounted block pool that owns block
 *      pa_seq_*             tables, hands out slots, decides copy-on-write and
 *                           swaps sequences out and in
 *
 * Conventions (all calls):
 *   - Every call returns pa_status; nothing throws or aborts across the ABI.
 *     On any error no kernel is launched and no pool state changes;
 *     pa_last_error() returns a thread-local message for the last failure.
 *   - Device calls take raw device pointers owned by the caller and a HIP
 *     stream (hipStream_t passed as void*, NULL = the default stream).  They
 *     enqueue work asynchronously and never synchronize.  The library
 *     allocates no device memory: the decode workspace is caller-provided.
 *   - Every device pointer must be 16-byte aligned; one for an array with no
 *     elements (no sequences, no query rows, a table with no columns) may be
 *     NULL.
 *   - Block size is fixed at PA_BLOCK_SIZE = 16 tokens.
 *
 * Cache layout (one layer).  k_cache and v_cache each hold num_blocks physical
 * blocks; block b holds, for every KV head g, one tile of 16 tokens x head_dim
 * dims starting at element (b * num_kv_heads + g) * 16 * head_dim.  With
 * X = 16 / sizeof(element) (8 for fp16/bf16, 4 for fp32):
 *   K tile, [head_dim/X][16][X]:  (t, d) -> (d / X)*16*X + t*X + d % X
 *   V tile, slabs of 4X dims, 64 16-byte vectors per slab, each vector holding
 *   X/4 dims x 4 consecutive tokens (dim-major):
 *     (t, d) -> (d / (4X))*64*X + ((t / 4)*16 + (d % (4X)) % 16)*X
 *               + ((d % (4X)) / 16)*4 + t % 4
 * Both tiles are layouts of this library's own choosing (the pages leave the
 * in-block order open): one 16-byte load per lane then hands each lane of a
 * 64-wide wavefront exactly the operand fragment the matrix-core tiles use.
 *
 * INT8 caches.  Row (token t, KV head g) of K (and of V) is stored as
 * head_dim int8 codes c and one float32 scale sc, standing for the values
 * c * sc.  Quantization ("KV Cache Explained Like You're an LLM Engineer",
 * section "Future Optimizations", subsection "KV Cache Quantization"):
 * sc = max_d |x_d| / 127 and c_d = x_d / sc truncated toward zero, both in
 * float32 (an all-zero row has sc = 0, codes 0).  A byte cache (K or V) is
 * one array of tiles of 16*(head_dim + 4) bytes, tile (b, g) at byte
 * (b*num_kv_heads + g)*16*(head_dim + 4): the 16 rows' codes, then their 16
 * float32 scales, so one (block, head) is one contiguous run.  In a tile:
 *   K code (t, d) -> (c*64 + q*16 + t)*16 + h*8 + e,  with c = d/64, w = d%64,
 *                    h = w/32, q = (w%32)/8, e = w%8
 *   V code (t, d) -> (m*64 + (t/4)*16 + d%16)*16 + ((d%64)/16)*4 + t%4,
 *                    m = d/64
 *   scale of t   -> bytes 16*head_dim + 4t .. +3 (float32)
 * (again one 16-byte lane load per operand fragment).
 *
 * FP8 caches (PA_FP8): the same tiles and scales with OCP E4M3 codes (sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 subnormal,
 * S.1111.111 NaN, largest finite 448) standing for value(c) * sc, with
 * sc = max_d |x_d| / 448 and c_d the E4M3 value nearest to x_d / sc (float32
 * division), ties to the even code, saturating at +-448 -- the int8 recipe
 * above with FP8's range ("Inference serving: the KV-cache machine", What
 * insiders know, names an fp8 KV cache with per-head scales but no recipe).
 * pa_copy_blocks_int8 and pa_swap_blocks_int8 move the tiles (codes and
 * scales) of either kind of byte cache.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16
/* pa_decode_params.partition_tokens value that asks for the balanced split */
#define PA_PARTITION_BALANCED (-1)
/* Size of the per-device workspace pa_decode_noalloc uses (64 MiB) */
#define PA_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* a null pointer, a size or an id out of range */
  PA_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement */
  PA_ERR_WORKSPACE = 3,    /* the decode workspace is missing or too small */
  PA_ERR_OOM = 4,          /* the block pool has too few free blocks */
  PA_ERR_HIP = 5           /* a HIP runtime call failed (e.g. launch error) */
} pa_status;

/* PA_I8 / PA_FP8: a cache of int8 / E4M3 codes with one float32 scale per
 * (token, KV head) row (see "INT8 caches" and "FP8 caches" above); never a q
 * or output type. */
typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_I8 = 3, PA_FP8 = 4 } pa_dtype;

/* Which decode kernel runs.  AUTO picks the matrix-core kernel for fp16/bf16
 * caches and the vector-ALU kernel for fp32. */
typedef enum pa_kernel { PA_KERNEL_AUTO = 0, PA_KERNEL_VALU = 1, PA_KERNEL_MFMA = 2 } pa_kernel;

/* Library version string. */
const char *pa_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *pa_last_error(void);

/* ------------------------------------------------------------------------
 * Paged decode attention.
 *
 * For every sequence s < num_seqs and query head h < num_q_heads, with
 * G = num_q_heads / num_kv_heads, kv head g = h / G (contiguous groups of
 * query heads share one KV head) and L = context_lens[s]:
 *   score_i = scale * sum_d q[s][h][d] * K(s, i, g, d),   i < L
 *   out[s][h][:] = sum_i softmax(score)_i * V(s, i, g, :)
 * where K(s, i, g, d) is element (i % 16, d) of tile (block_tables[s][i / 16],
 * g) in k_cache, and V likewise.  This is softmax(q.K^T / sqrt(d)).V for one
 * new query ("KV Cache Explained Like You're an LLM Engineer", section
 * "Transformer Attention: A Quick Refresher"), gathered block by block through
 * a per-sequence table ("LLM Inference Optimization: KV-Cache, PagedAttention,
 * and GPU Memory Efficiency", section "PagedAttention: OS Concepts Meet GPU
 * Memory"), with grouped-query head sharing ("Inference serving: the KV-cache
 * machine", section "The KV cache: attention's memory bill, derived").  The
 * context counts the token appended this step.  L = 0 yields a zero row.
 *
 * The work is split into pieces, each reduced with an online softmax into a
 * (max, sum, weighted V) partial, which a second kernel merges by
 * log-sum-exp rescaling.  Two splits exist:
 *   - partitions: every context is cut into partition_tokens-token pieces,
 *     one workgroup per (piece, KV head, sequence);
 *   - balanced (the matrix-core path, at most 1024 sequences and 2^15
 *     (sequence, KV head) pairs): all (sequence, KV head, 16-token block)
 *     units are cut into equal contiguous shares, one per wave of a grid
 *     that fills every CU once, whatever the length mix.
 * The result does not depend on the split beyond float32 rounding; it is
 * deterministic for a given device (the balanced shares depend on its CU
 * count).
 *
 * Arguments (all pointers are device memory):
 *   out           [num_seqs][num_q_heads][head_dim], out_dtype (F32 or kv_dtype;
 *                 a 16-bit output is the float32 result rounded to nearest even)
 *   q             [num_seqs][num_q_heads][head_dim], kv_dtype
 *   k_cache, v_cache  [num_blocks] blocks in the layout above, kv_dtype
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; only the first
 *                 ceil(L/16) entries of a row are read
 *   context_lens  int32 [num_seqs]
 *   max_context_len  host-known upper bound on every context_lens[s]; it sizes
 *                 the launch grid
 *   scale         usually 1/sqrt(head_dim)
 *   partition_tokens  0 = automatic: the balanced split where it applies
 *                 and the batch holds at least 48 units per wave at
 *                 max_context_len (always for INT8/FP8 caches and a shared
 *                 prefix); for a smaller batch on the matrix-core path,
 *                 partitions giving about one workgroup per compute unit
 *                 (one per (sequence, KV head) pair, with no merge, once the
 *                 pairs outnumber the compute units); else partitions of
 *                 1024, 512 or 256 tokens, the largest that gives >= 8
 *                 workgroups per compute unit.  Under a sliding window W the
 *                 partitions cover the attended range, at most W + 16
 *                 tokens.  PA_PARTITION_BALANCED (-1) = the balanced split
 *                 (an error where it cannot run).  A positive multiple of
 *                 16 = partitions of that size.
 * Supported: head_dim in {64, 128}; num_q_heads % num_kv_heads == 0;
 *   G <= 64 (up to multi-query attention, every query head on one KV head:
 *   "Inference serving: the KV-cache machine", section "The KV cache:
 *   attention's memory bill, derived"); fp16/bf16 with any kernel, fp32
 *   with the VALU kernel.  The matrix-core kernels read every K/V block once
 *   for all G heads (ceil(G/16) score tiles per block); the VALU kernel takes
 *   a group of more than 16 heads as 16-head chunks, one workgroup each.
 * Contract violations found on the device (a table entry outside
 * [0, num_blocks), or L outside [0, min(max_context_len,
 * 16*max_blocks_per_seq)]) are never dereferenced: that sequence's output row
 * is set to NaN.
 * Workspace: pa_decode_workspace_bytes() bytes of device memory (0 when no
 * context is split); scratch for this call only (no initialization needed),
 * reusable by any later call once the stream has passed this one.  Under the
 * balanced split its size depends on the current device's CU count: query it
 * with that device current.
 * ------------------------------------------------------------------------ */
typedef struct pa_decode_params {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t max_context_len;
  float scale;
  pa_dtype kv_dtype;
  pa_dtype out_dtype;
  int32_t partition_tokens;
  pa_kernel kernel;
  /* Optional fused append (all three set, or all NULL).  Equivalent to
   * pa_reshape_and_cache(k_new, v_new, ..., slot_mapping, num_seqs) followed
   * by the decode, for a decode step that appends one token per sequence:
   *   k_new, v_new  [num_seqs][num_kv_heads][head_dim], kv_dtype (q_dtype
   *                 for an INT8/FP8 cache, below)
   *   slot_mapping  int64 [num_seqs]: the slot of position context_lens[s]-1,
   *                 i.e. block_tables[s][(L-1)/16]*16 + (L-1)%16, or negative
   *                 for no append.  Any other slot writes nothing and makes
   *                 that sequence's row NaN.
   * A block written this way must be private to its sequence (copy-on-write
   * copies done beforehand with pa_copy_blocks / pa_copy_blocks_int8). */
  const void *k_new;
  const void *v_new;
  const int64_t *slot_mapping;
  /* INT8 and FP8 caches (kv_dtype = PA_I8 or PA_FP8) only, else ignored: the
   * type of q (F16 or BF16; out_dtype is F32 or q_dtype).  k_cache / v_cache
   * are then byte caches (codes and row scales in their tiles, above).
   * Decoding a byte cache needs the matrix-core kernel and automatic
   * partitioning (the balanced split).  With a byte cache the fused append's
   * k_new / v_new rows are q_dtype (F16 or BF16) and are quantized exactly as
   * pa_reshape_and_cache_int8 / _fp8 quantize them (codes and the scale
   * written to the cache, the same values attended). */
  pa_dtype q_dtype;
  /* Optional hipEvent_t handles (NULL = none), created by the caller.  They
   * are recorded from the kernel dispatches' own start and end times
   * (hipExtLaunchKernel), so timing a launch adds no marker to the stream:
   *   pa_decode_partitions  start and end of the attention kernel;
   *   pa_decode_merge       start and end of the merge kernel;
   *   pa_decode             start of the attention kernel, end of the last
   *                         kernel of the call.
   * A call that launches nothing (no sequences, or no merge needed) records
   * the given events on the stream instead, so they always complete after
   * the call's work.  The events are not read back by the library. */
  void *start_event;
  void *stop_event;
  /* Sliding window ("KV Cache Explained Like You're an LLM Engineer", section
   * "Future Optimizations", subsection "Sliding Window Attention": token i
   * attends to [i-W, i]).  0 = none.  W > 0: the query of sequence s, at position
   * L-1, attends to positions max(0, L-1-W) .. L-1 (W+1 tokens, both ends
   * included).  Table entries of blocks wholly before position L-1-W are
   * never read (they may be -1 or stale); negative values are rejected. */
  int32_t sliding_window;
  /* Shared prefix (0 = none): the first shared_prefix_blocks entries of every
   * sequence's table are the same physical blocks (sequence 0's row is read
   * for them; the other rows' entries there are not), as when every sequence
   * forks one prefix owner ("Modern AI Infrastructure and Agentic System
   * Design", section 9.1; "Inference serving: the KV-cache machine", Lab B).
   * The attention over the prefix is then computed once for all sequences
   * (a third kernel, on a second stream the library owns, beside the
   * attention launch of pa_decode / pa_decode_partitions; the caller's
   * stream waits for it right after that launch) and folded into each row;
   * the result is the same attention.  Needs an fp16/bf16 cache, no sliding window and the balanced
   * split; every context must reach past the prefix (L > 16 *
   * shared_prefix_blocks, else that sequence's rows are NaN).  The workspace
   * grows by num_seqs * num_q_heads * (head_dim + 2) floats. */
  int32_t shared_prefix_blocks;
} pa_decode_params;

/* Partition size (tokens) pa_decode will use for these parameters, 0 for the
 * balanced split, or a negative pa_status value if the parameters are
 * invalid. */
int32_t pa_decode_partition_tokens(const pa_decode_params *p);

/* Workspace bytes pa_decode needs for these parameters (0 if the whole context
 * fits one partition).  Returns 0 for invalid parameters as well; pa_decode
 * reports those. */
size_t pa_decode_workspace_bytes(const pa_decode_params *p);

pa_status pa_decode(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                    void *stream);

/* pa_decode in its two launches, for callers that time, overlap or combine
 * them; together they write every output row, and they give the same bits
 * as pa_decode.  Under the balanced split the workspace holds partials in an
 * internal layout and pa_decode_merge must follow pa_decode_partitions on
 * the same workspace.  With partitions, pa_decode_partitions writes the final
 * rows of sequences whose context fits one partition, and for the others one
 * partial per (sequence, query head, partition) into the workspace:
 *   float32 [num_seqs][num_q_heads][P][2]  (m, l): m = max score in log2
 *           units (score * log2(e)), l = sum of 2^(score*log2(e) - m)
 *   float32 [num_seqs][num_q_heads][P][head_dim]  sum of 2^(...) * V rows
 * (the second array follows the first; P = ceil(max_context_len /
 * partition_tokens)).  pa_decode_merge folds those partials into the output
 * rows: M = max_p m_p, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
 *
 * Partials of one sequence computed elsewhere (e.g. other devices holding
 * other context ranges) can be merged the same way.  Both calls take the same
 * parameters and workspace as pa_decode. */
pa_status pa_decode_partitions(const pa_decode_params *p, void *workspace,
                               size_t workspace_bytes, void *stream);
pa_status pa_decode_merge(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                          void *stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a fixed array inside the library
 * of PA_NOALLOC_WORKSPACE_BYTES bytes (64 MiB), one copy per
 * device, held from the first call on a device until the process ends; the
 * call itself allocates nothing.  A call whose pa_decode_workspace_bytes()
 * exceeds that size returns PA_ERR_WORKSPACE and launches nothing.  Every
 * call on one device shares that device's array: calls that overlap on the
 * device (on different streams, or from several host threads without stream
 * order between them) race on it and give undefined results.  The output is
 * the same, bit for bit, as pa_decode's for the same parameters (with a
 * shared prefix its kernel runs before the split on the caller's stream, not
 * beside it on a stream of the library's).  The first
 * call on a device looks up the array's address there (that device must be
 * current); other errors as pa_decode. */
pa_status pa_decode_noalloc(const pa_decode_params *p, void *stream);

/* ------------------------------------------------------------------------
 * KV append through a slot mapping.
 * For each new token n < num_tokens with slot s = slot_mapping[n] >= 0, and
 * every kv head g: K row k_new[n][g][:] becomes element (s % 16, :) of tile
 * (s / 16, g) in k_cache; likewise v_new into v_cache.  Negative slots are
 * skipped; slots >= 16*num_blocks are skipped too (contract violation).
 * Appending the new token's K/V before attending is the decode step of "KV
 * Cache Explained Like You're an LLM Engineer", section "What KV Cache
 * Stores".  Bytes are copied unchanged (bit-exact).
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping  int64 [num_tokens] (device)
 * Two tokens mapped to one slot leave either row there (no ordering).
 * ------------------------------------------------------------------------ */
pa_status pa_reshape_and_cache(const void *k_new, const void *v_new, void *k_cache,
                               void *v_cache, const int64_t *slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                               pa_dtype dtype, void *stream);

/* pa_reshape_and_cache into an INT8 cache: each (token, KV head) row of
 * k_new / v_new (src_dtype F16 or BF16) is quantized as described under
 * "INT8 caches" and stored with its scale in its tile.  Codes and scales are
 * bit-exact with that definition (float32 division, correctly rounded). */
pa_status pa_reshape_and_cache_int8(const void *k_new, const void *v_new, int8_t *k_cache,
                                    int8_t *v_cache, const int64_t *slot_mapping, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                    pa_dtype src_dtype, void *stream);

/* ------------------------------------------------------------------------
 * Whole-block copies for copy-on-write: for each pair i, block
 * src_dst_pairs[2i] (all heads, K and V) is copied to block src_dst_pairs[2i+1]
 * ("Modern AI Infrastructure and Agentic System Design", section 9.1: a write
 * to a shared block is copied into a fresh block first).  Pairs are applied in
 * parallel: a block may not be both a source and a destination in one call.
 * Pairs with an id outside [0, num_blocks) are skipped.
 *   src_dst_pairs int32 [num_pairs][2] (device)
 * ------------------------------------------------------------------------ */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t num_blocks, pa_dtype dtype, void *stream);

/* ------------------------------------------------------------------------
 * Multi-query ("extend") attention: several new tokens per sequence, each
 * attending causally ("Inference serving: the KV-cache machine": chunked
 * prefill interleaves ~2k-token prompt chunks with decode; speculative
 * decoding verifies k drafted tokens in one pass).  Sequence s brings
 * n_s = query_start[s+1] - query_start[s] new tokens whose K/V are already in
 * the cache (pa_reshape_and_cache) at positions L-n_s .. L-1, L =
 * context_lens[s]; query row t = query_start[s] + i is the token at position
 * p = L - n_s + i and attends to positions 0 .. p:
 *   out[t][h] = softmax_j(scale * q[t][h] . K[j][g]) V[j][g], j = 0 .. p,
 *   g = h / (num_q_heads / num_kv_heads).
 *   q, out      [num_query_rows][num_q_heads][head_dim] (out F32 or kv_dtype,
 *               16-bit outputs rounded to nearest even from float32)
 *   query_start int32 [num_seqs + 1], ascending, query_start[0] = 0 and
 *               query_start[num_seqs] = num_query_rows (device)
 *   max_query_len >= every n_s, max_context_len >= every L (host bounds)
 * fp16 / bf16 caches, head_dim 64 or 128, up to 64 query heads per KV head.
 * A sequence with n_s > L, L outside [0, max_context_len] or beyond its
 * table row, or n_s > max_query_len, or a table entry outside the pool, gets
 * NaN rows (never dereferenced); a sequence whose rows fall outside
 * [0, num_query_rows) is skipped (nothing read or written).  n_s = 1 for every
 * sequence is the decode.
 * Workspace: pa_extend_workspace_bytes() (0 without split contexts); events
 * as for pa_decode (start of the attention kernel, end of the last kernel).
 * ------------------------------------------------------------------------ */
typedef struct pa_extend_params {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;
  int32_t num_seqs;
  int32_t num_query_rows;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t max_context_len;
  int32_t max_query_len;
  float scale;
  pa_dtype kv_dtype;
  pa_dtype out_dtype;
  int32_t partition_tokens; /* 0 = automatic; else a multiple of 16 */
  void *start_event;
  void *stop_event;
} pa_extend_params;

/* Partition size in tokens pa_extend will use, or a negative pa_status. */
int32_t pa_extend_partition_tokens(const pa_extend_params *p);
size_t pa_extend_workspace_bytes(const pa_extend_params *p);
pa_status pa_extend(const pa_extend_params *p, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Swap copies: whole blocks (all heads, K and V) between two pools of the
 * same tile layout, for preemption by swapping ("Inference serving: the
 * KV-cache machine", section "Paged KV": a block table lets a sequence's
 * private blocks be swapped out and reloaded anywhere; the Lab B loop swaps a
 * victim to CPU DRAM and back into new blocks).  Either pool may be device
 * memory or pinned host memory the GPU can address (hipHostMalloc, or a
 * PyTorch tensor made with pin_memory=True).  For each pair i, block
 * src_dst_pairs[2i] of the source pool is copied to block src_dst_pairs[2i+1]
 * of the destination pool; pairs outside [0, src_num_blocks) or
 * [0, dst_num_blocks) are skipped.
 *   src_dst_pairs int32 [num_pairs][2], device or pinned host memory;
 *                 num_pairs <= 65535 per call.
 * Asynchronous like every device call: a host-side pool is complete after
 * the stream passes the call, and must not be changed before then.  Swap a
 * sequence out with pa_seq_swap_out, then copy its released blocks before
 * anything on the stream writes into them again (stream order suffices).
 * ------------------------------------------------------------------------ */
pa_status pa_swap_blocks(const void *src_k, const void *src_v, int32_t src_num_blocks, void *dst_k,
                         void *dst_v, int32_t dst_num_blocks, const int32_t *src_dst_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                         void *stream);

/* pa_swap_blocks for INT8 and FP8 caches: the tiles (codes and row scales)
 * of every head. */
pa_status pa_swap_blocks_int8(const int8_t *src_k, const int8_t *src_v, int32_t src_num_blocks,
                              int8_t *dst_k, int8_t *dst_v, int32_t dst_num_blocks,
                              const int32_t *src_dst_pairs, int32_t num_pairs, int32_t num_kv_heads,
                              int32_t head_dim, void *stream);

/* pa_reshape_and_cache_int8 for an FP8 (E4M3) cache: codes and scales are
 * bit-exact to the recipe under "FP8 caches". */
pa_status pa_reshape_and_cache_fp8(const void *k_new, const void *v_new, uint8_t *k_cache,
                                   uint8_t *v_cache, const int64_t *slot_mapping, int32_t num_tokens,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                   pa_dtype src_dtype, void *stream);

/* pa_copy_blocks for an INT8 or FP8 cache: the tiles (codes and scales) of
 * every head. */
pa_status pa_copy_blocks_int8(int8_t *k_cache, int8_t *v_cache, const int32_t *src_dst_pairs,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_blocks, void *stream);

/* ------------------------------------------------------------------------
 * Host-side block pool.  Blocks are allocated on demand and returned when
 * their refcount reaches zero ("PagedAttention vs Traditional KV Cache",
 * section 4 "PagedAttention: How It Works"; "Inference serving: the KV-cache
 * machine", section "Paged KV: virtual memory for tokens").
 *   - Free blocks form a stack: allocation pops the top; a block whose
 *     refcount reaches zero is pushed.  initial_free_order (host, nullable)
 *     seeds the stack bottom-to-top; NULL means 0..num_blocks-1 (so block
 *     num_blocks-1 is handed out first).
 *   - A sequence owns a block table and a token count.  pa_seq_fork copies
 *     the parent's table and increments every block (the prefix is shared).
 *   - Appending a token when the last block is full (or there is none) takes a
 *     fresh block.  Appending into a partly filled last block whose refcount
 *     is > 1 first takes a fresh block, reports (src, dst) for a whole-block
 *     copy (pa_copy_blocks), decrements src and replaces the table entry.
 *   - Freeing a sequence decrements its blocks in table order.
 *   - Sequence ids are the lowest ids not in use.
 *   - Running out of blocks returns PA_ERR_OOM with the pool unchanged.
 * The pool is not thread-safe (one scheduler thread owns it).  All pointers
 * here are host memory.
 * ------------------------------------------------------------------------ */
typedef struct pa_block_pool pa_block_pool;

pa_status pa_block_pool_create(int32_t num_blocks, int32_t block_size,
                               const int32_t *initial_free_order, pa_block_pool **out);
void pa_block_pool_destroy(pa_block_pool *pool);
int32_t pa_block_pool_num_blocks(const pa_block_pool *pool);
int32_t pa_block_pool_num_free(const pa_block_pool *pool);
/* Refcount of a block, or -1 for an invalid id. */
int32_t pa_block_pool_refcount(const pa_block_pool *pool, int32_t block);
/* Copies the free stack bottom-to-top into out[capacity]; returns its size. */
int32_t pa_block_pool_free_list(const pa_block_pool *pool, int32_t *out, int32_t capacity);
pa_status pa_block_pool_alloc(pa_block_pool *pool, int32_t *block); /* refcount := 1 */
pa_status pa_block_pool_incref(pa_block_pool *pool, int32_t block);
pa_status pa_block_pool_decref(pa_block_pool *pool, int32_t block); /* frees at 0 */

pa_status pa_seq_create(pa_block_pool *pool, int32_t *seq_id);
pa_status pa_seq_fork(pa_block_pool *pool, int32_t parent, int32_t *child);
/* Append n_tokens >= 0 tokens to one sequence.  slots[n_tokens] receives the
 * flat slot table[i/16]*16 + i%16 of each new position i.  *cow_src and *cow_dst
 * receive the copy-on-write pair, or -1/-1 if none. */
pa_status pa_seq_append(pa_block_pool *pool, int32_t seq, int32_t n_tokens, int64_t *slots,
                        int32_t *cow_src, int32_t *cow_dst);
/* One token for each of n distinct sequences (a decode step), all or nothing.
 * slots[n]; cow_pairs[2*n] receives the copy pairs in sequence order and
 * *num_cow their count. */
pa_status pa_seq_append_batch(pa_block_pool *pool, const int32_t *seq_ids, int32_t n,
                              int64_t *slots, int32_t *cow_pairs, int32_t *num_cow);
pa_status pa_seq_free(pa_block_pool *pool, int32_t seq);
/* Preemption by swapping ("Inference serving: the KV-cache machine",
 * section "Paged KV" and Lab B).  pa_seq_swap_out releases the sequence's
 * private blocks -- the longest suffix of its table whose blocks it holds
 * alone (refcount 1) -- front to back, writes their ids in table order to
 * blocks_out[capacity] and their count to *n_out, and keeps the shared
 * blocks and the token count.  ceil(num_tokens / 16) is always enough
 * capacity.  Copy the blocks out (pa_swap_blocks) before they are written
 * again.  A swapped-out sequence cannot be appended to, forked or exported;
 * pa_seq_free releases its resident blocks.  pa_seq_swap_in takes that many
 * fresh blocks from the free stack, appends them to the table and writes
 * their ids to blocks_out (all or nothing: PA_ERR_OOM leaves the pool as it
 * was); copy the contents back into them.  pa_seq_swapped_blocks: the count
 * held outside for a swapped-out sequence, else -1. */
pa_status pa_seq_swap_out(pa_block_pool *pool, int32_t seq, int32_t *blocks_out, int32_t capacity,
                          int32_t *n_out);
pa_status pa_seq_swap_in(pa_block_pool *pool, int32_t seq, int32_t *blocks_out, int32_t capacity,
                         int32_t *n_out);
int32_t pa_seq_swapped_blocks(const pa_block_pool *pool, int32_t seq);
/* Token count of a sequence, or -1 for an invalid id. */
int32_t pa_seq_num_tokens(const pa_block_pool *pool, int32_t seq);
/* Tables [n][max_blocks] padded with -1, and context lengths [n]. */
pa_status pa_seq_export(const pa_block_pool *pool, const int32_t *seq_ids, int32_t n,
                        int32_t max_blocks, int32_t *tables_out, int32_t *context_lens_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
