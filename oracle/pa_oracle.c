/*
 * pa_oracle.c -- plain, slow, obviously correct CPU oracle for paged decode
 * attention, the KV append through a slot mapping, and whole-block copies.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library; the cache layout it addresses is re-implemented
 * here from the written layout contract.
 *
 * Arithmetic is IEEE double throughout.  Every cache element, whatever its
 * stored type (fp32, fp16, bf16), is widened exactly to double before use.
 *
 * What is computed, and where it is stated on the pages:
 *  - out = softmax(q . K^T / sqrt(d)) . V for one new query per (sequence,
 *    head): "KV Cache Explained Like You're an LLM Engineer", section
 *    "Transformer Attention: A Quick Refresher" (the attention formula), and
 *    "What Happens Inside an LLM During Inference", section on self-attention
 *    (the division by sqrt(d_k)).
 *  - the decode query attends over every cached position including the one
 *    just appended: "LLM Inference Optimization: KV-Cache, PagedAttention, and
 *    GPU Memory Efficiency", section "The Attention Bottleneck in Decode-Phase
 *    Inference" (the decode snippet that slices the cache up to and including
 *    the current step).
 *  - a logical position maps to (table[pos / block_size], pos % block_size):
 *    same page, section "PagedAttention: OS Concepts Meet GPU Memory" (the
 *    block-table lookup); the kernel walks the table block by block and
 *    accumulates with an online softmax.  The online rescaling reaches the
 *    same real number as the two-pass max / exp-sum form used here, so the
 *    oracle writes the plain definition out.
 *  - several query heads share one KV head (grouped-query attention): "What
 *    Happens Inside an LLM During Inference" (GQA paragraph) and "Inference
 *    serving: the KV-cache machine", section "The KV cache: attention's memory
 *    bill, derived".  Reading taken: contiguous groups, kv head = h / G.
 *  - appending a new token's K/V and copying a shared block on write:
 *    "KV Cache Explained ...", section "What KV Cache Stores" (append, then
 *    attend) and "Modern AI Infrastructure and Agentic System Design", section
 *    9.1, the shared-prefix diagram (a write to a shared block is copied into a
 *    fresh block).
 *
 * Summation order is fixed: dot products ascend in d, the exponential sum and
 * the weighted V sum ascend in logical position i.  The table walk and the
 * contiguous brute force therefore produce bit-identical doubles.
 *
 * The INT8 cache variant (quantize on append, attend over the dequantized
 * rows) is at the end of this file.
 *
 * Parity pins (tests marked "not gpu"): contiguous brute force (bitwise),
 * numpy float64 softmax attention, closed forms (length 1, uniform weights,
 * constant V, hard-max limit), block-permutation / shared-prefix / GQA-vs-MHA
 * invariants, the pages' worked block table, and hand-computed layout offsets.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element types, numbered for this file only. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

static int elem_bytes(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* IEEE binary16 -> double, from the format definition
 * (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits). */
static double f16_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16 -> double: bf16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == ORC_F32) {
    float f;
    memcpy(&f, (const char *)base + idx * 4, 4);
    return (double)f;
  }
  uint16_t bits;
  memcpy(&bits, (const char *)base + idx * 2, 2);
  return dtype == ORC_F16 ? f16_bits_to_double(bits) : bf16_bits_to_double(bits);
}

/* ---------------------------------------------------------------------------
 * Cache layout contract (element offsets).  Both caches hold num_blocks
 * physical blocks; a block holds, per KV head, one tile of 16 tokens x D dims.
 * X = 16 / element bytes is the number of elements in one 16-byte vector.
 *
 *   K tile: [D/X][16][X]    element (t, d) at (d / X)*16*X + t*X + d % X
 *   V tile: slabs of 4X dims; inside a slab, 64 vectors indexed by
 *           (t/4)*16 + (d % 4X) % 16, each vector holding (X/4) dims x 4
 *           tokens, dim-major:
 *           element (t, d) at (d/(4X))*64*X + ((t/4)*16 + (d%(4X))%16)*X
 *                              + ((d%(4X))/16)*4 + t%4
 *   tile (b, g) starts at (b*Hkv + g) * 16 * D elements.
 * ------------------------------------------------------------------------ */
#define ORC_BS 16

int64_t oracle_k_offset(int64_t block, int head, int tok, int dim, int num_kv_heads,
                        int head_dim, int dtype) {
  int X = 16 / elem_bytes(dtype);
  int64_t tile = (block * num_kv_heads + head) * (int64_t)ORC_BS * head_dim;
  return tile + (int64_t)(dim / X) * ORC_BS * X + (int64_t)tok * X + dim % X;
}

int64_t oracle_v_offset(int64_t block, int head, int tok, int dim, int num_kv_heads,
                        int head_dim, int dtype) {
  int X = 16 / elem_bytes(dtype);
  int slab_dims = 4 * X;
  int slab = dim / slab_dims;
  int e = dim % slab_dims;
  int64_t tile = (block * num_kv_heads + head) * (int64_t)ORC_BS * head_dim;
  int64_t vec = (int64_t)(tok / 4) * 16 + e % 16;
  return tile + (int64_t)slab * 64 * X + vec * X + (e / 16) * 4 + tok % 4;
}

/* ---------------------------------------------------------------------------
 * KV append through a slot mapping.  Token n's K/V row for every KV head is
 * written at slot s = slot_mapping[n]: block s / 16, in-block position s % 16.
 * Negative slots are skipped.  k_new, v_new: [T][Hkv][D] in the cache type.
 * Returns the number of out-of-range slots (nothing is written for them).
 * ------------------------------------------------------------------------ */
int oracle_reshape_and_cache(const void *k_new, const void *v_new, void *k_cache,
                             void *v_cache, const int64_t *slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int64_t num_blocks, int dtype) {
  int eb = elem_bytes(dtype);
  int bad = 0;
  for (int n = 0; n < num_tokens; ++n) {
    int64_t s = slot_mapping[n];
    if (s < 0) continue;
    if (s >= num_blocks * ORC_BS) { ++bad; continue; }
    int64_t blk = s / ORC_BS;
    int t = (int)(s % ORC_BS);
    for (int g = 0; g < num_kv_heads; ++g)
      for (int d = 0; d < head_dim; ++d) {
        int64_t src = ((int64_t)n * num_kv_heads + g) * head_dim + d;
        memcpy((char *)k_cache + oracle_k_offset(blk, g, t, d, num_kv_heads, head_dim, dtype) * eb,
               (const char *)k_new + src * eb, eb);
        memcpy((char *)v_cache + oracle_v_offset(blk, g, t, d, num_kv_heads, head_dim, dtype) * eb,
               (const char *)v_new + src * eb, eb);
      }
  }
  return bad;
}

/* Whole-block copy (all heads, K and V) for each (src, dst) pair, in order. */
void oracle_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int num_pairs,
                        int num_kv_heads, int head_dim, int dtype) {
  size_t block_bytes = (size_t)num_kv_heads * ORC_BS * head_dim * elem_bytes(dtype);
  for (int p = 0; p < num_pairs; ++p) {
    size_t src = (size_t)pairs[2 * p] * block_bytes, dst = (size_t)pairs[2 * p + 1] * block_bytes;
    memmove((char *)k_cache + dst, (const char *)k_cache + src, block_bytes);
    memmove((char *)v_cache + dst, (const char *)v_cache + src, block_bytes);
  }
}

/* ---------------------------------------------------------------------------
 * Attention of one query row over L keys/values given by accessor callbacks.
 * sigma_i = scale * sum_d q[d]*k_i[d];  M = max_i sigma_i;
 * w_i = exp(sigma_i - M);  Z = sum_i w_i;  out[d] = (sum_i w_i * v_i[d]) / Z.
 * L == 0 gives a zero row (softmax over an empty set is left undefined by the
 * pages; the reading taken is a defined, finite zero output).
 * ------------------------------------------------------------------------ */
typedef struct {
  /* paged source */
  const void *k_cache, *v_cache;
  const int32_t *table; /* this sequence's row */
  int num_kv_heads, head_dim, dtype, kv_head;
  /* contiguous source ([Lmax][Hkv][D]); used when table == NULL */
  const void *k_seq, *v_seq;
} orc_src;

static double key_at(const orc_src *s, int i, int d) {
  if (s->table) {
    int64_t blk = s->table[i / ORC_BS];
    return load_elem(s->k_cache,
                     oracle_k_offset(blk, s->kv_head, i % ORC_BS, d, s->num_kv_heads,
                                     s->head_dim, s->dtype),
                     s->dtype);
  }
  return load_elem(s->k_seq, ((int64_t)i * s->num_kv_heads + s->kv_head) * s->head_dim + d,
                   s->dtype);
}

static double value_at(const orc_src *s, int i, int d) {
  if (s->table) {
    int64_t blk = s->table[i / ORC_BS];
    return load_elem(s->v_cache,
                     oracle_v_offset(blk, s->kv_head, i % ORC_BS, d, s->num_kv_heads,
                                     s->head_dim, s->dtype),
                     s->dtype);
  }
  return load_elem(s->v_seq, ((int64_t)i * s->num_kv_heads + s->kv_head) * s->head_dim + d,
                   s->dtype);
}

/* First position a decode query attends to.  The query is the newest token,
 * position i = L-1.  Without a window (window <= 0) it sees every position;
 * with a sliding window W it sees positions i-W .. i (clipped at 0): the
 * interval "[i-W, i]" of "KV Cache Explained Like You're an LLM Engineer",
 * section "Future Optimizations" (subsection "Sliding Window Attention"),
 * read with both ends included. */
static int first_attended(int L, int window) {
  if (window <= 0 || L - 1 - window <= 0) return 0;
  return L - 1 - window;
}

static void attend_one(double *out, const double *q, const orc_src *src, int L, int window,
                       double scale, double *sigma /* scratch, >= L */) {
  int D = src->head_dim;
  if (L <= 0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    return;
  }
  int i0 = first_attended(L, window);
  double M = -INFINITY;
  for (int i = i0; i < L; ++i) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * key_at(src, i, d);
    sigma[i] = scale * dot;
    if (sigma[i] > M) M = sigma[i];
  }
  double Z = 0.0;
  for (int i = i0; i < L; ++i) {
    sigma[i] = exp(sigma[i] - M); /* sigma now holds the weights w_i */
    Z += sigma[i];
  }
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int i = i0; i < L; ++i) acc += sigma[i] * value_at(src, i, d);
    out[d] = acc / Z;
  }
}

/* ---------------------------------------------------------------------------
 * Paged decode attention by walking each sequence's block table.
 *   out:    [S][Hq][D] doubles
 *   q:      [S][Hq][D] in the cache type
 *   tables: [S][max_blocks] int32;  lens: [S] int32
 *   scale:  taken as the fp32 value the caller passes, widened to double
 *   window: sliding window W (<= 0: none); positions before L-1-W are
 *           never read, table entries included
 *   nthreads: OpenMP threads for the (s, h) loop; <= 0 means the default
 * Returns the number of threads used.
 * ------------------------------------------------------------------------ */
int oracle_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *tables, const int32_t *lens, int num_seqs, int num_q_heads,
                  int num_kv_heads, int head_dim, int max_blocks, float scale, int dtype,
                  int window, int nthreads) {
  int G = num_q_heads / num_kv_heads;
  int Lmax = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (lens[s] > Lmax) Lmax = lens[s];
  int used = 1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
#pragma omp single
    used = omp_get_num_threads();
#endif
    double *sigma = (double *)malloc(sizeof(double) * (Lmax > 0 ? Lmax : 1));
    double *qd = (double *)malloc(sizeof(double) * head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int sh = 0; sh < num_seqs * num_q_heads; ++sh) {
      int s = sh / num_q_heads, h = sh % num_q_heads;
      for (int d = 0; d < head_dim; ++d)
        qd[d] = load_elem(q, (int64_t)sh * head_dim + d, dtype);
      orc_src src = {k_cache, v_cache, tables + (int64_t)s * max_blocks, num_kv_heads,
                     head_dim, dtype, h / G, NULL, NULL};
      attend_one(out + (int64_t)sh * head_dim, qd, &src, lens[s], window, (double)scale, sigma);
    }
    free(sigma);
    free(qd);
#ifdef _OPENMP
  }
#endif
  (void)nthreads;
  return used;
}

/* ---------------------------------------------------------------------------
 * Multi-query ("extend") attention: sequence s brings n_s = query_start[s+1] -
 * query_start[s] new tokens, already in the cache, at positions L-n_s .. L-1
 * (L = lens[s]).  Query row t = query_start[s] + i sits at p = L - n_s + i and
 * attends to positions 0 .. p: causal within the new tokens, everything
 * before them ("Inference serving: the KV-cache machine": chunked prefill
 * interleaves prompt chunks with decode; speculative decoding verifies k
 * drafted tokens in one pass).  A sequence with n_s > L has NaN rows.
 *   out: [T][Hq][D] doubles, T = query_start[S];  q: [T][Hq][D] in dtype
 * Returns the number of threads used.
 * ------------------------------------------------------------------------ */
int oracle_extend(double *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *tables, const int32_t *lens, const int32_t *query_start,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_blocks,
                  float scale, int dtype, int nthreads) {
  int G = num_q_heads / num_kv_heads;
  int T = query_start[num_seqs];
  int Lmax = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (lens[s] > Lmax) Lmax = lens[s];
  int used = 1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
#pragma omp single
    used = omp_get_num_threads();
#endif
    double *sigma = (double *)malloc(sizeof(double) * (Lmax > 0 ? Lmax : 1));
    double *qd = (double *)malloc(sizeof(double) * head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t th = 0; th < (int64_t)T * num_q_heads; ++th) {
      int t = (int)(th / num_q_heads), h = (int)(th % num_q_heads);
      int s = 0;
      while (query_start[s + 1] <= t) ++s;
      int n = query_start[s + 1] - query_start[s];
      int p = lens[s] - n + (t - query_start[s]);
      double *o = out + th * head_dim;
      if (n > lens[s]) {
        for (int d = 0; d < head_dim; ++d) o[d] = NAN;
        continue;
      }
      for (int d = 0; d < head_dim; ++d) qd[d] = load_elem(q, th * head_dim + d, dtype);
      orc_src src = {k_cache, v_cache, tables + (int64_t)s * max_blocks, num_kv_heads,
                     head_dim, dtype, h / G, NULL, NULL};
      attend_one(o, qd, &src, p + 1, 0, (double)scale, sigma);
    }
    free(sigma);
    free(qd);
#ifdef _OPENMP
  }
#endif
  (void)nthreads;
  return used;
}

/* ---------------------------------------------------------------------------
 * Brute force over contiguous per-sequence arrays k_seq, v_seq:
 * [S][Lmax][Hkv][D] in the cache type.  Never touches a table.
 * ------------------------------------------------------------------------ */
void oracle_bruteforce_contiguous(double *out, const void *q, const void *k_seq,
                                  const void *v_seq, const int32_t *lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int Lmax,
                                  float scale, int dtype, int window) {
  int G = num_q_heads / num_kv_heads;
  int eb = elem_bytes(dtype);
  double *sigma = (double *)malloc(sizeof(double) * (Lmax > 0 ? Lmax : 1));
  double *qd = (double *)malloc(sizeof(double) * head_dim);
  size_t seq_elems = (size_t)Lmax * num_kv_heads * head_dim;
  for (int s = 0; s < num_seqs; ++s)
    for (int h = 0; h < num_q_heads; ++h) {
      int64_t sh = (int64_t)s * num_q_heads + h;
      for (int d = 0; d < head_dim; ++d) qd[d] = load_elem(q, sh * head_dim + d, dtype);
      orc_src src = {NULL, NULL, NULL, num_kv_heads, head_dim, dtype, h / G,
                     (const char *)k_seq + s * seq_elems * eb,
                     (const char *)v_seq + s * seq_elems * eb};
      attend_one(out + sh * head_dim, qd, &src, lens[s], window, (double)scale, sigma);
    }
  free(sigma);
  free(qd);
}

/* ===========================================================================
 * INT8 KV cache with one scale per (token, KV head) row.
 *
 * Quantization follows "KV Cache Explained Like You're an LLM Engineer",
 * section "Future Optimizations" (subsection "KV Cache Quantization"):
 * scale = max |x| over the row's last dimension / 127, code = (x / scale)
 * converted to int8, dequantized value = code * scale.
 * Readings: the arithmetic is float32 (the row's 16-bit values are widened
 * exactly; the division is IEEE single precision, correctly rounded); the
 * conversion to int8 truncates toward zero, as a float-to-integer cast does;
 * an all-zero row has scale 0 and codes 0.  "Inference serving: the KV-cache
 * machine" ("What insiders know") names per-head / per-channel scales as what
 * keeps outlier heads accurate; here every (token, head) row has its own.
 *
 * Layout contract (byte offsets into the K or V cache array).  A tile holds
 * the 16 tokens x D codes of one (block b, KV head g) followed by their 16
 * float32 row scales: 16*(D+4) bytes, starting at byte (b*Hkv + g)*16*(D+4).
 * Inside the tile:
 *   K code (t, d): c = d/64, w = d%64, h = w/32, q = (w%32)/8, e = w%8
 *      -> byte (c*64 + q*16 + t)*16 + h*8 + e
 *   V code (t, d): m = d/64, k = (d%64)/16, r = d%16
 *      -> byte (m*64 + (t/4)*16 + r)*16 + k*4 + t%4
 *   scale of token t -> bytes 16*D + 4t .. 16*D + 4t + 3 (float32, host
 *      byte order)
 * ------------------------------------------------------------------------ */
static int64_t tile_i8(int64_t block, int head, int num_kv_heads, int head_dim) {
  return (block * num_kv_heads + head) * (int64_t)ORC_BS * (head_dim + 4);
}

int64_t oracle_k_offset_i8(int64_t block, int head, int tok, int dim, int num_kv_heads,
                           int head_dim) {
  int c = dim / 64, w = dim % 64, h = w / 32, q = (w % 32) / 8, e = w % 8;
  return tile_i8(block, head, num_kv_heads, head_dim) + (int64_t)(c * 64 + q * 16 + tok) * 16 + h * 8 + e;
}

int64_t oracle_v_offset_i8(int64_t block, int head, int tok, int dim, int num_kv_heads,
                           int head_dim) {
  int m = dim / 64, k = (dim % 64) / 16, r = dim % 16;
  return tile_i8(block, head, num_kv_heads, head_dim) + (int64_t)(m * 64 + (tok / 4) * 16 + r) * 16 + k * 4 +
         tok % 4;
}

int64_t oracle_scale_offset_i8(int64_t block, int head, int tok, int num_kv_heads, int head_dim) {
  return tile_i8(block, head, num_kv_heads, head_dim) + (int64_t)ORC_BS * head_dim + 4 * tok;
}

static float load_scale(const void *cache, int64_t off) {
  float v;
  memcpy(&v, (const uint8_t *)cache + off, sizeof v);
  return v;
}

static void store_scale(void *cache, int64_t off, float v) { memcpy((uint8_t *)cache + off, &v, sizeof v); }

/* Quantizes n elements of a row (src_dtype F16/BF16/F32) into int8 codes and
 * returns the row's scale. */
float oracle_quantize_row_i8(const void *x, int64_t first, int n, int src_dtype, int8_t *codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = (float)fabs(load_elem(x, first + i, src_dtype));
    if (a > amax) amax = a;
  }
  float scale = amax / 127.0f;
  for (int i = 0; i < n; ++i) {
    if (scale == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float v = (float)load_elem(x, first + i, src_dtype) / scale;
    codes[i] = (v == v) ? (int8_t)(int)v : 0; /* C conversion truncates toward zero */
  }
  return scale;
}

/* ===========================================================================
 * FP8 (OCP E4M3) codes, same tiles and per-row scales as the int8 cache.
 * A code is s eeee mmm: exponent bias 7; e = 0 is subnormal (m * 2^-9);
 * e = 15 with m = 7 is NaN (no infinities); largest finite 448 (0x7E).
 * Quantization, read from the int8 recipe of "KV Cache Explained Like You're
 * an LLM Engineer" (Future Optimizations, KV Cache Quantization) with FP8's
 * range ("Inference serving: the KV-cache machine",
 * What insiders know, names an fp8 KV cache with per-head scales but gives no
 * recipe): scale = max |x| / 448 in float32, code = the E4M3 value
 * nearest to x / scale (float32 division), ties to the even code, values
 * beyond 448 saturate to +-448, NaN -> 0x7F; an all-zero row has scale 0.
 * ------------------------------------------------------------------------ */
double oracle_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Nearest finite E4M3 value by search in the table of the 127 non-negative
 * codes, whose values increase with the code: the last code not above |x|,
 * then the nearer of it and the next one, ties to the even code. */
int oracle_e4m3_encode(float x) {
  if (x != x) return 0x7F;
  int sign = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int lo = 0, hi = 0x7E; /* value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_value(mid) <= a) lo = mid; else hi = mid;
  }
  double dl = a - oracle_e4m3_value(lo), dh = oracle_e4m3_value(hi) - a;
  int best = dl < dh ? lo : dh < dl ? hi : ((lo & 1) == 0 ? lo : hi);
  return sign | best;
}

float oracle_quantize_row_fp8(const void *x, int64_t first, int n, int src_dtype, uint8_t *codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) {
    float a = (float)fabs(load_elem(x, first + i, src_dtype));
    if (a > amax) amax = a;
  }
  float scale = amax / 448.0f;
  for (int i = 0; i < n; ++i) {
    if (scale == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float v = (float)load_elem(x, first + i, src_dtype) / scale;
    codes[i] = (uint8_t)oracle_e4m3_encode(v);
  }
  return scale;
}

int oracle_reshape_and_cache_fp8(const void *k_new, const void *v_new, uint8_t *k_cache,
                                 uint8_t *v_cache, const int64_t *slot_mapping, int num_tokens,
                                 int num_kv_heads, int head_dim, int64_t num_blocks, int src_dtype) {
  int bad = 0;
  uint8_t *codes = (uint8_t *)malloc((size_t)head_dim);
  for (int n = 0; n < num_tokens; ++n) {
    int64_t s = slot_mapping[n];
    if (s < 0) continue;
    if (s >= num_blocks * ORC_BS) { ++bad; continue; }
    int64_t blk = s / ORC_BS;
    int t = (int)(s % ORC_BS);
    for (int g = 0; g < num_kv_heads; ++g) {
      int64_t row = ((int64_t)n * num_kv_heads + g) * head_dim;
      int64_t soff = oracle_scale_offset_i8(blk, g, t, num_kv_heads, head_dim);
      store_scale(k_cache, soff, oracle_quantize_row_fp8(k_new, row, head_dim, src_dtype, codes));
      for (int d = 0; d < head_dim; ++d)
        k_cache[oracle_k_offset_i8(blk, g, t, d, num_kv_heads, head_dim)] = codes[d];
      store_scale(v_cache, soff, oracle_quantize_row_fp8(v_new, row, head_dim, src_dtype, codes));
      for (int d = 0; d < head_dim; ++d)
        v_cache[oracle_v_offset_i8(blk, g, t, d, num_kv_heads, head_dim)] = codes[d];
    }
  }
  free(codes);
  return bad;
}

/* Append with quantization: like oracle_reshape_and_cache, into int8 tiles
 * with their per-row scales.  Returns the number of out-of-range slots. */
int oracle_reshape_and_cache_i8(const void *k_new, const void *v_new, int8_t *k_cache,
                                int8_t *v_cache, const int64_t *slot_mapping, int num_tokens,
                                int num_kv_heads, int head_dim, int64_t num_blocks, int src_dtype) {
  int bad = 0;
  int8_t *codes = (int8_t *)malloc((size_t)head_dim);
  for (int n = 0; n < num_tokens; ++n) {
    int64_t s = slot_mapping[n];
    if (s < 0) continue;
    if (s >= num_blocks * ORC_BS) { ++bad; continue; }
    int64_t blk = s / ORC_BS;
    int t = (int)(s % ORC_BS);
    for (int g = 0; g < num_kv_heads; ++g) {
      int64_t row = ((int64_t)n * num_kv_heads + g) * head_dim;
      int64_t soff = oracle_scale_offset_i8(blk, g, t, num_kv_heads, head_dim);
      store_scale(k_cache, soff, oracle_quantize_row_i8(k_new, row, head_dim, src_dtype, codes));
      for (int d = 0; d < head_dim; ++d)
        k_cache[oracle_k_offset_i8(blk, g, t, d, num_kv_heads, head_dim)] = codes[d];
      store_scale(v_cache, soff, oracle_quantize_row_i8(v_new, row, head_dim, src_dtype, codes));
      for (int d = 0; d < head_dim; ++d)
        v_cache[oracle_v_offset_i8(blk, g, t, d, num_kv_heads, head_dim)] = codes[d];
    }
  }
  free(codes);
  return bad;
}

/* Whole-block copy of an int8 / E4M3 cache: the tiles (codes and scales) of
 * every head. */
void oracle_copy_blocks_i8(int8_t *k_cache, int8_t *v_cache, const int32_t *pairs, int num_pairs,
                           int num_kv_heads, int head_dim) {
  size_t block_bytes = (size_t)num_kv_heads * ORC_BS * (head_dim + 4);
  for (int p = 0; p < num_pairs; ++p) {
    size_t src = (size_t)pairs[2 * p], dst = (size_t)pairs[2 * p + 1];
    memmove(k_cache + dst * block_bytes, k_cache + src * block_bytes, block_bytes);
    memmove(v_cache + dst * block_bytes, v_cache + src * block_bytes, block_bytes);
  }
}

/* Decode over an int8 cache: the keys and values attended are the
 * dequantized rows code * scale (exact in double); q is F16 or BF16. */
typedef struct {
  const int8_t *k_cache, *v_cache;
  const int32_t *table;
  int num_kv_heads, head_dim, kv_head;
  int fp8; /* codes are E4M3 (else int8) */
} orc_src_i8;

static double code_value(const orc_src_i8 *s, int8_t c) {
  return s->fp8 ? oracle_e4m3_value((uint8_t)c) : (double)c;
}

static void attend_one_i8(double *out, const double *q, const orc_src_i8 *s, int L, int window,
                          double scale, double *sigma) {
  int D = s->head_dim;
  if (L <= 0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    return;
  }
  int i0 = first_attended(L, window);
  double M = -INFINITY;
  for (int i = i0; i < L; ++i) {
    int64_t blk = s->table[i / ORC_BS];
    int t = i % ORC_BS;
    double ks = (double)load_scale(s->k_cache, oracle_scale_offset_i8(blk, s->kv_head, t, s->num_kv_heads, D));
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += q[d] * (code_value(s, s->k_cache[oracle_k_offset_i8(blk, s->kv_head, t, d, s->num_kv_heads, D)]) * ks);
    sigma[i] = scale * dot;
    if (sigma[i] > M) M = sigma[i];
  }
  double Z = 0.0;
  for (int i = i0; i < L; ++i) {
    sigma[i] = exp(sigma[i] - M);
    Z += sigma[i];
  }
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int i = i0; i < L; ++i) {
      int64_t blk = s->table[i / ORC_BS];
      int t = i % ORC_BS;
      double vs = (double)load_scale(s->v_cache, oracle_scale_offset_i8(blk, s->kv_head, t, s->num_kv_heads, D));
      acc += sigma[i] * (code_value(s, s->v_cache[oracle_v_offset_i8(blk, s->kv_head, t, d, s->num_kv_heads, D)]) * vs);
    }
    out[d] = acc / Z;
  }
}

/* Decode over an int8 (fp8 = 0) or E4M3 (fp8 = 1) cache. */
int oracle_decode_codes(double *out, const void *q, int q_dtype, const int8_t *k_cache,
                        const int8_t *v_cache, const int32_t *tables, const int32_t *lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int max_blocks, float scale, int window,
                        int fp8, int nthreads) {
  int G = num_q_heads / num_kv_heads;
  int Lmax = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (lens[s] > Lmax) Lmax = lens[s];
  int used = 1;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
  {
#pragma omp single
    used = omp_get_num_threads();
#endif
    double *sigma = (double *)malloc(sizeof(double) * (Lmax > 0 ? Lmax : 1));
    double *qd = (double *)malloc(sizeof(double) * head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int sh = 0; sh < num_seqs * num_q_heads; ++sh) {
      int s = sh / num_q_heads, h = sh % num_q_heads;
      for (int d = 0; d < head_dim; ++d) qd[d] = load_elem(q, (int64_t)sh * head_dim + d, q_dtype);
      orc_src_i8 src = {k_cache, v_cache, tables + (int64_t)s * max_blocks,
                        num_kv_heads, head_dim, h / G, fp8};
      attend_one_i8(out + (int64_t)sh * head_dim, qd, &src, lens[s], window, (double)scale, sigma);
    }
    free(sigma);
    free(qd);
#ifdef _OPENMP
  }
#endif
  (void)nthreads;
  return used;
}
