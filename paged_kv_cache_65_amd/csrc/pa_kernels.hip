// Paged decode attention, KV append and block copy kernels for gfx950
// (CDNA4, wavefront 64), with their C-ABI entry points.
//
// Decode ("LLM Inference Optimization: KV-Cache, PagedAttention, and GPU
// Memory Efficiency", section "PagedAttention: OS Concepts Meet GPU Memory":
// walk the sequence's block table, load K and V of each physical block, score
// it and fold it in with an online softmax).  Every wave keeps an
// online-softmax state (running max m, running sum l, weighted V sum) for all
// query heads of a KV head's group, so every K/V tile is read from HBM once
// and reused by the whole group.  Two ways to split the work:
//   * partitions: one workgroup of four waves takes one (context partition,
//     KV head, sequence); the waves split the partition's 16-token blocks
//     round-robin and their states meet in LDS at the end;
//   * balanced: a persistent grid whose waves each stream an equal share of
//     all (sequence, KV head, block) units (see pa_balanced_kernel).
// A piece of work either writes its final rows or an (m, l, acc) partial that
// the merge kernel folds with log-sum-exp rescaling.
//
// Two per-wave math policies share that skeleton:
//   * MfmaWave (fp16/bf16): q.K^T for the whole group is one 16x16x32 matrix
//     core tile per 32 dims (tokens x heads, heads padded to 16), and P.V is
//     16x16x16 tiles (dims x heads, contracting the block's 16 tokens).  The
//     cache layout makes each lane's 16-byte load exactly its operand
//     fragment, and the q.K^T output fragment is exactly the P.V operand
//     fragment, so scores never leave registers.  P is split into a high and
//     a low 16-bit part (two P.V tiles) so the softmax weights keep ~16
//     mantissa bits.
//   * ValuWave (any type): the same data flow with float32 FMAs, q staged in
//     LDS, cross-lane reductions by shuffles.
// Scores are kept in the log2 domain (scale * log2(e) folded into one
// multiply) so the exponentials are single v_exp_f32 instructions.
//
// Also here: MfmaWaveI8, the same matrix-core policy over INT8 / FP8 code
// tiles with per-row scales; multi-query ("extend") attention; the kernel that
// computes attention over a shared prefix once for every sequence; the
// quantizing append; and block copies between a device cache and pinned host
// memory (swap).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pa.h"
#include "pa_error.h"

namespace {

constexpr int kBS = 16;        // tokens per block
constexpr int kWaves = 4;      // waves per partition workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kTileCols = 16;  // query heads per MFMA column tile
constexpr int kGMax = 64;      // query heads per KV head (up to four column tiles)
constexpr int kDMax = 128;
constexpr float kLazyLog2 = 8.0f;  // MFMA path: softmax weights stay below 2^8

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element types
template <int DT> struct Ty;
template <> struct Ty<PA_F32> {
  static constexpr int bytes = 4;
  __device__ static float to_f32(uint32_t bits) { return __uint_as_float(bits); }
};
template <> struct Ty<PA_F16> {
  static constexpr int bytes = 2;
  __device__ static float to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
};
template <> struct Ty<PA_BF16> {
  static constexpr int bytes = 2;
  __device__ static float to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }
};

__device__ inline uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}
__device__ inline uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

__device__ inline void store_out(void *out, int64_t idx, float v, int out_dtype) {
  if (out_dtype == PA_F32)
    static_cast<float *>(out)[idx] = v;
  else if (out_dtype == PA_F16)
    static_cast<uint16_t *>(out)[idx] = f32_to_f16_bits(v);
  else
    static_cast<uint16_t *>(out)[idx] = f32_to_bf16_bits(v);
}

// Four consecutive elements (idx a multiple of 4).
__device__ inline void store_out4(void *out, int64_t idx, f32x4_t v, int out_dtype) {
  if (out_dtype == PA_F32) {
    *reinterpret_cast<f32x4_t *>(static_cast<float *>(out) + idx) = v;
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = out_dtype == PA_F16 ? f32_to_f16_bits(v[e]) : f32_to_bf16_bits(v[e]);
    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(out) + idx) = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  }
}

// Four consecutive floats of a partial row: the partial accumulators follow
// the (m, l) pairs in the workspace, so they are 8-byte aligned.
__device__ inline void store_partial4(float *dst, f32x4_t v) {
  reinterpret_cast<f32x2_t *>(dst)[0] = f32x2_t{v[0], v[1]};
  reinterpret_cast<f32x2_t *>(dst)[1] = f32x2_t{v[2], v[3]};
}

__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Workgroup barrier that orders LDS only: a wave's global stores in flight
// need not be acknowledged first (each output element has one writer).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-wave timeline of the balanced and extend kernels, in a traced build
// only (compiled with -DPA_TRACE; the library's own build has none of it):
// each wave stamps the real-time counter (100 MHz) at entry, when its
// inputs are ready (lengths scanned / contexts ranked), at its first block,
// when its stream ends and at its exit, and records its XCD and the blocks it
// streamed; pa_trace_read copies the records of the last launch back.
#ifdef PA_TRACE
constexpr int kTraceWaves = 65536;
__device__ uint64_t pa_trace_buf[kTraceWaves * 8];
struct WaveTrace {
  uint64_t t[4] = {0, 0, 0, 0};
  __device__ void stamp(int k) { t[k] = __builtin_amdgcn_s_memrealtime(); }
  __device__ void first() {
    if (t[2] == 0) stamp(2);
  }
  __device__ void write(int64_t wave, int lane, uint64_t units) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (lane == 0 && wave >= 0 && wave < kTraceWaves) {
      uint64_t *p = pa_trace_buf + wave * 8;
      for (int k = 0; k < 4; ++k) p[k] = t[k];
      p[4] = t_end;
      p[5] = xcc;
      p[6] = units;
      p[7] = 1;
    }
  }
};
#else
struct WaveTrace {
  __device__ void stamp(int) {}
  __device__ void first() {}
  __device__ void write(int64_t, int, uint64_t) {}
};
#endif

// Cross-lane combines that stay in the vector ALU (no LDS round trip).
// permlane16_swap / permlane32_swap of a value with itself leave, in the two
// results, the lane's own value and the value of the lane 16 (resp. 32)
// apart; DPP quad permutes and row mirrors pair lanes inside a 16-lane row.
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Reductions over the 16 lanes of a row: quad_perm [1,0,3,2], [2,3,0,1],
// then row_half_mirror and row_mirror.
__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}
__device__ inline float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}
// 2^x for x <= 0 (one v_exp_f32; results below 2^-126 flush to zero).
__device__ inline float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- arguments
struct DecodeArgs {
  void *out;
  const void *q;
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *ws_ml;   // [S][Hq][max_parts][2]  (m in log2 units, l)
  float *ws_acc;  // [S][Hq][max_parts][D]  unnormalised weighted V sums
  const uint8_t *k_new;          // fused append: [S][Hkv][D] rows of the step's token, or null
  const uint8_t *v_new;
  const int64_t *slot_mapping;   // fused append: [S] slot of position L-1 (negative = no append)
  int32_t *ws_pre;               // balanced split: [S+1] blocks of the sequences before s
  int32_t num_seqs, num_q_heads, num_kv_heads, group, max_blocks, num_blocks, max_ctx, max_parts,
      part_tokens, out_dtype, num_workers, window;
  float scale_log2;
  int32_t prefix_blocks;   // shared prefix: the first table entries, the same blocks for every sequence
  int32_t park_slots;      // balanced split: LDS parking slots per wave (1 .. kParkSlotsMax)
  float *ws_pfx_ml;        // shared prefix: [S][Hq][2] (m, l) of every row over the prefix
  float *ws_pfx_acc;       //                [S][Hq][D]
};

__device__ inline bool ctx_valid(int L, const DecodeArgs &a) {
  return L >= 0 && L <= a.max_ctx && (int64_t)L <= (int64_t)a.max_blocks * kBS;
}

// Sliding window ("KV Cache Explained Like You're an LLM Engineer", section
// "Future Optimizations", subsection "Sliding Window Attention"): the query
// at position L-1 sees positions L-1-W .. L-1 (clipped at 0); W <= 0: no
// window.  Blocks before the one holding the first such position are never
// touched.
__device__ inline int window_first_token(int L, int W) { return (W > 0 && L - 1 - W > 0) ? L - 1 - W : 0; }

constexpr uint32_t kAllTokens = 0xFFFFu;

// Tokens lo .. hi-1 of a block (0 <= lo < hi <= 16) as a bit mask.
__device__ inline uint32_t token_mask(int lo, int hi) { return ((1u << hi) - 1u) & ~((1u << lo) - 1u); }

// Floats of padding after each row of a fold buffer: a wave writes its
// accumulators as 16-byte pieces of 16 rows at once, and rows a multiple of
// 128 bytes apart would put all 16 in the same LDS banks.
constexpr int kAccPad = 4;

// Per-wave online-softmax states meet here at the end of a partition, one
// column tile (16 heads) at a time.
struct __align__(16) SmemBase {
  float acc[kWaves][kTileCols][kDMax + kAccPad];
  float m[kWaves][kTileCols];
  float l[kWaves][kTileCols];
  float fac[kWaves][kTileCols];  // each wave's weight in the fold of a head
  float mx[kTileCols];
  float den[kTileCols];
  uint32_t knew[kDMax];  // fused append: the new token's K and V rows (raw bits, up to 512 B)
  uint32_t vnew[kDMax];
};
struct __align__(16) SmemValu : SmemBase {
  float qs[kTileCols][kDMax];        // q of the workgroup's heads in float32
  float ps[kWaves][kTileCols][kBS];  // softmax weights of the current block
};

// ---------------------------------------------------------------- fused append
// Fragment layouts shared by both wave policies (X = 16 / element bytes):
//   K fragment c of lane l: token l % 16, dims X*(4c + l/16) .. +X-1;
//   V fragment c of lane l: element sub*4 + i = (token 4*(l/16) + i,
//     dim c*4X + sub*16 + l % 16), sub < X/4.
// Replaces token t's elements in a tile's fragments with the staged new row,
// so the step's own token is attended from registers even while its store to
// the cache is still in flight.
template <int EB, int NCF>
__device__ inline void patch_new_token(u32x4_t (&fk)[NCF], u32x4_t (&fv)[NCF], int t, int lane,
                                       const uint32_t *knew, const uint32_t *vnew) {
  constexpr int X = 16 / EB;
  const int r = lane % 16, tq = lane / 16;
  // Every register index below is a compile-time constant (runtime indices
  // into the fragments would send the whole ring to scratch memory).
#pragma unroll
  for (int c = 0; c < NCF; ++c) {
    const u32x4_t kx = *reinterpret_cast<const u32x4_t *>(knew + (X * (4 * c + tq)) * EB / 4);
    fk[c] = (r == t) ? kx : fk[c];
  }
  const bool in_quad = tq == t / 4;
  const int i = t % 4;
#pragma unroll
  for (int c = 0; c < NCF; ++c) {
#pragma unroll
    for (int e = 0; e < X; ++e) {  // element e = (token 4*tq + e%4, dim c*4X + (e/4)*16 + r)
      const bool hit = in_quad && (e % 4 == i);
      const int d = c * 4 * X + (e / 4) * 16 + r;
      if constexpr (EB == 4) {
        fv[c][e] = hit ? vnew[d] : fv[c][e];
      } else {
        const uint32_t val = (vnew[d / 2] >> ((d & 1) * 16)) & 0xFFFFu;
        const uint32_t old = fv[c][e / 2];
        const uint32_t upd = (e & 1) ? ((old & 0x0000FFFFu) | (val << 16)) : ((old & 0xFFFF0000u) | val);
        fv[c][e / 2] = hit ? upd : old;
      }
    }
  }
}

// Writes one token's K and V rows of one KV head into its slot (tile layouts
// as in pa_reshape_and_cache), by the 64 lanes of one wave.
template <int EB, int D>
__device__ inline void write_token_row(uint8_t *k_cache, uint8_t *v_cache, int64_t blk, int t, int g,
                                       int num_kv_heads, const uint32_t *knew, const uint32_t *vnew,
                                       int lane) {
  constexpr int X = 16 / EB;
  const int64_t tile = (blk * num_kv_heads + g) * kBS * D;
  if (lane < D / X) {
    const u32x4_t kx = *reinterpret_cast<const u32x4_t *>(knew + lane * 4);
    reinterpret_cast<u32x4_t *>(k_cache + (tile + (int64_t)lane * kBS * X + t * X) * EB)[0] = kx;
  }
  for (int d = lane; d < D; d += 64) {
    const int slab = d / (4 * X), de = d % (4 * X);
    const int64_t off = tile + (int64_t)slab * 64 * X + ((t / 4) * 16 + de % 16) * X + (de / 16) * 4 + t % 4;
    if constexpr (EB == 4)
      reinterpret_cast<uint32_t *>(v_cache)[off] = vnew[d];
    else
      reinterpret_cast<uint16_t *>(v_cache)[off] = (uint16_t)((vnew[d / 2] >> ((d & 1) * 16)) & 0xFFFFu);
  }
}

// One 4-wave workgroup per CU (one wave per SIMD), each wave with a ring of
// four blocks (32 KiB) in flight: fewer, longer wave shares mean fewer
// segments, hence fewer partial stores and a cheaper merge, and 128 KiB in
// flight per CU still saturates HBM.
#ifndef PA_BALANCED_WG_PER_CU
#define PA_BALANCED_WG_PER_CU 1
#endif
#ifndef PA_BALANCED_RING
#define PA_BALANCED_RING 4
#endif
#ifndef PA_BALANCED_WAVES
#define PA_BALANCED_WAVES 4
#endif
#ifndef PA_I8_RING
#define PA_I8_RING 2
#endif
#ifndef PA_I8_WG_PER_CU
#define PA_I8_WG_PER_CU 2
#endif
#ifndef PA_FP8_RING
#define PA_FP8_RING PA_I8_RING
#endif
#ifndef PA_FP8_WG_PER_CU
#define PA_FP8_WG_PER_CU PA_I8_WG_PER_CU
#endif

// ============================================================================
// MFMA wave: fp16 / bf16 caches.
//
// Lane l, with r = l % 16 and tq = l / 16:
//   K fragment c (c < D/32): the 16 bytes at tile + 1024c + 16l = token r,
//     dims 32c + 8tq .. +7  -> A operand of mfma_f32_16x16x32 (row = token).
//   q fragment [ct][c]: head 16ct + r of the group (zero past G), same dims
//     -> B operand of column tile ct.
//   score tile ct: sc[v] = s(token 4tq+v, head 16ct + r).
//   V fragment m (m < D/32): 16 bytes at tile + 1024m + 16l = tokens
//     4tq..4tq+3 of dim 32m+r (first 8 bytes) and of dim 32m+16+r (last 8)
//     -> A operands of mfma_f32_16x16x16 for output tiles n = 2m, 2m+1
//     (row = dim, contraction = token).
//   P operand = the lane's own 4 weights (tokens 4tq..4tq+3, head 16ct + r).
//   acc[ct][n][v] = O(head 16ct + r, dim 16n + 4tq + v).
// NCT = ceil(G / 16) column tiles: a group of more than 16 query heads (up
// to all 64 heads on one shared KV head, multi-query attention) takes
// several 16-head tiles, each with its own softmax state, and every K and V
// fragment in registers feeds all of them, so a block is still read once.
// ============================================================================
template <int DT, int D, int NCT_ = 1>
struct MfmaWave {
  static constexpr int NCT = NCT_;   // 16-head column tiles
  static constexpr int NC = D / 32;  // 16-byte fragments per tile
  static constexpr int NT = D / 16;  // output tiles
  static constexpr int TILE = kBS * D * 2;
#ifndef PA_MFMA_RING
#define PA_MFMA_RING 2
#endif
  // Blocks held in registers per wave in the partition kernel: two (one in
  // the matrix ops, the next loading) at twelve waves per CU measured 1-3%
  // faster than three, at 137 instead of 165 VGPRs (D = 128).
  static constexpr int kRing = PA_MFMA_RING;
  // Partition workgroups per CU: each more column tile holds another set of
  // q fragments and accumulators in registers.
  static constexpr int kPartWgPerCu = NCT == 1 ? 3 : NCT == 2 ? 2 : 1;
  using v8 = typename std::conditional<DT == PA_BF16, bf16x8_t, f16x8_t>::type;

  struct Frag {
    u32x4_t k[NC];
    u32x4_t v[NC];
  };

  using Smem = SmemBase;

  v8 qB[NCT][NC];
  f32x4_t acc[NCT][NT];
  float m[NCT], l[NCT];

  __device__ void reset() {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[ct][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[ct] = -INFINITY;
      l[ct] = 0.f;
    }
  }

  // q fragments from the group's G rows of D 16-bit values (rows >= G are 0).
  // The pointer may be global or LDS memory; the load instructions follow it.
  template <class P>
  __device__ void load_q(const P *rows, int G, int lane) {
    const int r = lane % 16, tq = lane / 16;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int h = 16 * ct + r;
      const u32x4_t *qrow = reinterpret_cast<const u32x4_t *>(rows) + (h < G ? h : 0) * (D / 8);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4_t x = qrow[4 * c + tq];
        if (h >= G) x = u32x4_t{0, 0, 0, 0};
        qB[ct][c] = __builtin_bit_cast(v8, x);
      }
    }
  }

  // q rows of KV head g of sequence s.
  __device__ void init(const DecodeArgs &a, int s, int g, int lane) {
    const int G = a.group;
    load_q(static_cast<const uint8_t *>(a.q) + ((int64_t)s * a.num_q_heads + g * G) * D * 2, G, lane);
    reset();
  }

  __device__ static void load(Frag &f, const uint8_t *ktile, const uint8_t *vtile, int lane) {
    const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(ktile);
    const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vtile);
#pragma unroll
    for (int c = 0; c < NC; ++c) f.k[c] = __builtin_nontemporal_load(&kp[c * 64 + lane]);
#pragma unroll
    for (int c = 0; c < NC; ++c) f.v[c] = __builtin_nontemporal_load(&vp[c * 64 + lane]);
  }

  static constexpr bool kAppend = true;  // supports the fused append
  // Balanced kernel: blocks in flight per wave (each more column tile takes
  // registers from the ring) and workgroups per CU.
  static constexpr int kBalRing = NCT == 1 ? PA_BALANCED_RING : NCT == 2 ? 3 : 2;
  static constexpr int kBalWgPerCu = PA_BALANCED_WG_PER_CU;
  // Tile index = block * Hkv + head.
  __device__ static void load_tile(Frag &f, const DecodeArgs &a, int64_t tile, int lane) {
    load(f, a.k_cache + tile * TILE, a.v_cache + tile * TILE, lane);
  }

  // Fused append, balanced kernel: a new token's K and V rows (two 16-bit
  // elements per lane, lanes < D/2) staged as they are, and later written to
  // their slot.  Called by the whole wave.
  __device__ static void stage_new(uint32_t *kdst, uint32_t *vdst, uint32_t kr, uint32_t vr, int lane) {
    if (lane < D / 2) {
      kdst[lane] = kr;
      vdst[lane] = vr;
    }
  }
  __device__ static void write_new(const DecodeArgs &a, int64_t blk, int t, int g, const uint32_t *knew,
                                   const uint32_t *vnew, int lane) {
    write_token_row<2, D>(const_cast<uint8_t *>(a.k_cache), const_cast<uint8_t *>(a.v_cache), blk, t, g,
                          a.num_kv_heads, knew, vnew, lane);
  }

  __device__ static f32x4_t mma_qk(const v8 &a, const v8 &b, f32x4_t c) {
    if constexpr (DT == PA_BF16)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }

  __device__ static f32x4_t mma_pv(u32x2_t a, u32x2_t b, f32x4_t c) {
    if constexpr (DT == PA_BF16)
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                       __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                   __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }

  // Two floats rounded to nearest even and packed into one word (the first
  // in the low half): one v_cvt_pk_{bf16,f16}_f32.
  __device__ static uint32_t pack2(float a, float b) {
    if constexpr (DT == PA_BF16)
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
    else
      return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
  }
  // The two 16-bit values of a packed word, widened back to float.
  __device__ static f32x2_t unpack2(uint32_t w) {
    if constexpr (DT == PA_BF16)
      return f32x2_t{__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
    else
      return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
  }
  // Splits p into hi + lo 16-bit values (hi = round(p), lo = round(p - hi)),
  // two values per conversion.
  __device__ static void split(const float p[4], u32x2_t &hi, u32x2_t &lo) {
    const uint32_t h01 = pack2(p[0], p[1]), h23 = pack2(p[2], p[3]);
    const f32x2_t b01 = unpack2(h01), b23 = unpack2(h23);
    hi = u32x2_t{h01, h23};
    lo = u32x2_t{pack2(p[0] - b01.x, p[1] - b01.y), pack2(p[2] - b23.x, p[3] - b23.y)};
  }

  // Online-softmax step of column tile ct for the block's scores s[] (log2
  // units, masked tokens -inf): lazy reference max, weights, running sum.
  // The state is rescaled only when a head's block max exceeds its
  // reference by more than kLazyLog2, so weights stay below 2^kLazyLog2 and
  // most blocks skip the rescale (a wave-uniform branch).
  __device__ void softmax_step(int ct, const float s[4], float p[4]) {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max_xor32(max_xor16(mx));
    const bool bump = mx > m[ct] + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(bump)) {
      const float m_new = bump ? mx : m[ct];
      const float alpha = exp2_neg(m[ct] - m_new);
      l[ct] *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[ct][n] *= alpha;
      m[ct] = m_new;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(s[v] - m[ct]);
    l[ct] += (p[0] + p[1]) + (p[2] + p[3]);
  }

  // One block; bit t of `vm` set = token t of the block is attended (inside
  // the context and the window); new_tok >= 0: that token's K/V come from
  // the staged new row.
  __device__ void compute(Frag &f, uint32_t vm, float scale_log2, int lane, int new_tok,
                          const uint32_t *knew, const uint32_t *vnew) {
    const int tq = lane / 16;
    if (new_tok >= 0) patch_new_token<2, NC>(f.k, f.v, new_tok, lane, knew, vnew);
    const uint32_t mine = vm >> (4 * tq);  // this lane's 4 tokens in the low bits
    if (vm != kAllTokens) {
      // Slots outside the attended range may hold anything (NaN included):
      // zero the V elements so 0 * V stays 0; scores are masked below.
      const uint32_t lo = ((mine & 1u) ? 0x0000FFFFu : 0u) | ((mine & 2u) ? 0xFFFF0000u : 0u);
      const uint32_t hi = ((mine & 4u) ? 0x0000FFFFu : 0u) | ((mine & 8u) ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] &= u32x4_t{lo, hi, lo, hi};
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc = mma_qk(__builtin_bit_cast(v8, f.k[c]), qB[ct][c], sc);
      float s[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) s[v] = sc[v] * scale_log2;
      if (vm != kAllTokens) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] = ((mine >> v) & 1u) ? s[v] : -INFINITY;
      }
      float p[4];
      softmax_step(ct, s, p);
      u32x2_t ph, pl;
      split(p, ph, pl);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x2_t a0 = u32x2_t{f.v[c][0], f.v[c][1]};
        const u32x2_t a1 = u32x2_t{f.v[c][2], f.v[c][3]};
        acc[ct][2 * c] = mma_pv(a0, ph, acc[ct][2 * c]);
        acc[ct][2 * c + 1] = mma_pv(a1, ph, acc[ct][2 * c + 1]);
        acc[ct][2 * c] = mma_pv(a0, pl, acc[ct][2 * c]);
        acc[ct][2 * c + 1] = mma_pv(a1, pl, acc[ct][2 * c + 1]);
      }
    }
  }

  // Publishes this wave's state for column tile ct (heads 16ct .. 16ct+15 of
  // the group, those below G) into LDS rows 0 .. 15.
  __device__ void finish(Smem &sm, int w, int lane, int G, int ct) {
    const int r = lane % 16, tq = lane / 16;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      if (c != ct) continue;  // register indices stay compile-time constants
      const float lt = sum_xor32(sum_xor16(l[c]));
      if (16 * c + r < G) {
#pragma unroll
        for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4_t *>(&sm.acc[w][r][16 * n + 4 * tq]) = acc[c][n];
        if (tq == 0) {
          sm.m[w][r] = m[c];
          sm.l[w][r] = lt;
        }
      }
    }
  }

  // Balanced split: writes this wave's state for one (sequence, KV head)
  // pair whose query rows start at row0: the normalised output rows when the
  // wave saw the whole pair (never with a shared prefix: the merge folds the
  // prefix in), else an (m, l, acc) partial at partial row prow0.  `bad`
  // turns them into NaN.
  __device__ void store_segment(const DecodeArgs &a, int64_t row0, int64_t prow0, bool whole, bool bad,
                                int lane, int G) const {
    const int r = lane % 16, tq = lane / 16;
    const f32x4_t nan4 = {NAN, NAN, NAN, NAN};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float lt = sum_xor32(sum_xor16(l[ct]));
      const int h = 16 * ct + r;
      if (h >= G) continue;
      if (whole) {
        const int64_t o = (row0 + h) * D + 4 * tq;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4_t v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[ct][n][e] / lt;
          store_out4(a.out, o + 16 * n, bad ? nan4 : v, a.out_dtype);
        }
      } else {
        float *pacc = a.ws_acc + (prow0 + h) * D + 4 * tq;
#pragma unroll
        for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4_t *>(pacc + 16 * n) = bad ? nan4 : acc[ct][n];
        if (tq == 0) {
          a.ws_ml[(prow0 + h) * 2] = bad ? NAN : m[ct];
          a.ws_ml[(prow0 + h) * 2 + 1] = lt;
        }
      }
    }
  }

  // Balanced split: parks the state in LDS instead (acc rows [G][D] with
  // kAccPad floats after each, then m[G], l[G]); flush_parked() writes it
  // out later.
  __device__ void park_segment(float *st, int lane, int G) const {
    constexpr int RS = D + kAccPad;
    const int r = lane % 16, tq = lane / 16;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float lt = sum_xor32(sum_xor16(l[ct]));
      const int h = 16 * ct + r;
      if (h >= G) continue;
#pragma unroll
      for (int n = 0; n < NT; ++n) *reinterpret_cast<f32x4_t *>(st + h * RS + 16 * n + 4 * tq) = acc[ct][n];
      if (tq == 0) {
        st[G * RS + h] = m[ct];
        st[G * RS + G + h] = lt;
      }
    }
  }
};

// Writes a state parked by park_segment exactly as store_segment would have.
template <int D>
__device__ void flush_parked(const DecodeArgs &a, const float *st, int64_t row0, int64_t prow0, bool whole,
                             bool bad, int lane, int G) {
  const f32x4_t nan4 = {NAN, NAN, NAN, NAN};
  constexpr int RS = D + kAccPad;
  for (int e = lane * 4; e < G * D; e += 256) {
    const int r = e / D;
    f32x4_t v = *reinterpret_cast<const f32x4_t *>(st + r * RS + e % D);
    if (whole) {
      const float lt = st[G * RS + G + r];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = v[k] / lt;
      store_out4(a.out, (row0 + r) * D + e % D, bad ? nan4 : v, a.out_dtype);
    } else {
      *reinterpret_cast<f32x4_t *>(a.ws_acc + prow0 * D + e) = bad ? nan4 : v;
    }
  }
  if (!whole && lane < G) {
    a.ws_ml[(prow0 + lane) * 2] = bad ? NAN : st[G * RS + lane];
    a.ws_ml[(prow0 + lane) * 2 + 1] = st[G * RS + G + lane];
  }
}

// ---------------------------------------------------------------- INT8 / FP8 codes
// One wave per (token, KV head) row: max |x| over the row by a wave
// reduction, scale = max / 127 (int8) or max / 448 (E4M3), codes from
// x / scale (float32, correctly rounded division): truncated toward zero
// (int8) or rounded to the nearest E4M3 value, ties to even, saturating at
// +-448 (e4m3_code); codes scattered into the byte tile layout, the scale
// stored beside it.

// Nearest E4M3 code of x: below 2^-6 the step is 2^-9 (subnormals, and 2^-6
// itself as code 8); above, 3 mantissa bits under the exponent of x.
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);
  int e;
  (void)frexpf(a, &e);                       // a in [2^(e-1), 2^e)
  const int E = e - 1;                       // -6 .. 8
  int q = (int)rintf((ldexpf(a, -E) - 1.f) * 8.f);  // 0 .. 8, ties to even
  int ef = E + 7;
  if (q == 8) {
    q = 0;
    ++ef;
  }
  return sign | min((uint32_t)((ef << 3) | q), 0x7Eu);
}

// A 16-bit row element (SDT = PA_BF16 or PA_F16 bits) as float32.
template <int SDT>
__device__ inline float half_value(uint32_t bits) {
  return SDT == PA_BF16 ? __uint_as_float(bits << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

template <int FMT>
__device__ inline float code_scale(float amax) {
  return amax / (FMT == PA_FP8 ? 448.0f : 127.0f);
}

template <int FMT>
__device__ inline int code_of(float v, float scale) {
  const float qv = scale == 0.f ? 0.f : v / scale;
  if constexpr (FMT == PA_FP8)
    return scale == 0.f ? 0 : (int)e4m3_code(qv);
  else
    return qv == qv ? (int)qv : 0;  // conversion truncates toward zero
}

// Byte offsets of (token t, dim d) in a code tile: K as 16-byte vectors
// (dim block c = d / 64, lane ((d % 32) / 8) * 16 + t; dims 8q .. 8q+7 of the
// block, then 32 + 8q .. 32 + 8q + 7), V as 4 tokens x 4 dim quarters per
// vector (lane (t / 4) * 16 + d % 16, byte ((d % 64) / 16) * 4 + t % 4).
__device__ inline int k_code_off(int d, int t) {
  const int c = d / 64, w = d % 64;
  return (c * 64 + ((w % 32) / 8) * 16 + t) * 16 + (w / 32) * 8 + w % 8;
}
__device__ inline int v_code_off(int d, int t) {
  return ((d / 64) * 64 + (t / 4) * 16 + d % 16) * 16 + ((d % 64) / 16) * 4 + t % 4;
}

// ============================================================================
// MFMA wave over an INT8 cache (q in QDT = fp16 / bf16).
//
// Codes are small integers, exact in fp16 and bf16, so the matrix cores take
// them unscaled: the K scale multiplies the token's score after q.K^T, and
// the V scale joins the token's softmax weight before P.V (the running sum l
// keeps the unscaled weights).  With c = lane / 16 and r = lane % 16:
//   K code vector x (x < D/64) of lane l: token r; bytes 0-7 dims
//     64x + 8c .. +7 (q.K^T chunk 2x), bytes 8-15 dims 64x + 32 + 8c .. +7
//     (chunk 2x + 1);
//   V code vector x: tokens 4c .. 4c+3 of dims 64x + 16k + r, bytes 4k .. 4k+3
//     -> A operand of the P.V tile n = 4x + k;
//   scales: the four tokens 4c .. 4c+3 of the lane's score rows.
// Several column tiles (G > 16) share the block's codes: they are converted
// once per block and feed every tile.
// ============================================================================
// Byte-code caches: FMT = PA_I8 (int8 codes) or PA_FP8 (OCP E4M3 codes),
// one float32 scale per (token, KV head) row.
template <int QDT, int D, int FMT = PA_I8, int NCT_ = 1>
struct MfmaWaveI8 : MfmaWave<PA_F16, D, NCT_> {
  // fp16 matrix ops: a code becomes an fp16 value exactly (pair16: three
  // instructions per pair for int8, one conversion for E4M3), and q (QDT) is
  // carried in fp16 with a power-of-two prescale per (sequence, KV head) pair
  // (load_q).
  using Base = MfmaWave<PA_F16, D, NCT_>;
  using typename Base::v8;
  using Base::NC;
  using Base::NCT;
  using Base::NT;
  static constexpr int NV = D / 64;        // 16-byte code vectors per lane and tile
  static constexpr int TILE = kBS * (D + 4);  // bytes per (block, head) tile: codes, then 16 row scales
  static constexpr bool kAppend = true;    // new rows (QDT) quantized as pa_reshape_and_cache_int8 / _fp8 do
  // The code conversions add ~250 VALU instructions per block: more waves per
  // SIMD hide their latency, a shallower ring keeps them in registers.  With
  // several column tiles the q fragments and accumulators no longer fit two
  // waves per SIMD: one wave per SIMD with a deeper ring instead.
  static constexpr int kBalRing = NCT > 1 ? 3 : FMT == PA_FP8 ? PA_FP8_RING : PA_I8_RING;
  // Partition kernel: a code tile is half a 16-bit tile, so three blocks per
  // wave hold as many bytes in flight as 1.5 16-bit blocks.
  static constexpr int kRing = 3;
  static constexpr int kBalWgPerCu = NCT > 1 ? 1 : FMT == PA_FP8 ? PA_FP8_WG_PER_CU : PA_I8_WG_PER_CU;

  struct Frag {
    u32x4_t k[NV];
    u32x4_t v[NV];
    f32x4_t ks, vs;
  };

  __device__ static void load_tile(Frag &f, const DecodeArgs &a, int64_t tile, int lane) {
    const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(a.k_cache + tile * TILE);
    const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(a.v_cache + tile * TILE);
#pragma unroll
    for (int x = 0; x < NV; ++x) f.k[x] = __builtin_nontemporal_load(&kp[x * 64 + lane]);
#pragma unroll
    for (int x = 0; x < NV; ++x) f.v[x] = __builtin_nontemporal_load(&vp[x * 64 + lane]);
    // the tile's 16 row scales follow its codes (lane l takes those of its tokens 4(l/16) ..)
    const f32x4_t *ksp = reinterpret_cast<const f32x4_t *>(a.k_cache + tile * TILE + kBS * D);
    const f32x4_t *vsp = reinterpret_cast<const f32x4_t *>(a.v_cache + tile * TILE + kBS * D);
    f.ks = __builtin_nontemporal_load(&ksp[lane / 16]);
    f.vs = __builtin_nontemporal_load(&vsp[lane / 16]);
  }

  // Codes i, i+1 of w as a packed pair of fp16 values, exactly: each byte b
  // goes under a 0x64 high byte with its top bit flipped, which is the fp16
  // value 1024 + (b ^ 0x80) = 1152 + int8(b); one packed subtraction of 1152
  // leaves int8(b).
  __device__ static uint32_t pair16(uint32_t w, int i) {
    using h2 = _Float16 __attribute__((ext_vector_type(2)));
    if constexpr (FMT == PA_FP8) {
      // every finite E4M3 value is an fp16 value (3 mantissa bits, 2^-9 .. 448)
      return i == 0 ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false))
                    : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
    } else {
      // (one XOR flips the top bits of all four bytes; the permute then puts
      // two of them under 0x64 high bytes)
      const uint32_t biased = __builtin_amdgcn_perm(0x64646464u, w ^ 0x80808080u, i == 0 ? 0x04010400u : 0x04030402u);
      const h2 x = __builtin_bit_cast(h2, biased) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
      return __builtin_bit_cast(uint32_t, x);
    }
  }

  float qscale;  // 2^-e undoes the prescale of q in the scores

  // Element e (0..7) of 8 packed QDT values as float32.
  __device__ static float qval(const u32x4_t &w, int e) {
    const uint32_t h = (w[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
    if constexpr (QDT == PA_BF16)
      return __uint_as_float(h << 16);
    else
      return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }

  // q rows (QDT) -> fp16 fragments scaled by 2^e, e chosen per wave so the
  // largest |q| of the G rows lands in [2^14, 2^15): a bf16 or fp16 value is
  // then exact in fp16 unless it is below 2^-28 of that largest one.
  template <class P>
  __device__ void load_q(const P *rows, int G, int lane) {
    const int r = lane % 16, tq = lane / 16;
    u32x4_t w[NCT][NC];
    float mx = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int h = 16 * ct + r;
      const u32x4_t *qrow = reinterpret_cast<const u32x4_t *>(rows) + (h < G ? h : 0) * (D / 8);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        w[ct][c] = qrow[4 * c + tq];
        if (h >= G) w[ct][c] = u32x4_t{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qval(w[ct][c], e)));
      }
    }
    mx = max_xor32(max_xor16(row_max16(mx)));
    int ex = 0;
    if (mx > 0.f && mx == mx && mx != INFINITY) {
      int k;
      (void)frexpf(mx, &k);  // mx = f * 2^k, f in [0.5, 1)
      ex = min(max(15 - k, -126), 126);  // 2^ex and 2^-ex stay finite
    }
    const float up = ldexpf(1.f, ex);
    qscale = ldexpf(1.f, -ex);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          h[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(qval(w[ct][c], 2 * e) * up)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(qval(w[ct][c], 2 * e + 1) * up)) << 16);
        this->qB[ct][c] = __builtin_bit_cast(v8, u32x4_t{h[0], h[1], h[2], h[3]});
      }
    }
  }

  // Fused append: a new row (QDT bits, two elements per lane, lanes < D/2)
  // quantized as the append kernel does (the same scale and the same code per
  // element), staged as D code bytes in dim order with the scale after them.
  // Called by the whole wave; the K and V row maxima are reduced together
  // (DPP and lane swaps; a maximum does not depend on the order).
  __device__ static void stage_row(uint32_t *dst, float x0, float x1, float scale, int lane) {
    if (lane < D / 2)
      reinterpret_cast<uint16_t *>(dst)[lane] =
          (uint16_t)((code_of<FMT>(x0, scale) & 0xFF) | ((code_of<FMT>(x1, scale) & 0xFF) << 8));
    if (lane == 0) reinterpret_cast<float *>(dst)[D / 4] = scale;
  }
  __device__ static void stage_new(uint32_t *kdst, uint32_t *vdst, uint32_t kr, uint32_t vr, int lane) {
    const bool mine = lane < D / 2;
    const float k0 = mine ? half_value<QDT>(kr & 0xFFFFu) : 0.f, k1 = mine ? half_value<QDT>(kr >> 16) : 0.f;
    const float v0 = mine ? half_value<QDT>(vr & 0xFFFFu) : 0.f, v1 = mine ? half_value<QDT>(vr >> 16) : 0.f;
    float km = fmaxf(fmaxf(0.f, fabsf(k0)), fabsf(k1));
    float vm = fmaxf(fmaxf(0.f, fabsf(v0)), fabsf(v1));
    km = row_max16(km);
    vm = row_max16(vm);
    km = max_xor32(max_xor16(km));
    vm = max_xor32(max_xor16(vm));
    stage_row(kdst, k0, k1, code_scale<FMT>(km), lane);
    stage_row(vdst, v0, v1, code_scale<FMT>(vm), lane);
  }
  // Codes and scales of a staged token into its slot (tile layouts as in
  // pa_reshape_and_cache_int8).
  __device__ static void write_new(const DecodeArgs &a, int64_t blk, int t, int g, const uint32_t *knew,
                                   const uint32_t *vnew, int lane) {
    const int64_t tile = blk * a.num_kv_heads + g;
    uint8_t *kc = const_cast<uint8_t *>(a.k_cache) + tile * TILE;
    uint8_t *vc = const_cast<uint8_t *>(a.v_cache) + tile * TILE;
    const uint8_t *kb = reinterpret_cast<const uint8_t *>(knew), *vb = reinterpret_cast<const uint8_t *>(vnew);
    for (int d = lane; d < D; d += 64) {
      kc[k_code_off(d, t)] = kb[d];
      vc[v_code_off(d, t)] = vb[d];
    }
    if (lane == 0) {
      reinterpret_cast<float *>(kc + kBS * D)[t] = reinterpret_cast<const float *>(knew)[D / 4];
      reinterpret_cast<float *>(vc + kBS * D)[t] = reinterpret_cast<const float *>(vnew)[D / 4];
    }
  }
  // Replaces token t's codes and scales in a tile's fragments with the staged
  // row (register indices all compile-time constants).
  __device__ static void patch_new(Frag &f, int t, int lane, const uint32_t *knew, const uint32_t *vnew) {
    const int r = lane % 16, tq = lane / 16;
#pragma unroll
    for (int x = 0; x < NV; ++x) {  // K vector x of lane (tq, t): dims 64x + 8tq .., 64x + 32 + 8tq ..
      const uint32_t *lo = knew + (64 * x + 8 * tq) / 4;
      const uint32_t *hi = knew + (64 * x + 32 + 8 * tq) / 4;
      const u32x4_t kx = {lo[0], lo[1], hi[0], hi[1]};
      f.k[x] = r == t ? kx : f.k[x];
    }
    const bool in_quad = tq == t / 4;
    const int sh = 8 * (t % 4);
    const uint32_t keep = ~(0xFFu << sh);
    const uint8_t *vb = reinterpret_cast<const uint8_t *>(vnew);
#pragma unroll
    for (int x = 0; x < NV; ++x) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // byte 4j + i = (token 4tq + i, dim 64x + 16j + r)
        const uint32_t c = vb[64 * x + 16 * j + r];
        f.v[x][j] = in_quad ? ((f.v[x][j] & keep) | (c << sh)) : f.v[x][j];
      }
    }
    const float ksc = reinterpret_cast<const float *>(knew)[D / 4];
    const float vsc = reinterpret_cast<const float *>(vnew)[D / 4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool hit = in_quad && i == t % 4;
      f.ks[i] = hit ? ksc : f.ks[i];
      f.vs[i] = hit ? vsc : f.vs[i];
    }
  }

  __device__ void compute(Frag &f, uint32_t vm, float scale_log2, int lane, int new_tok,
                          const uint32_t *knew, const uint32_t *vnew) {
    const int tq = lane / 16;
    if (new_tok >= 0) patch_new(f, new_tok, lane, knew, vnew);
    const uint32_t mine = vm >> (4 * tq);
    // K codes as fp16 A operands, once for every column tile
    v8 kb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t w0 = f.k[c / 2][(c % 2) * 2], w1 = f.k[c / 2][(c % 2) * 2 + 1];
      kb[c] = __builtin_bit_cast(v8, u32x4_t{pair16(w0, 0), pair16(w0, 2), pair16(w1, 0), pair16(w1, 2)});
    }
    if constexpr (FMT == PA_FP8) {
      // an unwritten or stale E4M3 slot may hold a NaN code: clear the V
      // bytes of tokens outside the attended range (a word holds this
      // lane's four tokens of one dim, one byte each)
      if (vm != kAllTokens) {
        const uint32_t bm = ((mine & 1u) ? 0x000000FFu : 0u) | ((mine & 2u) ? 0x0000FF00u : 0u) |
                            ((mine & 4u) ? 0x00FF0000u : 0u) | ((mine & 8u) ? 0xFF000000u : 0u);
#pragma unroll
        for (int x = 0; x < NV; ++x) f.v[x] &= u32x4_t{bm, bm, bm, bm};
      }
    }
    const float sl = scale_log2 * qscale;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) sc = Base::mma_qk(kb[c], this->qB[ct][c], sc);
      float s[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) s[v] = sc[v] * f.ks[v] * sl;
      // tokens outside the attended range: scores masked (their scales may be anything)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[v] = ((mine >> v) & 1u) ? s[v] : -INFINITY;
      float p[4], pw[4];
      this->softmax_step(ct, s, p);
#pragma unroll
      for (int v = 0; v < 4; ++v) pw[v] = ((mine >> v) & 1u) ? p[v] * f.vs[v] : 0.f;
      u32x2_t ph, pl;
      Base::split(pw, ph, pl);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint32_t w = f.v[n / 4][n % 4];
        const u32x2_t av = {pair16(w, 0), pair16(w, 2)};
        this->acc[ct][n] = Base::mma_pv(av, ph, this->acc[ct][n]);
        this->acc[ct][n] = Base::mma_pv(av, pl, this->acc[ct][n]);
      }
    }
  }
};

// ============================================================================
// Vector-ALU wave: any cache type, GM = compile-time bound on the heads one
// workgroup takes (at most 16: a group of more than 16 query heads is split
// into 16-head chunks, one workgroup each, that read the same blocks).
//
// With X = 16 / element bytes and NC = D*bytes/1024 sixteen-byte fragments:
//   K fragment c of lane l holds token r = l % 16, dims X*(4c + tq) .. +X-1;
//   V fragment c holds tokens 4tq..4tq+3 of dims c*4X + sub*16 + r
//   (sub < X/4).  q comes from LDS.  A token's score is reduced over the
//   four lanes that share r; the block max over the 16 lanes of a row; the
//   weights go through LDS to the lanes that hold the matching V tokens.
// ============================================================================
template <int DT, int D, int GM>
struct ValuWave {
  static constexpr int EB = Ty<DT>::bytes;
  static constexpr int X = 16 / EB;
  static constexpr int NCF = D * EB / 64;  // 16-byte fragments per lane per tile
  static constexpr int VD = D / 16;        // V dims per lane
  static constexpr int TILE = kBS * D * EB;
  static constexpr int kRing = 2;
  using Smem = SmemValu;

  struct Frag {
    u32x4_t k[NCF];
    u32x4_t v[NCF];
  };

  float acc[GM][VD];  // partial over this lane's 4-token quad
  float m[GM], l[GM];

  // q rows h0 .. h0+G-1 of sequence s (G <= 16) into LDS as float32.
  __device__ void stage(const DecodeArgs &a, Smem &sm, int s, int h0, int G, int tid) {
    const uint8_t *qb = static_cast<const uint8_t *>(a.q);
    for (int i = tid; i < G * D; i += kThreads) {
      const int64_t e = ((int64_t)s * a.num_q_heads + h0) * D + i;
      uint32_t bits;
      if constexpr (EB == 4)
        bits = reinterpret_cast<const uint32_t *>(qb)[e];
      else
        bits = reinterpret_cast<const uint16_t *>(qb)[e];
      sm.qs[i / D][i % D] = Ty<DT>::to_f32(bits);
    }
  }

  __device__ void reset() {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int k = 0; k < VD; ++k) acc[h][k] = 0.f;
    }
  }

  __device__ static void load(Frag &f, const uint8_t *ktile, const uint8_t *vtile, int lane) {
    const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(ktile);
    const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vtile);
#pragma unroll
    for (int c = 0; c < NCF; ++c) f.k[c] = __builtin_nontemporal_load(&kp[c * 64 + lane]);
#pragma unroll
    for (int c = 0; c < NCF; ++c) f.v[c] = __builtin_nontemporal_load(&vp[c * 64 + lane]);
  }

  // element e (0..X-1) of a 16-byte fragment as float
  __device__ static float elem(const u32x4_t &x, int e) {
    if constexpr (EB == 4) {
      return __uint_as_float(x[e]);
    } else {
      const uint32_t wrd = x[e / 2];
      return Ty<DT>::to_f32((e & 1) ? (wrd >> 16) : (wrd & 0xFFFFu));
    }
  }

  __device__ void compute(Frag &f, uint32_t vm, float scale_log2, int lane, int new_tok, Smem &sm,
                          int w, int G) {
    const int r = lane % 16, tq = lane / 16;
    if (new_tok >= 0) patch_new_token<EB, NCF>(f.k, f.v, new_tok, lane, sm.knew, sm.vnew);
    float kf[NCF * X];
#pragma unroll
    for (int c = 0; c < NCF; ++c)
#pragma unroll
      for (int e = 0; e < X; ++e) kf[c * X + e] = elem(f.k[c], e);
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < NCF; ++c) {
          const float *qv = &sm.qs[h][X * (4 * c + tq)];
#pragma unroll
          for (int e = 0; e < X; ++e) part = fmaf(qv[e], kf[c * X + e], part);
        }
        part = sum_xor32(sum_xor16(part));
        const float sv = ((vm >> r) & 1u) ? part * scale_log2 : -INFINITY;
        const float mx = row_max16(sv);
        const float m_new = fmaxf(m[h], mx);
        const float alpha = exp2_neg(m[h] - m_new);
        const float pv = exp2_neg(sv - m_new);
        l[h] = l[h] * alpha + pv;
        m[h] = m_new;
        if (tq == 0) sm.ps[w][h][r] = pv;
#pragma unroll
        for (int k = 0; k < VD; ++k) acc[h][k] *= alpha;
      }
    }
    // V of this lane: VD dims x 4 tokens (4tq + i), zeroed past the context
    float vf[VD][4];
#pragma unroll
    for (int c = 0; c < NCF; ++c)
#pragma unroll
      for (int sub = 0; sub < X / 4; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = elem(f.v[c], sub * 4 + i);
          vf[c * (X / 4) + sub][i] = ((vm >> (4 * tq + i)) & 1u) ? x : 0.f;
        }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const f32x4_t pq = *reinterpret_cast<const f32x4_t *>(&sm.ps[w][h][4 * tq]);
#pragma unroll
        for (int k = 0; k < VD; ++k)
          acc[h][k] = fmaf(pq[0], vf[k][0],
                           fmaf(pq[1], vf[k][1], fmaf(pq[2], vf[k][2], fmaf(pq[3], vf[k][3], acc[h][k]))));
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  __device__ void finish(Smem &sm, int w, int lane, int G) {
    const int r = lane % 16, tq = lane / 16;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float lt = row_sum16(l[h]);
#pragma unroll
        for (int k = 0; k < VD; ++k) {
          const float a = sum_xor32(sum_xor16(acc[h][k]));
          const int dim = (k / (X / 4)) * 4 * X + (k % (X / 4)) * 16 + r;
          if (tq == 0) sm.acc[w][h][dim] = a;
        }
        if (lane == 0) {
          sm.m[w][h] = m[h];
          sm.l[w][h] = lt;
        }
      }
    }
  }
};

// ---------------------------------------------------------------- partition kernel
template <int D>
__device__ void write_rows(const DecodeArgs &a, int s, int h0, int G, float val) {
  for (int i = threadIdx.x; i < G * D; i += kThreads)
    store_out(a.out, ((int64_t)s * a.num_q_heads + h0 + i / D) * D + i % D, val, a.out_dtype);
}

template <int D>
__device__ void write_partial_nan(const DecodeArgs &a, int s, int h0, int G, int p) {
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int64_t row = ((int64_t)s * a.num_q_heads + h0 + i / D) * a.max_parts + p;
    a.ws_acc[row * D + i % D] = NAN;
    if (i % D == 0) {
      a.ws_ml[row * 2] = NAN;
      a.ws_ml[row * 2 + 1] = NAN;
    }
  }
}

// Partition workgroups per CU: the matrix-core wave's choice (three for one
// column tile: 3 waves per SIMD, <= 168 VGPRs); one for the vector-ALU wave.
template <class W, bool kMfma>
constexpr int partition_wg_per_cu() {
  if constexpr (kMfma)
    return W::kPartWgPerCu;
  else
    return 1;
}

// Column tiles of the wave's state (the vector-ALU wave holds one group of
// at most 16 heads).
template <class W, bool kMfma>
constexpr int wave_tiles() {
  if constexpr (kMfma)
    return W::NCT;
  else
    return 1;
}

template <class W, int D, bool kMfma>
__global__ __launch_bounds__(kThreads, (partition_wg_per_cu<W, kMfma>())) void pa_partition_kernel(DecodeArgs a) {
  __shared__ typename W::Smem sm;
  // 1-D grid, KV head fastest, then sequence, then partition.  Workgroups are
  // dealt round-robin to the 8 XCDs by linear id, so this order spreads every
  // sequence's (unequal) partitions evenly over the XCDs; with the partition
  // index fastest, partition p of every sequence would land on the same XCD.
  // The vector-ALU wave takes at most 16 heads: a larger group is split into
  // 16-head chunks, the fastest grid index (they read the same blocks at
  // about the same time).
  const int G = a.group;
  const int nch = kMfma ? 1 : (G + kTileCols - 1) / kTileCols;
  const int hc = kMfma ? 0 : (int)(blockIdx.x % nch);
  const int id = kMfma ? (int)blockIdx.x : (int)(blockIdx.x / nch);
  const int g = id % a.num_kv_heads;
  const int s = (id / a.num_kv_heads) % a.num_seqs;
  const int p = id / (a.num_kv_heads * a.num_seqs);
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
  const int h0 = g * G + hc * kTileCols;        // first query head of this workgroup
  const int Gc = min(G - hc * kTileCols, kMfma ? G : kTileCols);  // and how many
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // Loads that do not depend on the context length go out together with it:
  // the q fragments, and this wave's first 64 block ids (speculative: only
  // bounded by the table row; validated once the length is known).
  // Partitions split the attended blocks: from the block holding the
  // window's first position (block 0 without a window) to the last one.
  const int L = a.context_lens[s];
  int blk0 = (int)((int64_t)p * a.part_tokens / kBS);
  const int32_t *trow = a.block_tables + (int64_t)s * a.max_blocks + blk0;
  int ids_first = (int64_t)blk0 + wu + lane * kWaves < a.max_blocks ? trow[wu + lane * kWaves] : 0;
  W wave;
  if constexpr (kMfma)
    wave.init(a, s, g, lane);
  else
    wave.reset();
  if (!ctx_valid(L, a)) {
    if (p == 0) write_rows<D>(a, s, h0, Gc, NAN);
    return;
  }
  if (L == 0) {
    if (p == 0) write_rows<D>(a, s, h0, Gc, 0.f);
    return;
  }
  const int first = window_first_token(L, a.window);
  const int jb = first / kBS;
  const int nparts = (L - jb * kBS + a.part_tokens - 1) / a.part_tokens;
  if (p >= nparts) return;
  if (jb > 0) {  // the speculative id load above assumed no window
    blk0 += jb;
    trow += jb;
    ids_first = (int64_t)blk0 + wu + lane * kWaves < a.max_blocks ? trow[wu + lane * kWaves] : 0;
  }
  const int tok0 = blk0 * kBS;
  const int tok1 = min(L, tok0 + a.part_tokens);
  const int nblk = (tok1 - tok0 + kBS - 1) / kBS;
  const int last_valid = tok1 - (blk0 + nblk - 1) * kBS;
  const int first_lo = p == 0 ? first - jb * kBS : 0;  // masked tokens of the partition's block 0

  if constexpr (!kMfma) {
    wave.stage(a, sm, s, h0, Gc, tid);
    __syncthreads();  // q staged in LDS
  }
  int bad = 0;  // a block id outside the pool was seen (never dereferenced)
  // Fused append (one new token per sequence, at position L-1, in the last
  // block of the last partition): the wave that computes that block checks
  // the slot against the table, stages the token's K/V rows for head g in
  // LDS, stores them into the slot (only the first head chunk's workgroup),
  // and later takes the token from LDS.  A slot that is not position L-1's
  // slot marks the sequence bad: nothing is written and the row is NaN.
  // Only that wave is involved (no barrier).
  int new_tok = -1;
  if (a.k_new != nullptr && p == nparts - 1 && wu == (nblk - 1) % kWaves) {
    const int64_t slot = a.slot_mapping[s];
    if (slot >= 0) {
      const int pos = L - 1;
      const int32_t blk = trow[nblk - 1];
      if ((uint32_t)blk >= (uint32_t)a.num_blocks || slot != (int64_t)blk * kBS + pos % kBS) {
        bad = 1;
      } else {
        constexpr int EB = W::TILE / (kBS * D);
        const int64_t row = ((int64_t)s * a.num_kv_heads + g) * D * EB;  // bytes
        for (int i = lane; i < D * EB / 4; i += 64) {
          sm.knew[i] = reinterpret_cast<const uint32_t *>(a.k_new + row)[i];
          sm.vnew[i] = reinterpret_cast<const uint32_t *>(a.v_new + row)[i];
        }
        new_tok = pos % kBS;
        if (hc == 0)
          write_token_row<EB, D>(const_cast<uint8_t *>(a.k_cache), const_cast<uint8_t *>(a.v_cache),
                                 blk, new_tok, g, a.num_kv_heads, sm.knew, sm.vnew, lane);
      }
    }
  }

  const int64_t head_off = (int64_t)g * W::TILE;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * W::TILE;
  constexpr int NB = W::kRing;
  typename W::Frag fr[NB];
  const int nmine = nblk > wu ? (nblk - wu + kWaves - 1) / kWaves : 0;
  // Each wave streams its blocks (wu, wu+4, wu+8, ...) through a ring of NB
  // register fragments: block i is computed while blocks i+1 .. i+NB-1 are in
  // flight.  Block ids come 64 at a time, one per lane, and are read into
  // scalar registers.  Every ring slot is refilled unconditionally (past the
  // end a wave re-reads its last block, a valid address that hits in cache),
  // so the number of loads in flight is the same on every path and the
  // compiler's wait counts never drain the ring early.
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int nc = min(64, nmine - c0);
    int ids = c0 == 0 ? ids_first : trow[wu + (c0 + lane) * kWaves];
    ids = lane < nc ? ids : 0;
    const bool id_ok = (uint32_t)ids < (uint32_t)a.num_blocks;
    if (__builtin_amdgcn_ballot_w64(!id_ok)) bad = 1;
    ids = id_ok ? ids : 0;
    // Past the end of the chunk a ring slot is refilled with a dummy load of
    // the same shape in which every lane reads the pool's first 16 bytes.
    auto refill = [&](typename W::Frag &f, int i) {
      const bool real = i < nc;
      const int64_t off = real ? (int64_t)__builtin_amdgcn_readlane(ids, min(i, nc - 1)) * blk_stride + head_off : 0;
      W::load(f, a.k_cache + off, a.v_cache + off, real ? lane : 0);
    };
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) {
      refill(fr[b], b);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring's issue order
    }
    for (int i0 = 0; i0 < nc; i0 += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = i0 + b;
        refill(fr[(b + NB - 1) % NB], i + NB - 1);
        if (i < nc) {
          const int j = wu + (c0 + i) * kWaves;
          const uint32_t vm = token_mask(j == 0 ? first_lo : 0, (j == nblk - 1) ? last_valid : kBS);
          const int nt = (j == nblk - 1) ? new_tok : -1;
          if constexpr (kMfma)
            wave.compute(fr[b], vm, a.scale_log2, lane, nt, sm.knew, sm.vnew);
          else
            wave.compute(fr[b], vm, a.scale_log2, lane, nt, sm, w, Gc);
        }
      }
    }
  }
  // Fold the four wave states, one column tile (16 heads) at a time:
  // M = max m_w, out = sum 2^(m_w-M) acc_w / sum 2^(m_w-M) l_w.
  constexpr int kTiles = wave_tiles<W, kMfma>();
#pragma unroll
  for (int ct = 0; ct < kTiles; ++ct) {
    if constexpr (kMfma)
      wave.finish(sm, w, lane, Gc, ct);
    else
      wave.finish(sm, w, lane, Gc);
    if (ct == 0) {
      if (__syncthreads_or(bad)) {
        if (nparts == 1)
          write_rows<D>(a, s, h0, Gc, NAN);
        else
          write_partial_nan<D>(a, s, h0, Gc, p);
        return;
      }
    } else {
      lds_barrier();
    }
    const int hb = ct * kTileCols, nh = min(kTileCols, Gc - hb);  // heads of this tile
    // One weight per (wave, head) and the head's denominator first, then
    // four dims of a row per thread.
    if (tid < nh) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][tid]);
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = exp2f(sm.m[ww][tid] - M);  // 0 for a wave that saw no block
        sm.fac[ww][tid] = f;
        den += f * sm.l[ww][tid];
      }
      sm.mx[tid] = M;
      sm.den[tid] = den;
    }
    lds_barrier();
    constexpr int NQ = D / 4;
    for (int i = tid; i < nh * NQ; i += kThreads) {
      const int h = i / NQ, d4 = (i % NQ) * 4;
      f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) num += sm.fac[ww][h] * *reinterpret_cast<const f32x4_t *>(&sm.acc[ww][h][d4]);
      const int64_t row = (int64_t)s * a.num_q_heads + h0 + hb + h;
      if (nparts == 1) {
        const float den = sm.den[h];
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = num[e] / den;
        store_out4(a.out, row * D + d4, v, a.out_dtype);
      } else {
        const int64_t prow = row * a.max_parts + p;
        store_partial4(a.ws_acc + prow * D + d4, num);
        if (d4 == 0) {
          a.ws_ml[prow * 2] = sm.mx[h];
          a.ws_ml[prow * 2 + 1] = sm.den[h];
        }
      }
    }
    if (ct + 1 < kTiles) lds_barrier();  // the next tile reuses the LDS rows
  }
}

// ---------------------------------------------------------------- balanced split
// Matrix-core path with automatic partitioning.  The work is the list of
// units (sequence s, KV head g, block j), ordered by s, then g, then j, with
// ceil(L_s / 16) blocks per (s, g) pair.  A persistent grid (every wave slot
// of the GPU once, NW waves) cuts the list into NW equal contiguous shares
// of C = ceil(U / NW) units, so every wave streams the same number of K/V
// tiles whatever the mix of context lengths, and no workgroup is spent on
// an empty partition.  A share covers pieces ("segments") of one or more
// pairs; each segment keeps one online-softmax state.  A segment that is a
// whole pair writes its output rows itself; any other writes an (m, l, acc)
// partial into slot w + pair.  Walking along the unit list, every new
// segment starts a new wave share or a new pair (or both), so w + pair grows
// strictly from segment to segment: no two segments share a slot, and the
// NW + S*Hkv - 1 slots cover every case.  The merge kernel folds the
// partials of each pair that was split.
constexpr int kBWaves = PA_BALANCED_WAVES;  // waves per balanced workgroup
constexpr int kBThreads = kBWaves * 64;
constexpr int kSeqMax = 1024;    // sequences per launch on this path
constexpr int kQLds = 16384;     // bytes of q staged per workgroup
constexpr int kAppendMax = 4;    // fused-append rows staged per wave and chunk

struct __align__(16) SmemBalanced {
  uint32_t q[kQLds / 4];                        // q rows of pairs qbase .. qbase+nq-1
  uint32_t knew[kBWaves][kAppendMax][kDMax / 2];  // fused append: new K / V rows (16-bit)
  uint32_t vnew[kBWaves][kAppendMax][kDMax / 2];
  int32_t pre[kSeqMax + 1];                      // attended blocks of the sequences before s
  int32_t len[kSeqMax];                          // context length (-1 when invalid)
};

// First table entry the balanced split streams for a context of L tokens:
// the block holding the window's first position, or the first block after a
// shared prefix (whose attention comes from the prefix kernel).
__device__ inline int first_block(int L, const DecodeArgs &a) {
  return a.prefix_blocks > 0 ? a.prefix_blocks : window_first_token(L, a.window) / kBS;
}

// Blocks the balanced split streams for a context of L tokens (L = -1:
// invalid, none): from first_block to the one holding position L-1.
__device__ inline int attended_blocks(int L, const DecodeArgs &a) {
  return L > 0 ? (L + kBS - 1) / kBS - first_block(L, a) : 0;
}

// Floats of one wave's parking area: G rows of D, then m and l per row
// (rounded to 16 bytes).
__host__ __device__ constexpr int park_floats(int G, int D) { return (G * (D + kAccPad + 2) + 3) / 4 * 4; }
// One parking slot: the state, then its output row, partial row (int64) and flags.
__host__ __device__ constexpr int park_slot_floats(int G, int D) { return park_floats(G, D) + 8; }
#ifndef PA_PARK_SLOTS_MAX
#define PA_PARK_SLOTS_MAX 8
#endif
constexpr int kParkSlotsMax = PA_PARK_SLOTS_MAX;

// Per-unit flags, one unit per lane.
constexpr uint32_t kUValid = 0x1Fu;         // tokens of the block inside the context (1..16)
constexpr uint32_t kUFirst = 1u << 5;       // first unit of a segment
constexpr uint32_t kULast = 1u << 6;        // last unit of a segment
constexpr uint32_t kUPairStart = 1u << 7;   // block 0 of its pair
constexpr uint32_t kUPairEnd = 1u << 8;     // last block of its pair
constexpr uint32_t kUBad = 1u << 9;         // block id outside the pool, or a foreign slot
constexpr uint32_t kUNew = 1u << 10;        // holds the fused-append token
constexpr int kUNewTokShift = 11;           // its position in the block (4 bits)
constexpr int kUNewIdxShift = 15;           // its staging row (2 bits)
constexpr int kUPairShift = 17;             // (s, g) pair index s*Hkv + g (15 bits)
constexpr int kPairMax = 1 << 15;

// Instruction-issue priority of this wave (0..3).  The sequencer favours
// older waves; a wave of the balanced split (byte caches) or of an
// eight-wave extend workgroup lowers its priority as it works through its
// share, so waves that started later (or were starved) catch up and all
// shares end together.
__device__ inline void set_wave_priority(int level) {
  switch (level) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// Sequence that holds block b of the concatenated block list: the last s with pre[s] <= b.
__device__ inline int seq_of_block(const SmemBalanced &sm, int b, int S) {
  int lo = 0, hi = S;  // pre[lo] <= b < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sm.pre[mid] <= b) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline int pair_of_unit(const SmemBalanced &sm, int u, int Hkv, int S) {
  const int s = seq_of_block(sm, u / Hkv, S);
  const int nb = sm.pre[s + 1] - sm.pre[s];
  return s * Hkv + (u - Hkv * sm.pre[s]) / nb;
}

template <class W, int D>
__global__ __launch_bounds__(kBThreads, W::kBalWgPerCu) void pa_balanced_kernel(DecodeArgs a) {
  WaveTrace tr;
  tr.stamp(0);
  __shared__ SmemBalanced sm;
  extern __shared__ __align__(16) float park_lds[];  // kBWaves x park_slots x park_slot_floats(G, D)
  const int tid = threadIdx.x, lane = tid % 64;
  const int wu = __builtin_amdgcn_readfirstlane(tid / 64);
  const int S = a.num_seqs, Hkv = a.num_kv_heads, G = a.group;

  // Context lengths, then block offsets by an exclusive scan (wave 0: each
  // lane sums a run of ceil(S/64) sequences, then a scan across lanes).
  for (int s = tid; s < S; s += kBThreads) {
    const int L = a.context_lens[s];
    // -1: invalid (no blocks, NaN rows); with a shared prefix a context must
    // reach past it
    sm.len[s] = ctx_valid(L, a) && (a.prefix_blocks == 0 || L > a.prefix_blocks * kBS) ? L : -1;
  }
  __syncthreads();
  if (wu == 0) {
    const int per = (S + 63) / 64;
    const int s0 = min(S, lane * per), s1 = min(S, s0 + per);
    int sum = 0;
    for (int s = s0; s < s1; ++s) sum += attended_blocks(sm.len[s], a);
    int inc = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    int run = inc - sum;
    for (int s = s0; s < s1; ++s) {
      sm.pre[s] = run;
      run += attended_blocks(sm.len[s], a);
    }
    if (lane == 63) sm.pre[S] = inc;
  }
  __syncthreads();
  tr.stamp(1);
  const int U = Hkv * sm.pre[S];
  const int NW = a.num_workers;
  const int C = (U + NW - 1) / NW;
  if (blockIdx.x == 0)
    for (int s = tid; s <= S; s += kBThreads) a.ws_pre[s] = sm.pre[s];
  // Rows of empty (L = 0: zeros) and invalid (NaN) contexts, spread over the grid.
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    const int L = sm.len[s];
    if (L <= 0) {
      const f32x4_t v = L == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : f32x4_t{NAN, NAN, NAN, NAN};
      for (int e = tid * 4; e < a.num_q_heads * D; e += kBThreads * 4)
        store_out4(a.out, (int64_t)s * a.num_q_heads * D + e, v, a.out_dtype);
    }
  }
  const int wg0 = blockIdx.x * kBWaves * C;
  if (wg0 >= U) return;  // the whole workgroup is idle
  const int wg1 = min(U, wg0 + kBWaves * C);
  const int w = blockIdx.x * kBWaves + wu;
  const int u0 = w * C, u1 = min(U, u0 + C);
  constexpr int EB = 2;
  // A chunk's units, one per lane, with their loads issued: the block id and,
  // for fused appends, the slots and new K / V rows of the units holding a
  // pair's last position (at most kAppendMax per chunk: the chunk ends early).
  struct ChunkHead {
    int nc, s, g, j, L, nb, id;
    uint64_t amask;
    int64_t slot_l;
    int pos[kAppendMax];
    uint32_t kr[kAppendMax], vr[kAppendMax];
  };
  auto chunk_head = [&](int c0) {
    ChunkHead h;
    h.nc = min(64, u1 - c0);
    const int u = min(c0 + lane, u1 - 1);
    h.s = seq_of_block(sm, u / Hkv, S);
    h.nb = sm.pre[h.s + 1] - sm.pre[h.s];
    const int off = u - Hkv * sm.pre[h.s];
    h.g = off / h.nb;
    h.j = off - h.g * h.nb;
    h.L = sm.len[h.s];
    const int jb = first_block(h.L, a);  // attended block j is table entry jb + j
    h.id = a.block_tables[(int64_t)h.s * a.max_blocks + jb + h.j];
    h.amask = 0;
    if (W::kAppend && a.k_new != nullptr) {
      h.amask = __builtin_amdgcn_ballot_w64(lane < h.nc && h.j == h.nb - 1);
      uint64_t rest = h.amask;
#pragma unroll
      for (int k = 0; k < kAppendMax; ++k) rest &= rest - 1;
      if (rest) {
        h.nc = __builtin_ctzll(rest);
        h.amask &= (1ull << h.nc) - 1;
      }
    }
    h.slot_l = ((h.amask >> lane) & 1) ? a.slot_mapping[h.s] : -1;
    uint64_t mm = h.amask;
#pragma unroll
    for (int k = 0; k < kAppendMax; ++k) {
      h.pos[k] = mm ? __builtin_ctzll(mm) : -1;
      mm &= mm - 1;
      h.kr[k] = h.vr[k] = 0;
      if (h.pos[k] >= 0 && lane < D * EB / 4) {
        const int sk = __builtin_amdgcn_readlane(h.s, h.pos[k]), gk = __builtin_amdgcn_readlane(h.g, h.pos[k]);
        const int64_t row = ((int64_t)sk * Hkv + gk) * D * EB / 4;
        h.kr[k] = reinterpret_cast<const uint32_t *>(a.k_new)[row + lane];
        h.vr[k] = reinterpret_cast<const uint32_t *>(a.v_new)[row + lane];
      }
    }
    return h;
  };
  // The first chunk's loads go out with the q staging below (one latency for both).
  ChunkHead h;
  if (u0 < u1) h = chunk_head(u0);

  // q rows of the pairs this workgroup touches (as many as fit), contiguous in q.
  const int pair_bytes = G * D * 2;
  const int qbase = pair_of_unit(sm, wg0, Hkv, S);
  const int nq = min(pair_of_unit(sm, wg1 - 1, Hkv, S) - qbase + 1, kQLds / pair_bytes);
  // Every q load goes out before the first LDS write: one memory latency.
  constexpr int kQPer = kQLds / 16 / kBThreads;
  static_assert(kQLds % (16 * kBThreads) == 0, "q staging: whole vectors per thread");
  const int nvec = nq * pair_bytes / 16;
  u32x4_t qv[kQPer];
  {
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                                           (int64_t)qbase * pair_bytes);
#pragma unroll
    for (int k = 0; k < kQPer; ++k)
      if (tid + k * kBThreads < nvec) qv[k] = src[tid + k * kBThreads];
  }
  // A wave writes its q vectors to LDS once its first blocks are requested:
  // the q loads are older than the ring's, so waiting for them leaves the
  // ring in flight.  Every wave passes this barrier exactly once (an idle
  // wave right away, any other in its first chunk); it orders LDS only.
  auto q_to_lds = [&]() {
#pragma unroll
    for (int k = 0; k < kQPer; ++k)
      if (tid + k * kBThreads < nvec) reinterpret_cast<u32x4_t *>(sm.q)[tid + k * kBThreads] = qv[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  if (u0 >= u1) {
    q_to_lds();
    tr.write(w, lane, 0);
    return;
  }

  W wave;
  constexpr int NB = W::kBalRing;  // blocks held in registers per wave
  typename W::Frag fr[NB];
  bool bad = false, whole = false;
  // A segment that ends before the wave's share does is parked in LDS (up
  // to park_slots of them, sized by the host to the LDS left) and written
  // when the share is done: stores count in the same counter as the ring's
  // loads, so a store in mid-stream would make the next block wait for its
  // acknowledgement.
  const int slot_f = park_slot_floats(G, D);
  float *park = park_lds + wu * a.park_slots * slot_f;
  int nparked = 0;
  for (int c0 = u0; c0 < u1;) {
    // ---- this chunk's units, one per lane
    if (c0 != u0) h = chunk_head(c0);
    const int nc = h.nc, s = h.s, g = h.g, L = h.L;
    const bool pend = h.j == h.nb - 1;
    int id = lane < nc ? h.id : 0;
    uint32_t meta = (uint32_t)(pend ? L - (first_block(L, a) + h.nb - 1) * kBS : kBS) |
                    (h.j == 0 ? kUPairStart : 0u) | (pend ? kUPairEnd : 0u) |
                    (c0 + lane == u0 || h.j == 0 ? kUFirst : 0u) |
                    (c0 + lane == u1 - 1 || pend ? kULast : 0u);
    // Cache rows of this chunk's appended tokens, written after its stream
    // (the blocks' fragments take the token from LDS, so the store may come
    // later; stores issued before the ring's loads would make its first wait
    // cover their acknowledgement too).
    int n_app = 0;
    int app_blk[kAppendMax], app_tg[kAppendMax];
    if (h.amask) {
#pragma unroll
      for (int k = 0; k < kAppendMax; ++k) {
        if (h.pos[k] < 0) break;
        const int p = h.pos[k];
        const uint32_t slo = __builtin_amdgcn_readlane((uint32_t)h.slot_l, p);
        const uint32_t shi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)h.slot_l >> 32), p);
        const int64_t slot = (int64_t)(((uint64_t)shi << 32) | slo);
        if (slot < 0) continue;
        const int blk = __builtin_amdgcn_readlane(id, p);
        const int t = (__builtin_amdgcn_readlane(L, p) - 1) % kBS;
        if ((uint32_t)blk >= (uint32_t)a.num_blocks || slot != (int64_t)blk * kBS + t) {
          if (lane == p) meta |= kUBad;
          continue;
        }
        W::stage_new(sm.knew[wu][k], sm.vnew[wu][k], h.kr[k], h.vr[k], lane);
        app_blk[n_app] = blk;
        app_tg[n_app] = (k << 24) | (t << 16) | __builtin_amdgcn_readlane(g, p);
        ++n_app;
        if (lane == p) meta |= kUNew | ((uint32_t)t << kUNewTokShift) | ((uint32_t)k << kUNewIdxShift);
      }
    }
    if ((uint32_t)id >= (uint32_t)a.num_blocks) {
      meta |= kUBad;
      id = 0;
    }
    // Per unit only two registers stay live through the ring: the K/V tile
    // index (block * Hkv + g) and the flags with the pair index.
    const uint32_t tile = (uint32_t)id * (uint32_t)Hkv + (uint32_t)g;
    meta |= (uint32_t)(s * Hkv + g) << kUPairShift;

    // ---- stream the chunk through the register ring as the partition kernel
    // does; the online-softmax state carries over from chunk to chunk.
    auto refill = [&](typename W::Frag &f, int i) {
      const bool real = i < nc;
      W::load_tile(f, a, real ? (int64_t)__builtin_amdgcn_readlane(tile, min(i, nc - 1)) : 0, real ? lane : 0);
    };
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) {
      refill(fr[b], b);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c0 == u0) q_to_lds();
    for (int i0 = 0; i0 < nc; i0 += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = i0 + b;
        refill(fr[(b + NB - 1) % NB], i + NB - 1);
        if (i < nc) {
          // With several waves per SIMD (byte caches) the ones further along
          // their share yield issue slots to the others; with one wave per
          // SIMD (16-bit caches) it only cost time (1 % on workloads 3, 4, 7).
          if constexpr (W::kBalWgPerCu > 1) set_wave_priority((u1 - c0 - i) * 4 / (C + 1));
          const uint32_t mt = __builtin_amdgcn_readlane(meta, i);
          const int pq = (int)(mt >> kUPairShift);
          if (mt & kUFirst) {
            wave.reset();
            if (pq - qbase < nq) {
              wave.load_q(sm.q + (pq - qbase) * (pair_bytes / 4), G, lane);
            } else {
              wave.load_q(static_cast<const uint8_t *>(a.q) + (int64_t)pq * pair_bytes, G, lane);
              __builtin_amdgcn_s_waitcnt(0);  // keep the ring's wait counts static
            }
            bad = false;
            whole = (mt & kUPairStart) != 0;
          }
          bad |= (mt & kUBad) != 0;
          const int nt = (mt & kUNew) ? (int)((mt >> kUNewTokShift) & 15) : -1;
          const int k = (mt >> kUNewIdxShift) & 3;
          // The window's first block masks the tokens before its first position.
          const int lo = (a.window > 0 && (mt & kUPairStart))
                             ? window_first_token(sm.len[pq / Hkv], a.window) % kBS : 0;
          tr.first();
          wave.compute(fr[b], token_mask(lo, (int)(mt & kUValid)), a.scale_log2, lane, nt, sm.knew[wu][k],
                       sm.vnew[wu][k]);
          if (mt & kULast) {  // (a segment may go on into the next chunk)
            // With a shared prefix every pair leaves a partial and the merge
            // folds the prefix in: a fold here would make each wave's last
            // stores wait on loads of the prefix state, one after another.
            const bool wh = whole && (mt & kUPairEnd) && a.prefix_blocks == 0;
            if (c0 + i == u1 - 1 || nparked == a.park_slots) {  // (all parking places taken: it stores)
              wave.store_segment(a, (int64_t)pq * G, (int64_t)(w + pq) * G, wh, bad, lane, G);
            } else {
              float *st = park + nparked * slot_f;
              wave.park_segment(st, lane, G);
              if (lane == 0) {
                int64_t *meta_p = reinterpret_cast<int64_t *>(st + park_floats(G, D));
                meta_p[0] = (int64_t)pq * G;
                meta_p[1] = (int64_t)(w + pq) * G;
                meta_p[2] = (wh ? 1 : 0) | (bad ? 2 : 0);
              }
              ++nparked;
            }
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int x = 0; x < kAppendMax; ++x) {
      if (x < n_app) {
        const int k = app_tg[x] >> 24, t = (app_tg[x] >> 16) & 0xFF, gx = app_tg[x] & 0xFFFF;
        W::write_new(a, app_blk[x], t, gx, sm.knew[wu][k], sm.vnew[wu][k], lane);
      }
    }
    c0 += nc;
  }
  tr.stamp(3);
  for (int k = 0; k < nparked; ++k) {
    const float *st = park + k * slot_f;
    const int64_t *meta_p = reinterpret_cast<const int64_t *>(st + park_floats(G, D));
    const int64_t fl = meta_p[2];
    flush_parked<D>(a, st, meta_p[0], meta_p[1], (fl & 1) != 0, (fl & 2) != 0, lane, G);
  }
  tr.write(w, lane, (uint64_t)(u1 - u0));
}

// ---------------------------------------------------------------- merge kernel
// One wave per (sequence, query head) row with more than one partition:
//   M = max_p m_p,  out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.
// Each lane owns D/64 output dims and sums the partitions in order.  A NaN
// partial (bad table entry) makes the row NaN.
constexpr int kMergeWaves = 4;

// Folds np partials (m, l at ml + q*ml_stride, acc at acc + q*acc_stride)
// into one output row.
template <int D>
__device__ void merge_row(void *out, int out_dtype, int64_t row, const float *ml, int64_t ml_stride,
                          const float *acc, int64_t acc_stride, int np, int lane, const float *xml = nullptr,
                          const float *xacc = nullptr) {
  // xml / xacc: one more partial (m, l) and acc row at its own place (a shared
  // prefix), or null.
  constexpr int PER = D / 64;  // output dims per lane
  constexpr int kFew = 8;
  float xm = -INFINITY, xl = 0.f, xa[PER];
  if (xml) {
    xm = xml[0];
    xl = xml[1];
#pragma unroll
    for (int e = 0; e < PER; ++e) xa[e] = xacc[lane * PER + e];
  }
  float M = xm;
  bool nan = xm != xm;
  float den = 0.f;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  if (np <= kFew) {
    // Every load first (one memory round trip), then the same arithmetic in
    // the same order as the general loop below.
    float mv[kFew], lv[kFew], av[kFew][PER];
#pragma unroll
    for (int q = 0; q < kFew; ++q) {
      if (q < np) {
        mv[q] = ml[q * ml_stride];
        lv[q] = ml[q * ml_stride + 1];
#pragma unroll
        for (int e = 0; e < PER; ++e) av[q][e] = acc[q * acc_stride + lane * PER + e];
      }
    }
#pragma unroll
    for (int q = 0; q < kFew; ++q) {
      if (q < np) {
        nan |= mv[q] != mv[q];
        M = fmaxf(M, mv[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < kFew; ++q) {
      if (q < np) {
        const float f = exp2f(mv[q] - M);
        den += f * lv[q];
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] += f * av[q][e];
      }
    }
  } else {
    // Many partials: their (m, l) 64 at a time, one per lane, then the acc
    // rows kFew at a time with every load of a batch issued first, so a
    // row costs about np / kFew memory round trips instead of np.
    for (int q0 = 0; q0 < np; q0 += 64) {
      const bool on = q0 + lane < np;
      const float mq = on ? ml[(int64_t)(q0 + lane) * ml_stride] : -INFINITY;
      nan |= __builtin_amdgcn_ballot_w64(on && mq != mq) != 0;
      M = fmaxf(M, max_xor32(max_xor16(row_max16(mq))));
    }
    for (int q0 = 0; q0 < np; q0 += 64) {
      const int nq = min(64, np - q0);
      const bool on = lane < nq;
      const float f = on ? exp2f(ml[(int64_t)(q0 + lane) * ml_stride] - M) : 0.f;
      const float fl = on ? f * ml[(int64_t)(q0 + lane) * ml_stride + 1] : 0.f;
      den += sum_xor32(sum_xor16(row_sum16(fl)));
      for (int qb = 0; qb < nq; qb += kFew) {
        // no branches between the loads (a batch past the end re-reads the
        // last partial with weight 0), so they all go out before one wait
        float av[kFew][PER];
#pragma unroll
        for (int k = 0; k < kFew; ++k) {
          const int64_t qk = q0 + min(qb + k, nq - 1);
#pragma unroll
          for (int e = 0; e < PER; ++e) av[k][e] = acc[qk * acc_stride + lane * PER + e];
        }
#pragma unroll
        for (int k = 0; k < kFew; ++k) {
          const float fk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(qb + k, nq - 1)));
          const float wk = qb + k < nq ? fk : 0.f;
#pragma unroll
          for (int e = 0; e < PER; ++e) num[e] += wk * av[k][e];
        }
      }
    }
  }
  if (xml) {
    const float f = exp2f(xm - M);
    den += f * xl;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += f * xa[e];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    store_out(out, row * D + lane * PER + e, nan ? NAN : num[e] / den, out_dtype);
}

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void pa_merge_kernel(DecodeArgs a, int32_t num_rows) {
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / 64;
  if (row >= num_rows) return;
  const int s = (int)(row / a.num_q_heads);
  const int L = a.context_lens[s];
  if (!ctx_valid(L, a)) return;
  const int skip = window_first_token(L, a.window) / kBS * kBS;  // tokens of the unattended blocks
  const int np = (L - skip + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  merge_row<D>(a.out, a.out_dtype, row, a.ws_ml + row * a.max_parts * 2, 2, a.ws_acc + row * a.max_parts * D, D, np, lane);
}

// Balanced split: the row of (s, head g*G + r) gathers the partials of its
// pair from slots w + pair, w = first .. last wave share that overlaps the
// pair's units.  A pair inside one share, and the rows of empty (L = 0) and
// invalid contexts, were written by the attention launch.
template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void pa_merge_balanced_kernel(DecodeArgs a, int32_t num_rows) {
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / 64;
  if (row >= num_rows) return;
  const int s = (int)(row / a.num_q_heads), h = (int)(row % a.num_q_heads);
  const int G = a.group, g = h / G, r = h % G, Hkv = a.num_kv_heads;
  const int pre_s = a.ws_pre[s], pre_s1 = a.ws_pre[s + 1], pre_end = a.ws_pre[a.num_seqs];
  const int nb = pre_s1 - pre_s;
  if (nb == 0) return;  // empty or invalid context: its rows come from the attention launch
  const int U = Hkv * pre_end;
  const int C = (U + a.num_workers - 1) / a.num_workers;
  const int us = Hkv * pre_s + g * nb;
  const int w0 = us / C, w1 = (us + nb - 1) / C;
  const bool pfx = a.prefix_blocks > 0;
  if (w0 == w1 && !pfx) return;  // a whole pair: written by the attention launch
  const int64_t prow = (int64_t)(w0 + s * Hkv + g) * G + r;
  merge_row<D>(a.out, a.out_dtype, row, a.ws_ml + prow * 2, (int64_t)G * 2, a.ws_acc + prow * D, (int64_t)G * D,
               w1 - w0 + 1, lane, pfx ? a.ws_pfx_ml + row * 2 : nullptr, pfx ? a.ws_pfx_acc + row * D : nullptr);
}

// ---------------------------------------------------------------- extend (multi-query)
// Sequence s brings n_s new tokens, already in the cache, at positions
// L-n_s .. L-1; query row i of it attends to positions 0 .. L-n_s+i (chunked
// prefill and speculative verification: "Inference serving: the KV-cache
// machine").  The score tile's 16 columns are (query token, head) pairs,
// token-major: a tile holds tpt = 16/G tokens of the group's G heads, a wave
// holds NCT tiles (tpg = NCT*tpt tokens: a "query group"), each column with
// its own online-softmax state and causal limit.  With G > 16 a tile holds
// 16 heads of one token and a query group NCT*16 of that token's heads
// (hparts query groups per token).  Workgroup = (KV head g,
// sequence s, query group, partition of the blocks the group needs); its
// EW waves (four, or eight with four tiles) take every EW-th block, their
// states meet in LDS, and the group writes final rows or (m, l, acc)
// partials for the merge.
struct ExtendArgs {
  void *out;                      // [T][Hq][D]
  const void *q;                  // [T][Hq][D]
  const uint8_t *k_cache;
  const uint8_t *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  const int32_t *query_start;     // [S+1]
  float *ws_ml;                   // [T][Hq][max_parts][2]
  float *ws_acc;                  // [T][Hq][max_parts][D]
  int32_t num_seqs, num_q_heads, num_kv_heads, group, max_blocks, num_blocks, max_ctx, max_q,
      num_rows, max_parts, part_tokens, out_dtype, qgroups, tpt, tpg, hparts;
  float scale_log2;
};

// Score tiles per extend wave: 1, 2 or 4 (four tiles hold 64 (token, head)
// columns: k = 8 drafted tokens at G = 8 read the context once).
constexpr int kExtNctMax = 4;
// Batches of up to this many sequences are dispatched longest context first.
constexpr int kExtRankMax = 256;

// Waves per extend workgroup: eight with four tiles (one workgroup per CU,
// two waves per SIMD), so a long context is streamed by eight waves; four
// otherwise.
template <int NCT>
constexpr int extend_waves() { return NCT >= 4 ? 8 : 4; }

// With four tiles (64 columns) a wave's q fragments live in LDS, not in
// registers (one copy per workgroup: its waves hold the same columns), and
// the waves' states meet a part of the columns at a time (32 at D = 128, in
// the LDS one workgroup per CU leaves; 16 at D = 64).
template <int D, int NCT>
struct __align__(16) SmemExtend {
  static constexpr int EW = extend_waves<NCT>();
  static constexpr bool kTiled = NCT >= 4;
  static constexpr int kCols = kTiled ? (D >= 128 ? 2 : 1) * kTileCols : NCT * kTileCols;  // folded at a time
  float acc[EW][kCols][D + kAccPad];
  float m[EW][kCols];
  float l[EW][kCols];
  u32x4_t q[kTiled ? NCT : 1][kTiled ? D / 32 : 1][64];  // q fragment [tile][c] of each lane
};
// Minimum waves per SIMD the register budget is set for.
template <int NCT>
constexpr int extend_wg_per_cu() { return NCT >= 4 ? 2 : 1; }

// Sequence whose query rows hold row t (query_start ascending).
__device__ inline int seq_of_row(const int32_t *qs, int S, int t) {
  int lo = 0, hi = S;  // qs[lo] <= t < qs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qs[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Rows q0 .. q0+n-1 inside [0, num_rows): otherwise nothing is read or written.
__device__ inline bool extend_rows_valid(int q0, int n, const ExtendArgs &a) {
  return q0 >= 0 && n >= 0 && (int64_t)q0 + n <= a.num_rows;
}

// Contract of one sequence; a violation makes its rows NaN.
__device__ inline bool extend_seq_valid(int L, int n, const ExtendArgs &a) {
  return L >= 0 && L <= a.max_ctx && (int64_t)L <= (int64_t)a.max_blocks * kBS && n <= L && n <= a.max_q;
}

template <int DT, int D, int NCT>
__global__ __launch_bounds__(extend_waves<NCT>() * 64, (extend_wg_per_cu<NCT>())) void pa_extend_kernel(ExtendArgs a) {
  constexpr int EW = extend_waves<NCT>(), ET = EW * 64;
  WaveTrace tr;
  tr.stamp(0);
  using M = MfmaWave<DT, D>;
  using v8 = typename M::v8;
  constexpr int NC = D / 32, NT = D / 16;
  constexpr int NB = 2;  // blocks in flight per wave
  __shared__ SmemExtend<D, NCT> sm;
  const int Hkv = a.num_kv_heads, G = a.group;
  // The query groups of one (sequence, KV head, partition) take grid slots 8
  // apart: workgroups are dealt to the 8 XCDs in turn, so they run together
  // on one XCD and the later groups' block reads are served from its L2.
  const int qg = (int)(blockIdx.x / 8) % a.qgroups;
  const int tg = qg / a.hparts, hp = qg % a.hparts;  // token group, head part
  int rest = (int)(blockIdx.x / 8 / a.qgroups) * 8 + (int)(blockIdx.x % 8);
  if (rest >= (int64_t)Hkv * a.num_seqs * a.max_parts) return;  // padding of the last 8 slots
  const int g = rest % Hkv;
  rest /= Hkv;
  int s = rest % a.num_seqs;
  const int p = rest / a.num_seqs;
  const int tid = threadIdx.x, lane = tid % 64, r = lane % 16, tq = lane / 16;
  const int wu = __builtin_amdgcn_readfirstlane(tid / 64);
  int L, q0, n;
  if (a.num_seqs > 1 && a.num_seqs <= kExtRankMax) {
    // Longest contexts first: workgroups start in index order, so the long
    // (sequence, KV head) pairs take the first round of CUs and the short
    // ones fill the CUs that free up (in sequence order a CU that drew two
    // long pairs ended last).  Slot s of the grid takes the sequence of rank
    // s (longer first, then lower index); which workgroup computes a row
    // does not change its result.  The S x S comparisons are spread over
    // the whole workgroup (tps threads per sequence, each a slice of the
    // others, counted with LDS adds), and the thread that finds rank s
    // passes its sequence's length and query rows on through LDS, so no
    // dependent load of them follows.
    __shared__ int32_t rank_len[kExtRankMax];
    __shared__ int32_t rank_cnt[kExtRankMax];
    __shared__ int32_t rank_qs[kExtRankMax + 1];
    __shared__ int32_t rank_pick[4];
    const int S = a.num_seqs;
    int sp = 1;
    while (sp < S) sp *= 2;
    const int tps = max(1, min(ET / sp, sp)), per = sp / tps;  // threads per sequence, comparisons per thread
    for (int i = tid; i <= S; i += ET) {
      if (i < S) {
        rank_len[i] = a.context_lens[i];
        rank_cnt[i] = 0;
      }
      rank_qs[i] = a.query_start[i];
    }
    __syncthreads();
    for (int t = tid; t < sp * tps; t += ET) {
      const int i = t / tps, j0 = (t % tps) * per;
      if (i >= S) continue;
      const int Li = rank_len[i];
      int rk = 0;
      for (int j = j0; j < min(S, j0 + per); ++j) {
        const int Lj = rank_len[j];
        rk += (Lj > Li || (Lj == Li && j < i)) ? 1 : 0;
      }
      if (rk) atomicAdd(&rank_cnt[i], rk);
    }
    __syncthreads();
    for (int i = tid; i < S; i += ET)
      if (rank_cnt[i] == s) {
        rank_pick[0] = i;
        rank_pick[1] = rank_len[i];
        rank_pick[2] = rank_qs[i];
        rank_pick[3] = rank_qs[i + 1];
      }
    __syncthreads();
    s = rank_pick[0];
    L = rank_pick[1];
    q0 = rank_pick[2];
    n = rank_pick[3] - q0;
  } else {
    L = a.context_lens[s];
    q0 = a.query_start[s];
    n = a.query_start[s + 1] - q0;
  }
  tr.stamp(1);
  const int i0 = tg * a.tpg;
  if (!extend_rows_valid(q0, n, a) || i0 >= n) return;  // no such query group
  const int ni = min(a.tpg, n - i0);
  const int Hq = a.num_q_heads;
  // column (ct, lane row rr): token i0 + col_token of the group's head col_head
  const bool wide = G > kTileCols;
  auto col_token = [&](int ct, int rr) { return wide ? 0 : (rr < a.tpt * G ? ct * a.tpt + rr / G : 1 << 30); };
  auto col_head = [&](int ct, int rr) { return wide ? (hp * NCT + ct) * kTileCols + rr : rr % G; };
  auto col_ok = [&](int ct, int rr) { return col_token(ct, rr) < ni && col_head(ct, rr) < G; };
  if (!extend_seq_valid(L, n, a)) {
    if (p == 0)
      for (int i = tid; i < NCT * kTileCols * D; i += ET) {
        const int col = i / D, d = i % D, ct = col / kTileCols, rr = col % kTileCols;
        if (col_ok(ct, rr))
          store_out(a.out, ((int64_t)(q0 + i0 + col_token(ct, rr)) * Hq + g * G + col_head(ct, rr)) * D + d, NAN,
                    a.out_dtype);
      }
    return;
  }
  const int pf = L - n + i0;       // position of the group's first token
  const int pl = pf + ni - 1;      // and of its last
  const int tok_end = pl + 1;      // the group reads positions 0 .. pl
  const int nparts = (tok_end + a.part_tokens - 1) / a.part_tokens;
  if (p >= nparts) return;
  const int blk0 = (int)((int64_t)p * a.part_tokens / kBS);
  const int tok1 = min(tok_end, (blk0 * kBS) + a.part_tokens);
  const int nblk = (tok1 - blk0 * kBS + kBS - 1) / kBS;
  const int32_t *trow = a.block_tables + (int64_t)s * a.max_blocks + blk0;

  // q fragments and causal limits of this lane's columns
  auto q_row = [&](int ct) {
    const bool ok = col_ok(ct, r);
    const int tk = ok ? col_token(ct, r) : 0, hd = g * G + (ok ? col_head(ct, r) : 0);
    return reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                             ((int64_t)(q0 + i0 + tk) * Hq + hd) * D * 2);
  };
  v8 qB[NCT][NC];
  int lim[NCT];
  f32x4_t acc[NCT][NT];
  float mm[NCT], ll[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const bool ok = col_ok(ct, r);
    lim[ct] = ok ? pf + col_token(ct, r) : -1;
    if constexpr (!SmemExtend<D, NCT>::kTiled) {
      const u32x4_t *qrow = q_row(ct);
#pragma unroll
      for (int c = 0; c < NC; ++c) qB[ct][c] = __builtin_bit_cast(v8, ok ? qrow[4 * c + tq] : u32x4_t{0, 0, 0, 0});
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[ct][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // no score yet: the lowest finite value, so that a block with every
    // score of the column masked (-inf) gives weights 2^(-inf) = 0 and the
    // first finite score always raises the reference
    mm[ct] = -FLT_MAX;
    ll[ct] = 0.f;
  }
  // Four tiles: the waves stage the q fragments in LDS together (fragment
  // f = ct * NC + c by wave f mod EW); a wave loads its share beside its
  // block ids (one memory latency for both) and writes it once its first
  // blocks are requested.  Every wave passes the barrier exactly once.
  constexpr int QF = (NCT * NC + EW - 1) / EW;  // fragments a wave stages
  u32x4_t qst[QF];
  if constexpr (SmemExtend<D, NCT>::kTiled) {
#pragma unroll
    for (int k = 0; k < QF; ++k) {
      const int fi = wu + k * EW, ct = fi / NC, c = fi % NC;
      qst[k] = fi < NCT * NC && col_ok(ct, r) ? q_row(ct)[4 * c + tq] : u32x4_t{0, 0, 0, 0};
    }
  }
  auto stage_q = [&]() {
    if constexpr (SmemExtend<D, NCT>::kTiled) {
#pragma unroll
      for (int k = 0; k < QF; ++k) {
        const int fi = wu + k * EW;
        if (fi < NCT * NC) sm.q[fi / NC][fi % NC][lane] = qst[k];
      }
      lds_barrier();
    }
  };
  // the first position any column of tile ct may not see (wave-uniform)
  int tile_min[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) tile_min[ct] = pf + (wide ? 0 : ct * a.tpt);

  const int64_t head_off = (int64_t)g * M::TILE;
  const int64_t blk_stride = (int64_t)Hkv * M::TILE;
  typename M::Frag fr[NB];
  int bad = 0;
  const int nmine = nblk > wu ? (nblk - wu + EW - 1) / EW : 0;
  if (nmine == 0) stage_q();
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int nc = min(64, nmine - c0);
    int ids = lane < nc ? trow[wu + (c0 + lane) * EW] : 0;
    const bool id_ok = (uint32_t)ids < (uint32_t)a.num_blocks;
    if (__builtin_amdgcn_ballot_w64(!id_ok)) bad = 1;
    ids = id_ok ? ids : 0;
    auto refill = [&](typename M::Frag &f, int i) {
      const bool real = i < nc;
      const int64_t off = real ? (int64_t)__builtin_amdgcn_readlane(ids, min(i, nc - 1)) * blk_stride + head_off : 0;
      M::load(f, a.k_cache + off, a.v_cache + off, real ? lane : 0);
    };
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) {
      refill(fr[b], b);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c0 == 0) stage_q();
    for (int j0 = 0; j0 < nc; j0 += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = j0 + b;
        refill(fr[(b + NB - 1) % NB], i + NB - 1);
        if (i < nc) {
          tr.first();
          // Eight waves share each SIMD two by two and the sequencer favours
          // the older one (waves 0-3 streamed about 1.25x faster than 4-7 in
          // per-wave timestamps, and every workgroup waited for its last
          // four): a wave yields issue priority as it works through its
          // share, so the pair ends together.
          if constexpr (EW == 8) set_wave_priority((nmine - c0 - i) * 4 / (nmine + 1));
          typename M::Frag &f = fr[b];
          const int b0 = (blk0 + wu + (c0 + i) * EW) * kBS;  // position of the block's token 0
          if (b0 + kBS > L) {
            // slots at and past L may hold anything: zero their V elements
            const int lo_ok = L - b0;  // tokens 0 .. lo_ok-1 exist
            const uint32_t mine = token_mask(0, max(0, min(kBS, lo_ok))) >> (4 * tq);
            const uint32_t lo = ((mine & 1u) ? 0x0000FFFFu : 0u) | ((mine & 2u) ? 0xFFFF0000u : 0u);
            const uint32_t hi = ((mine & 4u) ? 0x0000FFFFu : 0u) | ((mine & 8u) ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int c = 0; c < NC; ++c) f.v[c] &= u32x4_t{lo, hi, lo, hi};
          }
          // q fragments from LDS (four tiles) are read again for every block:
          // an opaque zero in the index keeps the compiler from hoisting the
          // reads out of the loop into registers
          int qz = 0;
          if constexpr (SmemExtend<D, NCT>::kTiled) asm volatile("v_mov_b32 %0, 0" : "=v"(qz));
          auto q_frag = [&](int ct, int c) -> v8 {
            if constexpr (SmemExtend<D, NCT>::kTiled)
              return __builtin_bit_cast(v8, sm.q[ct][c][lane + qz]);
            else
              return qB[ct][c];
          };
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) sc = M::mma_qk(__builtin_bit_cast(v8, f.k[c]), q_frag(ct, c), sc);
            float sv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) sv[v] = sc[v] * a.scale_log2;
            if (b0 + kBS - 1 > tile_min[ct]) {  // some column of the tile stops inside this block
#pragma unroll
              for (int v = 0; v < 4; ++v) sv[v] = (b0 + 4 * tq + v <= lim[ct]) ? sv[v] : -INFINITY;
            }
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mx = max_xor32(max_xor16(mx));
            const bool bump = mx > mm[ct] + kLazyLog2;
            if (__builtin_amdgcn_ballot_w64(bump)) {
              const float m_new = bump ? mx : mm[ct];
              const float alpha = exp2_neg(mm[ct] - m_new);  // 0 from -FLT_MAX
              ll[ct] *= alpha;
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[ct][t] *= alpha;
              mm[ct] = m_new;
            }
            float pw[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) pw[v] = __builtin_amdgcn_exp2f(sv[v] - mm[ct]);
            ll[ct] += (pw[0] + pw[1]) + (pw[2] + pw[3]);
            u32x2_t ph, pl2;
            M::split(pw, ph, pl2);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const u32x2_t a0 = u32x2_t{f.v[c][0], f.v[c][1]};
              const u32x2_t a1 = u32x2_t{f.v[c][2], f.v[c][3]};
              acc[ct][2 * c] = M::mma_pv(a0, ph, acc[ct][2 * c]);
              acc[ct][2 * c + 1] = M::mma_pv(a1, ph, acc[ct][2 * c + 1]);
              acc[ct][2 * c] = M::mma_pv(a0, pl2, acc[ct][2 * c]);
              acc[ct][2 * c + 1] = M::mma_pv(a1, pl2, acc[ct][2 * c + 1]);
            }
          }
        }
      }
    }
  }
  tr.stamp(3);
  if (__syncthreads_or(bad)) {
    for (int i = tid; i < NCT * kTileCols * D; i += ET) {
      const int col = i / D, d = i % D, ct = col / kTileCols, rr = col % kTileCols;
      if (!col_ok(ct, rr)) continue;
      const int64_t row = (int64_t)(q0 + i0 + col_token(ct, rr)) * Hq + g * G + col_head(ct, rr);
      if (nparts == 1) {
        store_out(a.out, row * D + d, NAN, a.out_dtype);
      } else {
        const int64_t prow = row * a.max_parts + p;
        a.ws_acc[prow * D + d] = NAN;
        if (d == 0) {
          a.ws_ml[prow * 2] = NAN;
          a.ws_ml[prow * 2 + 1] = NAN;
        }
      }
    }
    return;
  }
  // wave states -> LDS, then fold the waves, FC columns at a time; a wave
  // (or the whole group) that saw no position of a column leaves
  // m = -FLT_MAX, l = 0 for it (weight 0 beside any wave that did)
  constexpr int FC = SmemExtend<D, NCT>::kCols;  // columns per round
  constexpr int FT = FC / kTileCols;             // tiles per round
  constexpr int FG = NCT / FT;                   // fold rounds
#pragma unroll
  for (int fg = 0; fg < FG; ++fg) {
    if (fg > 0) lds_barrier();  // the previous round has read the buffer
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      if (ct / FT != fg) continue;
      const float lt = sum_xor32(sum_xor16(ll[ct]));
      const int col = (ct % FT) * kTileCols + r;
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4_t *>(&sm.acc[wu][col][16 * t + 4 * tq]) = acc[ct][t];
      if (tq == 0) {
        sm.m[wu][col] = mm[ct];
        sm.l[wu][col] = lt;
      }
    }
    lds_barrier();
    // four dims of a row per thread, with the column's wave weights
    // 2^(m_w - M) and denominator computed by each thread
    constexpr int NQ = D / 4;
    for (int i = tid; i < FC * NQ; i += ET) {
      const int cl = i / NQ, d4 = (i % NQ) * 4, colg = fg * FC + cl;
      const int ct = colg / kTileCols, rr = colg % kTileCols;
      if (!col_ok(ct, rr)) continue;
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < EW; ++w) Mx = fmaxf(Mx, sm.m[w][cl]);
      f32x4_t num = {0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < EW; ++w) {
        const float f = exp2f(sm.m[w][cl] - Mx);  // 0 for m = -FLT_MAX beside a real one
        num += f * *reinterpret_cast<const f32x4_t *>(&sm.acc[w][cl][d4]);
        den += f * sm.l[w][cl];
      }
      const int64_t row = (int64_t)(q0 + i0 + col_token(ct, rr)) * Hq + g * G + col_head(ct, rr);
      if (nparts == 1) {
        f32x4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = num[e] / den;
        store_out4(a.out, row * D + d4, v, a.out_dtype);
      } else {
        const int64_t prow = row * a.max_parts + p;
        store_partial4(a.ws_acc + prow * D + d4, num);
        if (d4 == 0) {
          a.ws_ml[prow * 2] = Mx;
          a.ws_ml[prow * 2 + 1] = den;
        }
      }
    }
  }
  tr.write((int64_t)blockIdx.x * EW + wu, lane, (uint64_t)nmine);
}

// One wave per (query row, head) whose group was split: folds its partials.
template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void pa_extend_merge_kernel(ExtendArgs a) {
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / 64;
  if (row >= (int64_t)a.num_rows * a.num_q_heads) return;
  const int t = (int)(row / a.num_q_heads);
  const int s = seq_of_row(a.query_start, a.num_seqs, t);
  const int L = a.context_lens[s];
  const int q0 = a.query_start[s], n = a.query_start[s + 1] - q0;
  if (!extend_rows_valid(q0, n, a) || !extend_seq_valid(L, n, a)) return;
  const int i = t - q0;
  if (i < 0 || i >= n) return;
  const int qg = i / a.tpg;
  const int pl = L - n + min(n, (qg + 1) * a.tpg) - 1;
  const int np = (pl + 1 + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  merge_row<D>(a.out, a.out_dtype, row, a.ws_ml + row * a.max_parts * 2, 2,
               a.ws_acc + row * a.max_parts * D, D, np, lane);
}

// ---------------------------------------------------------------- shared prefix
// Every sequence's table starts with the same prefix_blocks blocks (a shared
// prefix: "Modern AI Infrastructure and Agentic System Design", section 9.1,
// many requests mapping the same prefix blocks; "Inference serving: the
// KV-cache machine", Lab B, the system prompt paid once).  The attention of
// every query row over the prefix is computed once per KV head instead of
// once per sequence: the score tile's 16 columns are (sequence, head) pairs,
// sequence-major (16/G sequences of the G heads; with G > 16, 16 heads of
// one sequence), a wave holds kPfxNct tiles, the four waves of a workgroup take every fourth prefix block and
// meet in LDS, and the (m, l, acc) of each row over the prefix goes to the
// workspace; the balanced split then streams only the blocks after the
// prefix, leaving a partial for every pair, and the merge folds the prefix
// state in as one more partial.
#ifndef PA_PREFIX_NCT
#define PA_PREFIX_NCT 2
#endif
#ifndef PA_PREFIX_RING
#define PA_PREFIX_RING 2
#endif
constexpr int kPfxNct = PA_PREFIX_NCT;  // score tiles per wave

template <int D, int NCT>
struct __align__(16) SmemPrefix {
  float acc[kWaves][NCT * 16][D + kAccPad];
  float m[kWaves][NCT * 16];
  float l[kWaves][NCT * 16];
  float fac[kWaves][NCT * 16];  // each wave's weight in the fold of a column
  float mx[NCT * 16];
  float den[NCT * 16];
};
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void pa_prefix_kernel(DecodeArgs a) {
  using M = MfmaWave<DT, D>;
  using v8 = typename M::v8;
  constexpr int NC = D / 32, NT = D / 16, NCT = kPfxNct;
  constexpr int NB = PA_PREFIX_RING;
  __shared__ SmemPrefix<D, NCT> sm;
  const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
  const int g = blockIdx.x % Hkv;
  const int sg = blockIdx.x / Hkv;
  const int tid = threadIdx.x, lane = tid % 64, r = lane % 16, tq = lane / 16;
  const int wu = __builtin_amdgcn_readfirstlane(tid / 64);
  // Columns: with G <= 16 a tile holds tpt = 16/G whole sequences; with
  // G > 16 a tile holds 16 heads of one sequence and a workgroup's NCT tiles
  // cover NCT*16 of its heads (hparts workgroups per sequence).
  const bool wide = G > kTileCols;
  const int tpt = wide ? 1 : kTileCols / G;
  const int hparts = wide ? (G + NCT * kTileCols - 1) / (NCT * kTileCols) : 1;
  const int spg = wide ? 1 : NCT * tpt;  // sequences per workgroup
  const int s0 = (sg / hparts) * spg, hp = sg % hparts;
  const int ns = min(spg, a.num_seqs - s0);
  if (ns <= 0) return;
  // column (ct, lane row r): sequence s0 + col_seq, head col_head of the group
  auto col_seq = [&](int ct, int rr) { return wide ? 0 : (rr < tpt * G ? ct * tpt + rr / G : 1 << 30); };
  auto col_head = [&](int ct, int rr) { return wide ? (hp * NCT + ct) * kTileCols + rr : rr % G; };
  auto col_ok = [&](int ct, int rr) { return col_seq(ct, rr) < ns && col_head(ct, rr) < G; };
  v8 qB[NCT][NC];
  f32x4_t acc[NCT][NT];
  float mm[NCT], ll[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const bool ok = col_ok(ct, r);
    const int sk = ok ? col_seq(ct, r) : 0, hd = g * G + (ok ? col_head(ct, r) : 0);
    const u32x4_t *qrow = reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                                            ((int64_t)(s0 + sk) * Hq + hd) * D * 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4_t x = qrow[4 * c + tq];
      if (!ok) x = u32x4_t{0, 0, 0, 0};
      qB[ct][c] = __builtin_bit_cast(v8, x);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[ct][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    mm[ct] = -INFINITY;
    ll[ct] = 0.f;
  }
  const int nblk = a.prefix_blocks;
  const int64_t head_off = (int64_t)g * M::TILE;
  const int64_t blk_stride = (int64_t)Hkv * M::TILE;
  typename M::Frag fr[NB];
  int bad = 0;
  const int nmine = nblk > wu ? (nblk - wu + kWaves - 1) / kWaves : 0;
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int nc = min(64, nmine - c0);
    int ids = lane < nc ? a.block_tables[wu + (c0 + lane) * kWaves] : 0;  // sequence 0's row
    const bool id_ok = (uint32_t)ids < (uint32_t)a.num_blocks;
    if (__builtin_amdgcn_ballot_w64(!id_ok)) bad = 1;
    ids = id_ok ? ids : 0;
    auto refill = [&](typename M::Frag &f, int i) {
      const bool real = i < nc;
      const int64_t off = real ? (int64_t)__builtin_amdgcn_readlane(ids, min(i, nc - 1)) * blk_stride + head_off : 0;
      M::load(f, a.k_cache + off, a.v_cache + off, real ? lane : 0);
    };
#pragma unroll
    for (int b = 0; b < NB - 1; ++b) {
      refill(fr[b], b);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int j0 = 0; j0 < nc; j0 += NB) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int i = j0 + b;
        refill(fr[(b + NB - 1) % NB], i + NB - 1);
        if (i < nc) {
          typename M::Frag &f = fr[b];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) sc = M::mma_qk(__builtin_bit_cast(v8, f.k[c]), qB[ct][c], sc);
            float sv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) sv[v] = sc[v] * a.scale_log2;
            float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
            mx = max_xor32(max_xor16(mx));
            const bool bump = mx > mm[ct] + kLazyLog2;
            if (__builtin_amdgcn_ballot_w64(bump)) {
              const float m_new = bump ? mx : mm[ct];
              const float alpha = mm[ct] == -INFINITY ? 0.f : exp2_neg(mm[ct] - m_new);
              ll[ct] *= alpha;
#pragma unroll
              for (int t = 0; t < NT; ++t) acc[ct][t] *= alpha;
              mm[ct] = m_new;
            }
            float pw[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) pw[v] = __builtin_amdgcn_exp2f(sv[v] - mm[ct]);
            ll[ct] += (pw[0] + pw[1]) + (pw[2] + pw[3]);
            u32x2_t ph, pl2;
            M::split(pw, ph, pl2);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const u32x2_t a0 = u32x2_t{f.v[c][0], f.v[c][1]};
              const u32x2_t a1 = u32x2_t{f.v[c][2], f.v[c][3]};
              acc[ct][2 * c] = M::mma_pv(a0, ph, acc[ct][2 * c]);
              acc[ct][2 * c + 1] = M::mma_pv(a1, ph, acc[ct][2 * c + 1]);
              acc[ct][2 * c] = M::mma_pv(a0, pl2, acc[ct][2 * c]);
              acc[ct][2 * c + 1] = M::mma_pv(a1, pl2, acc[ct][2 * c + 1]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float lt = sum_xor32(sum_xor16(ll[ct]));
    const int col = ct * 16 + r;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4_t *>(&sm.acc[wu][col][16 * t + 4 * tq]) = acc[ct][t];
    if (tq == 0) {
      sm.m[wu][col] = mm[ct];
      sm.l[wu][col] = lt;
    }
  }
  const bool any_bad = __syncthreads_or(bad);
  // Fold the four waves' states: one weight per (wave, column) first, then
  // four floats of a row per thread.
  if (tid < NCT * 16) {
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, sm.m[w][tid]);
    float den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = Mx == -INFINITY ? 0.f : exp2f(sm.m[w][tid] - Mx);
      sm.fac[w][tid] = f;
      den += f * sm.l[w][tid];
    }
    sm.mx[tid] = Mx;
    sm.den[tid] = den;
  }
  lds_barrier();
  constexpr int NQ = D / 4;
  const f32x4_t nan4 = {NAN, NAN, NAN, NAN};
  for (int i = tid; i < NCT * kTileCols * NQ; i += kThreads) {
    const int col = i / NQ, d4 = (i % NQ) * 4;
    if (!col_ok(col / kTileCols, col % kTileCols)) continue;
    const int sk = col_seq(col / kTileCols, col % kTileCols), h = col_head(col / kTileCols, col % kTileCols);
    f32x4_t num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) num += sm.fac[w][col] * *reinterpret_cast<const f32x4_t *>(&sm.acc[w][col][d4]);
    const int64_t row = (int64_t)(s0 + sk) * Hq + g * G + h;
    *reinterpret_cast<f32x4_t *>(a.ws_pfx_acc + row * D + d4) = any_bad ? nan4 : num;
    if (d4 == 0) {
      a.ws_pfx_ml[row * 2] = any_bad ? NAN : sm.mx[col];
      a.ws_pfx_ml[row * 2 + 1] = sm.den[col];
    }
  }
}

// ---------------------------------------------------------------- KV append
// One thread per (token, kv head, X-dim chunk): reads X elements (16 bytes)
// of the new K and V rows and writes them at the slot's place in the tiles.
template <int EB, int D>
__global__ __launch_bounds__(256) void pa_reshape_and_cache_kernel(
    const uint8_t *__restrict__ k_new, const uint8_t *__restrict__ v_new, uint8_t *k_cache,
    uint8_t *v_cache, const int64_t *__restrict__ slots, int32_t num_tokens, int32_t num_kv_heads,
    int64_t num_slots) {
  constexpr int X = 16 / EB;
  constexpr int CH = D / X;  // chunks per row
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)num_tokens * num_kv_heads * CH) return;
  const int c = idx % CH;
  const int64_t row = idx / CH;  // token * Hkv + head
  const int g = row % num_kv_heads;
  const int64_t n = row / num_kv_heads;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / kBS;
  const int t = slot % kBS;
  const int64_t tile = (blk * num_kv_heads + g) * kBS * D;  // element offset
  const u32x4_t kx = reinterpret_cast<const u32x4_t *>(k_new + (row * D + c * X) * EB)[0];
  const u32x4_t vx = reinterpret_cast<const u32x4_t *>(v_new + (row * D + c * X) * EB)[0];
  // K tile [D/X][16][X]: the chunk's X dims are contiguous.
  reinterpret_cast<u32x4_t *>(k_cache + (tile + (int64_t)c * kBS * X + t * X) * EB)[0] = kx;
  // V tile: element (t, d) at (d/(4X))*64X + ((t/4)*16 + (d%4X)%16)*X + ((d%4X)/16)*4 + t%4.
#pragma unroll
  for (int e = 0; e < X; ++e) {
    const int d = c * X + e;
    const int slab = d / (4 * X), de = d % (4 * X);
    const int64_t off = tile + (int64_t)slab * 64 * X + ((t / 4) * 16 + de % 16) * X + (de / 16) * 4 + t % 4;
    if constexpr (EB == 4) {
      reinterpret_cast<uint32_t *>(v_cache)[off] = vx[e];
    } else {
      const uint32_t wrd = vx[e / 2];
      reinterpret_cast<uint16_t *>(v_cache)[off] = (uint16_t)((e & 1) ? (wrd >> 16) : (wrd & 0xFFFFu));
    }
  }
}

// ---------------------------------------------------------------- INT8 / FP8 append
// (quantizer helpers: with the byte-code wave policy above)
// One row into its tile: the codes at their places, the scale after the
// tile's codes (byte 16*D + 4t).
template <int SDT, int D, int FMT>
__device__ void quantize_row_i8(const uint16_t *x, int8_t *tile, int t, bool is_v, int lane) {
  constexpr int PER = D / 64;
  float v[PER];
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    v[e] = half_value<SDT>(x[lane * PER + e]);
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float scale = code_scale<FMT>(amax);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = lane * PER + e;
    tile[is_v ? v_code_off(d, t) : k_code_off(d, t)] = (int8_t)code_of<FMT>(v[e], scale);
  }
  if (lane == 0) reinterpret_cast<float *>(tile + kBS * D)[t] = scale;
}

template <int SDT, int D, int FMT>
__global__ __launch_bounds__(256) void pa_reshape_and_cache_i8_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new, int8_t *k_cache, int8_t *v_cache,
    const int64_t *__restrict__ slots, int32_t num_tokens, int32_t num_kv_heads, int64_t num_slots) {
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;  // token * Hkv + head
  if (row >= (int64_t)num_tokens * num_kv_heads) return;
  const int g = (int)(row % num_kv_heads);
  const int64_t n = row / num_kv_heads;
  const int64_t slot = slots[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t tile = (slot / kBS) * num_kv_heads + g;
  const int t = (int)(slot % kBS);
  constexpr int64_t kTileBytes = kBS * (D + 4);  // codes, then the 16 row scales
  quantize_row_i8<SDT, D, FMT>(k_new + row * D, k_cache + tile * kTileBytes, t, false, lane);
  quantize_row_i8<SDT, D, FMT>(v_new + row * D, v_cache + tile * kTileBytes, t, true, lane);
}

// ---------------------------------------------------------------- block copy
// grid.x = pair; each thread moves 16-byte vectors of the whole block (K and V).
__global__ __launch_bounds__(256) void pa_copy_blocks_kernel(uint8_t *k_cache, uint8_t *v_cache,
                                                             const int32_t *__restrict__ pairs,
                                                             int64_t block_bytes, int32_t num_blocks) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t nvec = block_bytes / 16;
  const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(k_cache + src * block_bytes);
  const u32x4_t *vs = reinterpret_cast<const u32x4_t *>(v_cache + src * block_bytes);
  u32x4_t *kd = reinterpret_cast<u32x4_t *>(k_cache + dst * block_bytes);
  u32x4_t *vd = reinterpret_cast<u32x4_t *>(v_cache + dst * block_bytes);
  for (int64_t i = threadIdx.x; i < nvec; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// ---------------------------------------------------------------- swap copies
// Block copies between two pools of the same tile layout, either of which
// may be pinned host memory (preemption by swapping: "Inference serving: the
// KV-cache machine", section "Paged KV").  Grid: (pair, chunk); a chunk is
// kSwapVecs 16-byte vectors of the pair's K tile followed by its V tile, and
// every thread has kSwapUnroll loads in flight before it stores (host memory
// is far away).
constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 4;
constexpr int kSwapVecs = kSwapThreads * kSwapUnroll;

__global__ __launch_bounds__(kSwapThreads) void pa_swap_blocks_kernel(
    const uint8_t *src_k, const uint8_t *src_v, int32_t src_nb, uint8_t *dst_k, uint8_t *dst_v,
    int32_t dst_nb, const int32_t *__restrict__ pairs, int64_t block_bytes) {
  const int32_t src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_nb || dst < 0 || dst >= dst_nb) return;
  const int64_t nvec = block_bytes / 16;  // per tile (K or V)
  const int64_t v0 = (int64_t)blockIdx.y * kSwapVecs + threadIdx.x;
  u32x4_t x[kSwapUnroll];
#pragma unroll
  for (int k = 0; k < kSwapUnroll; ++k) {
    const int64_t v = v0 + k * kSwapThreads;
    if (v < 2 * nvec) {
      const uint8_t *base = v < nvec ? src_k : src_v;
      x[k] = reinterpret_cast<const u32x4_t *>(base + src * block_bytes)[v < nvec ? v : v - nvec];
    }
  }
#pragma unroll
  for (int k = 0; k < kSwapUnroll; ++k) {
    const int64_t v = v0 + k * kSwapThreads;
    if (v < 2 * nvec) {
      uint8_t *base = v < nvec ? dst_k : dst_v;
      reinterpret_cast<u32x4_t *>(base + dst * block_bytes)[v < nvec ? v : v - nvec] = x[k];
    }
  }
}

// ============================================================================
// Host side
// ============================================================================
int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }
bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
bool byte_cache(pa_dtype d) { return d == PA_I8 || d == PA_FP8; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

pa_status validate(const pa_decode_params *p) {
  if (!p) return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: params is NULL");
  // An array with no elements (no sequences; no table columns) may be NULL.
  const bool rows = p->num_seqs > 0, cols = rows && p->max_blocks_per_seq > 0;
  if ((rows && (!p->out || !p->q || !p->context_lens)) || (cols && !p->block_tables) || !p->k_cache ||
      !p->v_cache)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: NULL device pointer");
  if (!aligned16(p->out) || !aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->v_cache) ||
      !aligned16(p->block_tables) || !aligned16(p->context_lens))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: device pointers must be 16-byte aligned");
  if (p->num_seqs < 0 || p->num_seqs > 65535)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: num_seqs must be in [0, 65535]");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: num_q_heads must be a positive multiple of num_kv_heads");
  if (p->num_kv_heads > 65535)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: num_kv_heads must be <= 65535");
  if (p->num_q_heads / p->num_kv_heads > kGMax)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: at most %d query heads per KV head", kGMax);
  if (p->head_dim != 64 && p->head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim must be 64 or 128");
  if (p->max_blocks_per_seq < 0 || p->num_blocks <= 0 || p->max_context_len < 0)
    return pa::fail(PA_ERR_INVALID_ARG,
                    "pa_decode: num_blocks must be positive, max_blocks_per_seq and max_context_len >= 0");
  if (!(valid_dtype(p->kv_dtype) || byte_cache(p->kv_dtype)) || !valid_dtype(p->out_dtype))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: unknown dtype");
  if (byte_cache(p->kv_dtype)) {
    if (p->q_dtype != PA_F16 && p->q_dtype != PA_BF16)
      return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: an INT8/FP8 cache needs q_dtype F16 or BF16");
    if (p->out_dtype != PA_F32 && p->out_dtype != p->q_dtype)
      return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: out_dtype must be F32 or q_dtype");
    if (p->kernel == PA_KERNEL_VALU || p->partition_tokens > 0)
      return pa::fail(PA_ERR_UNSUPPORTED,
                      "pa_decode: an INT8/FP8 cache is decoded by the matrix-core kernel with automatic "
                      "partitioning");
  } else if (p->out_dtype != PA_F32 && p->out_dtype != p->kv_dtype) {
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: out_dtype must be F32 or the cache type");
  }
  if (p->partition_tokens < PA_PARTITION_BALANCED || (p->partition_tokens > 0 && p->partition_tokens % kBS))
    return pa::fail(PA_ERR_INVALID_ARG,
                    "pa_decode: partition_tokens must be 0 (automatic), PA_PARTITION_BALANCED (-1) or a "
                    "positive multiple of 16");
  if (p->kernel != PA_KERNEL_AUTO && p->kernel != PA_KERNEL_VALU && p->kernel != PA_KERNEL_MFMA)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: unknown kernel");
  if (p->kernel == PA_KERNEL_MFMA && p->kv_dtype == PA_F32)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: the MFMA kernel needs an fp16 or bf16 cache");
  if ((p->k_new != nullptr) != (p->v_new != nullptr) || (p->k_new != nullptr) != (p->slot_mapping != nullptr))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: k_new, v_new and slot_mapping go together");
  if (p->k_new && (!aligned16(p->k_new) || !aligned16(p->v_new) || !aligned16(p->slot_mapping)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: device pointers must be 16-byte aligned");
  if (!(std::isfinite(p->scale)))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: scale must be finite");
  if (p->sliding_window < 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: sliding_window must be >= 0 (0 = none)");
  if (p->shared_prefix_blocks < 0 || p->shared_prefix_blocks > p->max_blocks_per_seq)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: shared_prefix_blocks must be in [0, max_blocks_per_seq]");
  if (p->shared_prefix_blocks > 0 &&
      ((p->kv_dtype != PA_F16 && p->kv_dtype != PA_BF16) || p->sliding_window != 0 ||
       p->partition_tokens > 0 || p->kernel == PA_KERNEL_VALU))
    return pa::fail(PA_ERR_UNSUPPORTED,
                    "pa_decode: a shared prefix needs an fp16/bf16 cache, no sliding window and the "
                    "matrix-core kernel with automatic partitioning");
  return PA_OK;
}

bool use_balanced(const pa_decode_params *p);

// validate() plus the checks that depend on the chosen split.
pa_status validate_all(const pa_decode_params *p) {
  pa_status st = validate(p);
  if (st != PA_OK) return st;
  if ((byte_cache(p->kv_dtype) || p->shared_prefix_blocks > 0 || p->partition_tokens == PA_PARTITION_BALANCED) &&
      !use_balanced(p))
    return pa::fail(PA_ERR_UNSUPPORTED,
                    "pa_decode: INT8/FP8 caches, a shared prefix and PA_PARTITION_BALANCED need the balanced "
                    "split (the matrix-core kernel, <= 1024 sequences, <= 32768 (sequence, KV head) pairs)");
  return PA_OK;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Automatic partition size: the largest of 1024 / 512 / 256 tokens whose grid
// still has >= 8 workgroups per CU (shorter partitions balance better but add
// merge work); a context that fits one such partition is not split.
bool balanced_fits(const pa_decode_params *p);

int32_t resolve_partition(const pa_decode_params *p) {
  if (p->partition_tokens > 0) return p->partition_tokens;
  const int32_t ctx = ((std::max(p->max_context_len, 1) + kBS - 1) / kBS) * kBS;
  // A small batch on the matrix-core path (one the balanced split could run
  // but leaves to partitions): about one workgroup per CU.  With at least as
  // many (sequence, KV head) pairs as CUs every pair is one partition and no
  // merge runs (7B MHA batch: 47.5 us per step against 50.5 with 512-token
  // partitions); fewer pairs cut each attended range into CUs / pairs pieces.
  if (balanced_fits(p)) {
    int64_t span = ctx;  // tokens a pair's partitions cover at most
    if (p->sliding_window > 0) span = std::min<int64_t>(span, (int64_t)p->sliding_window + kBS);
    const int64_t pairs = std::max<int64_t>(1, (int64_t)p->num_seqs * p->num_kv_heads);
    const int64_t pieces = std::max<int64_t>(1, (cu_count() + pairs - 1) / pairs);
    const int64_t t = (span + pieces - 1) / pieces;
    return (int32_t)std::min<int64_t>(ctx, (t + kBS - 1) / kBS * kBS);
  }
  const int64_t pairs = (int64_t)p->num_seqs * p->num_kv_heads;
  const int64_t target = 8LL * cu_count();
  int32_t pt = 256;
  for (int32_t cand : {1024, 512}) {
    if (pairs * ((ctx + cand - 1) / cand) >= target) {
      pt = cand;
      break;
    }
  }
  return ctx <= pt ? ctx : pt;
}

bool use_mfma(const pa_decode_params *p) {
  return p->kernel == PA_KERNEL_MFMA || (p->kernel == PA_KERNEL_AUTO && p->kv_dtype != PA_F32);
}

// Partition workgroups per (partition, KV head, sequence): the vector-ALU
// kernel takes at most 16 heads per workgroup, the matrix-core kernel all G.
int head_chunks(const pa_decode_params *p) {
  const int G = p->num_q_heads / p->num_kv_heads;
  return use_mfma(p) ? 1 : (G + kTileCols - 1) / kTileCols;
}

// Shared-prefix workgroups per KV head for S sequences of G query heads:
// kPfxNct score tiles each, a tile holding 16/G whole sequences (G <= 16) or
// 16 heads of one sequence.
int prefix_workgroups(int S, int G) {
  if (G > kTileCols) return S * ((G + kPfxNct * kTileCols - 1) / (kPfxNct * kTileCols));
  const int spg = kPfxNct * (kTileCols / G);
  return (S + spg - 1) / spg;
}

// Matrix-core column tiles for G query heads per KV head: ceil(G / 16),
// rounded up to 1, 2 or 4 (the instantiated kernels).
int nct_of(int G) { return G <= kTileCols ? 1 : G <= 2 * kTileCols ? 2 : 4; }

// Parking slots per wave: as many as the LDS left beside the kernel's own
// shared memory allows (per workgroup, with wg_per_cu workgroups on a CU),
// at most kParkSlotsMax; none when a slot does not fit (every segment then
// stores as it ends).
int park_slots(int G, int D, int wg_per_cu, int64_t reserve = 0) {
  static int lds_block[64] = {}, lds_cu[64] = {};
  int dev = 0, per_block = 64 * 1024, per_cu = 64 * 1024;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    if (!lds_block[dev]) {
      int b = 0, c = 0;
      if (hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
          hipDeviceGetAttribute(&c, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
          b <= 0 || c <= 0) {
        (void)hipGetLastError();
        b = c = 64 * 1024;
      }
      lds_cu[dev] = c;
      lds_block[dev] = b;
    }
    per_block = lds_block[dev];
    per_cu = lds_cu[dev];
  } else {
    (void)hipGetLastError();
  }
  const int64_t budget = std::min<int64_t>(per_block, per_cu / std::max(wg_per_cu, 1) - reserve) -
                         (int64_t)sizeof(SmemBalanced) - 2048;
  const int64_t slot = (int64_t)kBWaves * park_slot_floats(G, D) * sizeof(float);
  return (int)std::max<int64_t>(0, std::min<int64_t>(kParkSlotsMax, budget / slot));
}

size_t park_bytes(int G, int D, int slots) {
  return (size_t)kBWaves * slots * park_slot_floats(G, D) * sizeof(float);
}

// The balanced kernel for a cache type, q type, head size and group size,
// with the workgroups per CU it is built for.
struct BalancedKernel {
  const void *fn;
  int wg_per_cu;
};

template <class W, int D>
BalancedKernel kinfo() {
  return {reinterpret_cast<const void *>(&pa_balanced_kernel<W, D>), W::kBalWgPerCu};
}

template <int NCT>
BalancedKernel balanced_kernel_nct(pa_dtype kv, pa_dtype qt, int D) {
  if (kv == PA_I8) {
    if (qt == PA_BF16)
      return D == 128 ? kinfo<MfmaWaveI8<PA_BF16, 128, PA_I8, NCT>, 128>() : kinfo<MfmaWaveI8<PA_BF16, 64, PA_I8, NCT>, 64>();
    return D == 128 ? kinfo<MfmaWaveI8<PA_F16, 128, PA_I8, NCT>, 128>() : kinfo<MfmaWaveI8<PA_F16, 64, PA_I8, NCT>, 64>();
  }
  if (kv == PA_FP8) {
    if (qt == PA_BF16)
      return D == 128 ? kinfo<MfmaWaveI8<PA_BF16, 128, PA_FP8, NCT>, 128>()
                      : kinfo<MfmaWaveI8<PA_BF16, 64, PA_FP8, NCT>, 64>();
    return D == 128 ? kinfo<MfmaWaveI8<PA_F16, 128, PA_FP8, NCT>, 128>() : kinfo<MfmaWaveI8<PA_F16, 64, PA_FP8, NCT>, 64>();
  }
  if (kv == PA_BF16)
    return D == 128 ? kinfo<MfmaWave<PA_BF16, 128, NCT>, 128>() : kinfo<MfmaWave<PA_BF16, 64, NCT>, 64>();
  return D == 128 ? kinfo<MfmaWave<PA_F16, 128, NCT>, 128>() : kinfo<MfmaWave<PA_F16, 64, NCT>, 64>();
}

BalancedKernel balanced_kernel(pa_dtype kv, pa_dtype qt, int D, int G) {
  switch (nct_of(G)) {
    case 1: return balanced_kernel_nct<1>(kv, qt, D);
    case 2: return balanced_kernel_nct<2>(kv, qt, D);
    default: return balanced_kernel_nct<4>(kv, qt, D);
  }
}

// LDS of one shared-prefix workgroup, which runs beside the balanced split.
int64_t prefix_lds(int D) {
  return D == 128 ? (int64_t)sizeof(SmemPrefix<128, kPfxNct>) : (int64_t)sizeof(SmemPrefix<64, kPfxNct>);
}

// Parking slots of the balanced kernel; with a shared prefix, room is left
// on each CU for one prefix workgroup.
int balanced_park_slots(pa_dtype kv, pa_dtype qt, int G, int D, bool prefix = false) {
  return park_slots(G, D, balanced_kernel(kv, qt, D, G).wg_per_cu, prefix ? prefix_lds(D) : 0);
}

// Workgroups of the balanced grid: the kernel's workgroups per CU (checked
// against its occupancy with its parking LDS for G query heads per KV head
// where a device answers).
int balanced_workgroups(pa_dtype kv, pa_dtype qt, int D, int G) {
  static int cached[64][12][kGMax + 1] = {};
  int dev = 0;
  const bool bytes = byte_cache(kv);
  const BalancedKernel bk = balanced_kernel(kv, qt, D, G);
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return bk.wg_per_cu * cu_count();
  const int k = (kv == PA_I8 ? 4 : kv == PA_FP8 ? 8 : 0) + ((bytes ? qt : kv) == PA_BF16 ? 0 : 2) + (D == 128 ? 0 : 1);
  if (!cached[dev][k][G]) {
    const int want = bk.wg_per_cu;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bk.fn, kBThreads,
                                                     park_bytes(G, D, balanced_park_slots(kv, qt, G, D))) !=
            hipSuccess ||
        per_cu <= 0)
      per_cu = want;
    cached[dev][k][G] = std::min(per_cu, want) * cu_count();
  }
  return cached[dev][k][G];
}

int balanced_workgroups(const pa_decode_params *p) {
  return balanced_workgroups(p->kv_dtype, p->q_dtype, p->head_dim, p->num_q_heads / p->num_kv_heads);
}

// Automatic partitioning on the matrix-core path uses the balanced split
// when the batch fits its LDS tables and its unit counts fit 32 bits.
// Most units (sequence, KV head, attended block) the batch can hold.
int64_t max_units(const pa_decode_params *p) {
  int64_t blocks = (std::max(p->max_context_len, 0) + kBS - 1) / kBS;
  if (p->sliding_window > 0)  // W + 1 attended tokens span at most this many blocks
    blocks = std::min<int64_t>(blocks, (p->sliding_window + kBS) / kBS + 1);
  return (int64_t)p->num_kv_heads * p->num_seqs * blocks;
}

// Below this many units per wave at the longest context, automatic
// partitioning on a 16-bit cache uses partitions: wave shares that short
// spend most of their time in the launch's fixed latency chain (lengths,
// tables, first tiles) and leave many partials to merge, while a partition
// grid keeps several waves per SIMD streaming.  Measured: 7B MHA (8 x 2048
// tokens, ~36 units per wave) 46.6 us with 512-token partitions vs 50.1
// balanced; the 8-way head and context shares of the 70B and long-context
// batches (17 and 8 units per wave) 19.2 / 16.3 us vs 21.8 / 20.0; at 64
// (sliding window) and 135 (70B batch) units per wave the balanced split is
// as fast or faster.
constexpr int64_t kBalancedMinUnitsPerWave = 48;

// The balanced split can run this batch.
bool balanced_fits(const pa_decode_params *p) {
  if (p->partition_tokens > 0 || !use_mfma(p) || p->num_seqs < 1 || p->num_seqs > kSeqMax) return false;
  if ((int64_t)p->num_seqs * p->num_kv_heads > kPairMax) return false;
  if ((int64_t)p->num_blocks * p->num_kv_heads > UINT32_MAX) return false;
  const int64_t units = (int64_t)p->num_kv_heads * p->num_seqs * ((std::max(p->max_context_len, 0) + kBS - 1) / kBS);
  return units + (int64_t)kBWaves * balanced_workgroups(p) < INT32_MAX;
}

bool use_balanced(const pa_decode_params *p) {
  if (!balanced_fits(p)) return false;
  if (p->partition_tokens == PA_PARTITION_BALANCED || byte_cache(p->kv_dtype) || p->shared_prefix_blocks > 0)
    return true;
  // A sliding window caps what each pair attends, so with a pair for every CU
  // one partition per pair is even work and needs no merge (Mistral-shaped
  // batch, 256 pairs under W = 4096: 91 us per step against 97.6 balanced).
  if (p->sliding_window > 0 && (int64_t)p->num_seqs * p->num_kv_heads >= cu_count()) return false;
  return max_units(p) >= kBalancedMinUnitsPerWave * kBWaves * balanced_workgroups(p);
}

size_t round16(size_t x) { return (x + 15) / 16 * 16; }

// Balanced-split workspace: [S+1] int32 block offsets, then per slot
// (NW + S*Hkv - 1 of them) G rows of (m, l) and G rows of D accumulators,
// then with a shared prefix every row's (m, l) and acc over it.
size_t balanced_bytes(const pa_decode_params *p, size_t *ml_off, size_t *acc_off, size_t *pfx_off = nullptr) {
  const int64_t nw = (int64_t)kBWaves * balanced_workgroups(p);
  const int64_t slots = nw + (int64_t)p->num_seqs * p->num_kv_heads - 1;
  const int64_t G = p->num_q_heads / p->num_kv_heads;
  const size_t pre = round16(((size_t)p->num_seqs + 1) * 4);
  const size_t ml = round16((size_t)slots * G * 2 * 4);
  if (ml_off) *ml_off = pre;
  if (acc_off) *acc_off = pre + ml;
  const size_t base = pre + ml + round16((size_t)slots * G * p->head_dim * 4);
  if (pfx_off) *pfx_off = base;
  if (p->shared_prefix_blocks <= 0) return base;
  const size_t rows = (size_t)p->num_seqs * p->num_q_heads;
  return base + round16(rows * 2 * 4) + rows * p->head_dim * 4;
}

size_t partial_bytes(const pa_decode_params *p, int32_t np) {
  return (size_t)p->num_seqs * p->num_q_heads * np * (p->head_dim + 2) * sizeof(float);
}


// Partitions per (sequence, KV head): they cover the attended range from its
// first block, at most W + 16 tokens under a sliding window of W.
int32_t num_partitions(const pa_decode_params *p, int32_t pt) {
  int64_t span = std::max(p->max_context_len, 1);
  if (p->sliding_window > 0) span = std::min<int64_t>(span, (int64_t)p->sliding_window + kBS);
  return (int32_t)std::max<int64_t>(1, (span + pt - 1) / pt);
}

// Optional start/stop events of a launch, taken from the dispatch itself.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// One kernel launch: through hipExtLaunchKernel when events are attached, so
// they carry the dispatch's own timestamps and add no stream marker.
hipError_t launch_kernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds, hipStream_t hs,
                         const LaunchEvents &ev) {
  if (ev.start || ev.stop) return hipExtLaunchKernel(fn, grid, block, args, lds, hs, ev.start, ev.stop, 0);
  return hipLaunchKernel(fn, grid, block, args, lds, hs);
}

// Records the events of a call that launches no kernel.
pa_status record_events(const LaunchEvents &ev, hipStream_t hs, const char *who) {
  if (ev.start) {
    const hipError_t e = hipEventRecord(ev.start, hs);
    if (e != hipSuccess) return hip_check(e, who);
  }
  if (ev.stop) {
    const hipError_t e = hipEventRecord(ev.stop, hs);
    if (e != hipSuccess) return hip_check(e, who);
  }
  return PA_OK;
}

template <int DT, int D>
const void *valu_kernel(int G) {
  if (G <= 1) return reinterpret_cast<const void *>(&pa_partition_kernel<ValuWave<DT, D, 1>, D, false>);
  if (G <= 2) return reinterpret_cast<const void *>(&pa_partition_kernel<ValuWave<DT, D, 2>, D, false>);
  if (G <= 4) return reinterpret_cast<const void *>(&pa_partition_kernel<ValuWave<DT, D, 4>, D, false>);
  if (G <= 8) return reinterpret_cast<const void *>(&pa_partition_kernel<ValuWave<DT, D, 8>, D, false>);
  return reinterpret_cast<const void *>(&pa_partition_kernel<ValuWave<DT, D, 16>, D, false>);
}

template <int DT, int D>
const void *mfma_partition_kernel(int G) {
  switch (nct_of(G)) {
    case 1: return reinterpret_cast<const void *>(&pa_partition_kernel<MfmaWave<DT, D, 1>, D, true>);
    case 2: return reinterpret_cast<const void *>(&pa_partition_kernel<MfmaWave<DT, D, 2>, D, true>);
    default: return reinterpret_cast<const void *>(&pa_partition_kernel<MfmaWave<DT, D, 4>, D, true>);
  }
}

template <int D>
const void *partition_kernel(pa_dtype dt, bool mfma, int G) {
  if (mfma) return dt == PA_BF16 ? mfma_partition_kernel<PA_BF16, D>(G) : mfma_partition_kernel<PA_F16, D>(G);
  if (dt == PA_BF16) return valu_kernel<PA_BF16, D>(G);
  if (dt == PA_F16) return valu_kernel<PA_F16, D>(G);
  return valu_kernel<PA_F32, D>(G);
}

}  // namespace

extern "C" {

int32_t pa_decode_partition_tokens(const pa_decode_params *p) {
  pa_status st = validate_all(p);
  if (st != PA_OK) return -(int32_t)st;
  if (use_balanced(p)) return 0;
  return resolve_partition(p);
}

size_t pa_decode_workspace_bytes(const pa_decode_params *p) {
  if (validate_all(p) != PA_OK) return 0;
  if (use_balanced(p)) return balanced_bytes(p, nullptr, nullptr);
  const int32_t pt = resolve_partition(p);
  const int32_t np = num_partitions(p, pt);
  if (np <= 1) return 0;
  return partial_bytes(p, np);
}

}  // extern "C"

namespace {

// Validates, checks the workspace and fills the kernel arguments.
pa_status prepare(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                  const char *who, DecodeArgs &a) {
  pa_status st = validate_all(p);
  if (st != PA_OK) return st;
  const bool bal = use_balanced(p);
  const int32_t pt = bal ? 0 : resolve_partition(p);
  const int32_t np = bal ? 1 : num_partitions(p, pt);
  if ((int64_t)np * p->num_kv_heads * p->num_seqs * head_chunks(p) > INT32_MAX)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: more than 2^31-1 workgroups (raise partition_tokens)", who);
  const size_t need = pa_decode_workspace_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return pa::fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu",
                    who, need, workspace ? workspace_bytes : (size_t)0);
  a.out = p->out;
  a.q = p->q;
  a.k_cache = static_cast<const uint8_t *>(p->k_cache);
  a.v_cache = static_cast<const uint8_t *>(p->v_cache);
  a.block_tables = p->block_tables;
  a.context_lens = p->context_lens;
  a.k_new = static_cast<const uint8_t *>(p->k_new);
  a.v_new = static_cast<const uint8_t *>(p->v_new);
  a.slot_mapping = p->slot_mapping;
  const size_t rows = (size_t)p->num_seqs * p->num_q_heads * np;
  a.ws_ml = need ? static_cast<float *>(workspace) : nullptr;
  a.ws_acc = need ? static_cast<float *>(workspace) + rows * 2 : nullptr;
  a.ws_pre = nullptr;
  a.num_workers = 0;
  a.prefix_blocks = p->shared_prefix_blocks;
  a.park_slots = 1;
  a.ws_pfx_ml = nullptr;
  a.ws_pfx_acc = nullptr;
  if (bal) {
    size_t ml_off = 0, acc_off = 0;
    balanced_bytes(p, &ml_off, &acc_off);
    size_t pfx_off = 0;
    balanced_bytes(p, nullptr, nullptr, &pfx_off);
    a.ws_pre = static_cast<int32_t *>(workspace);
    a.ws_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + ml_off);
    a.ws_acc = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + acc_off);
    if (p->shared_prefix_blocks > 0) {
      const size_t rows = (size_t)p->num_seqs * p->num_q_heads;
      a.ws_pfx_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pfx_off);
      a.ws_pfx_acc = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pfx_off + round16(rows * 2 * 4));
    }
    a.num_workers = kBWaves * balanced_workgroups(p);
    a.park_slots = balanced_park_slots(p->kv_dtype, p->q_dtype, p->num_q_heads / p->num_kv_heads, p->head_dim,
                                       p->shared_prefix_blocks > 0);
  }

  a.num_seqs = p->num_seqs;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_ctx = p->max_context_len;
  a.max_parts = np;
  a.part_tokens = pt;
  a.out_dtype = p->out_dtype;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a.window = p->sliding_window;
  return PA_OK;
}

// A second stream of default priority per device, on which the shared-prefix
// kernel runs beside the balanced split, with the events that fork it from
// and join it back into the caller's stream.  The mutex keeps one call's
// fork, launches and join together when several host threads decode on
// one device.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

pa_status side_stream(SideStream **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static SideStream side[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_check(e, "pa_decode side stream: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: device %d beyond the first %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  SideStream &ss = side[dev];
  if (!ss.stream) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess)
      return hip_check(e, "pa_decode side stream: hipStreamCreateWithFlags");
    if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) != hipSuccess) {
      if (f) (void)hipEventDestroy(f);
      (void)hipStreamDestroy(st);
      return hip_check(e, "pa_decode side stream: hipEventCreateWithFlags");
    }
    ss.stream = st;
    ss.fork = f;
    ss.join = j;
  }
  *out = &ss;
  return PA_OK;
}

const void *prefix_kernel(pa_dtype kv, int D) {
  return kv == PA_BF16 ? (D == 128 ? reinterpret_cast<const void *>(&pa_prefix_kernel<PA_BF16, 128>)
                                   : reinterpret_cast<const void *>(&pa_prefix_kernel<PA_BF16, 64>))
                       : (D == 128 ? reinterpret_cast<const void *>(&pa_prefix_kernel<PA_F16, 128>)
                                   : reinterpret_cast<const void *>(&pa_prefix_kernel<PA_F16, 64>));
}

// side_stream_ok = false: a shared prefix's kernel runs before the split on
// the caller's stream (no stream of the library's own is created or used).
pa_status launch_partitions(const pa_decode_params *p, const DecodeArgs &a, hipStream_t hs,
                            const LaunchEvents &ev, bool side_stream_ok = true) {
  void *args[] = {const_cast<DecodeArgs *>(&a)};
  if (use_balanced(p)) {
    const dim3 grid((unsigned)(a.num_workers / kBWaves));
    const size_t lds = park_bytes(a.group, p->head_dim, a.park_slots);
    const void *bfn = balanced_kernel(p->kv_dtype, p->q_dtype, p->head_dim, a.group).fn;
    const dim3 pgrid((unsigned)(p->num_kv_heads * prefix_workgroups(p->num_seqs, a.group)));
    if (a.prefix_blocks == 0 || !side_stream_ok) {
      if (a.prefix_blocks > 0) {
        hipError_t e = hipLaunchKernel(prefix_kernel(p->kv_dtype, p->head_dim), pgrid, dim3(kThreads), args, 0, hs);
        if (e != hipSuccess) return hip_check(e, "pa_decode prefix launch");
        pa_status st = hip_check(hipGetLastError(), "pa_decode prefix launch");
        if (st != PA_OK) return st;
      }
      hipError_t e = launch_kernel(bfn, grid, dim3(kBThreads), args, lds, hs, ev);
      if (e != hipSuccess) return hip_check(e, "pa_decode balanced launch");
      return hip_check(hipGetLastError(), "pa_decode balanced launch");
    }
    // Shared prefix: every row's attention over the prefix, on the side
    // stream, runs beside the split (one prefix workgroup fits on each CU
    // next to the split's); the caller's stream waits for it after the
    // split, before anything that reads the workspace.
    SideStream *ss = nullptr;
    pa_status st = side_stream(&ss);
    if (st != PA_OK) return st;
    std::lock_guard<std::mutex> lock(ss->mu);
    hipError_t e = hipEventRecord(ss->fork, hs);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
    if (e != hipSuccess) return hip_check(e, "pa_decode prefix fork");
    e = hipLaunchKernel(prefix_kernel(p->kv_dtype, p->head_dim), pgrid, dim3(kThreads), args, 0, ss->stream);
    if (e != hipSuccess) return hip_check(e, "pa_decode prefix launch");
    if ((st = hip_check(hipGetLastError(), "pa_decode prefix launch")) != PA_OK) return st;
    if ((e = hipEventRecord(ss->join, ss->stream)) != hipSuccess) return hip_check(e, "pa_decode prefix join");
    e = launch_kernel(bfn, grid, dim3(kBThreads), args, lds, hs, ev);
    if (e != hipSuccess) return hip_check(e, "pa_decode balanced launch");
    if ((st = hip_check(hipGetLastError(), "pa_decode balanced launch")) != PA_OK) return st;
    return hip_check(hipStreamWaitEvent(hs, ss->join, 0), "pa_decode prefix join");
  }
  const bool mfma = use_mfma(p);
  const dim3 grid((unsigned)((int64_t)a.max_parts * p->num_kv_heads * p->num_seqs * head_chunks(p)));
  const void *fn = p->head_dim == 128 ? partition_kernel<128>(p->kv_dtype, mfma, a.group)
                                      : partition_kernel<64>(p->kv_dtype, mfma, a.group);
  hipError_t e = launch_kernel(fn, grid, dim3(kThreads), args, 0, hs, ev);
  if (e != hipSuccess) return hip_check(e, "pa_decode partition launch");
  return hip_check(hipGetLastError(), "pa_decode partition launch");
}

// True when the call's merge step launches a kernel.
bool has_merge(const pa_decode_params *p, const DecodeArgs &a) {
  return use_balanced(p) || a.max_parts > 1;
}

pa_status launch_merge(const pa_decode_params *p, const DecodeArgs &a, hipStream_t hs,
                       const LaunchEvents &ev) {
  if (!has_merge(p, a)) return record_events(ev, hs, "pa_decode merge events");
  int32_t rows = p->num_seqs * p->num_q_heads;
  const dim3 mgrid((rows + kMergeWaves - 1) / kMergeWaves);
  void *args[] = {const_cast<DecodeArgs *>(&a), &rows};
  const void *fn;
  if (use_balanced(p))
    fn = p->head_dim == 128 ? reinterpret_cast<const void *>(&pa_merge_balanced_kernel<128>)
                            : reinterpret_cast<const void *>(&pa_merge_balanced_kernel<64>);
  else
    fn = p->head_dim == 128 ? reinterpret_cast<const void *>(&pa_merge_kernel<128>)
                            : reinterpret_cast<const void *>(&pa_merge_kernel<64>);
  hipError_t e = launch_kernel(fn, mgrid, dim3(kMergeWaves * 64), args, 0, hs, ev);
  if (e != hipSuccess) return hip_check(e, "pa_decode merge launch");
  return hip_check(hipGetLastError(), "pa_decode merge launch");
}

LaunchEvents events_of(const pa_decode_params *p) {
  LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(p->start_event);
  ev.stop = static_cast<hipEvent_t>(p->stop_event);
  return ev;
}

// The attention launch(es) and the merge of one decode call.
pa_status decode_call(const pa_decode_params *p, void *workspace, size_t workspace_bytes, void *stream,
                      bool side_stream_ok, const char *who) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, who, a);
  if (st != PA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const LaunchEvents ev = events_of(p);
  if (p->num_seqs == 0) return record_events(ev, hs, "pa_decode events");
  const bool merge = has_merge(p, a);
  LaunchEvents first, second;
  first.start = ev.start;
  (merge ? second : first).stop = ev.stop;
  if ((st = launch_partitions(p, a, hs, first, side_stream_ok)) != PA_OK) return st;
  return merge ? launch_merge(p, a, hs, second) : PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                    void *stream) {
  return decode_call(p, workspace, workspace_bytes, stream, true, "pa_decode");
}

pa_status pa_decode_partitions(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                               void *stream) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, "pa_decode_partitions", a);
  if (st != PA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (p->num_seqs == 0) return record_events(events_of(p), hs, "pa_decode_partitions events");
  return launch_partitions(p, a, hs, events_of(p));
}

pa_status pa_decode_merge(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                          void *stream) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, "pa_decode_merge", a);
  if (st != PA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (p->num_seqs == 0) return record_events(events_of(p), hs, "pa_decode_merge events");
  return launch_merge(p, a, hs, events_of(p));
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- allocation-free decode
// Decode workspace for callers that cannot allocate device memory: a fixed
// array in the code object, one copy per device the library runs on, held
// until the process ends.  Every pa_decode_noalloc call on a device shares
// that device's copy.
constexpr size_t kScratchBytes = PA_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current (the array's name in host code is only a
// stand-in for the symbol).
pa_status scratch_address(void **out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_check(e, "pa_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d beyond the first %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_check(e, "pa_decode_noalloc: hipGetSymbolAddress");
    if (!ptr || !aligned16(ptr)) return pa::fail(PA_ERR_HIP, "pa_decode_noalloc: bad scratch address");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const pa_decode_params *p, void *stream) {
  const pa_status st = validate_all(p);
  if (st != PA_OK) return st;
  const size_t need = pa_decode_workspace_bytes(p);
  if (need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE,
                    "pa_decode_noalloc: the call needs %zu bytes of workspace, more than the %zu the library "
                    "holds per device (use pa_decode with a workspace)",
                    need, kScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const pa_status sa = scratch_address(&ws);
    if (sa != PA_OK) return sa;
  }
  // The workspace needs no initialization: every slot a launch reads was
  // written earlier in the same call.  A shared prefix's kernel runs before
  // the split on the caller's stream (no stream of the library's own).
  return decode_call(p, ws, need > 0 ? kScratchBytes : 0, stream, false, "pa_decode_noalloc");
}

pa_status pa_reshape_and_cache(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks, pa_dtype dtype, void *stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: bad sizes");
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: head_dim must be 64 or 128");
  if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: unknown dtype");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: NULL device pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(slot_mapping))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_reshape_and_cache: device pointers must be 16-byte aligned");
  const int eb = elem_bytes(dtype);
  const int64_t threads = (int64_t)num_tokens * num_kv_heads * (head_dim * eb / 16);
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto *kn = static_cast<const uint8_t *>(k_new);
  const auto *vn = static_cast<const uint8_t *>(v_new);
  auto *kc = static_cast<uint8_t *>(k_cache);
  auto *vc = static_cast<uint8_t *>(v_cache);
  const int64_t nslots = (int64_t)num_blocks * kBS;
  if (eb == 4 && head_dim == 128)
    hipLaunchKernelGGL((pa_reshape_and_cache_kernel<4, 128>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else if (eb == 4)
    hipLaunchKernelGGL((pa_reshape_and_cache_kernel<4, 64>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else if (head_dim == 128)
    hipLaunchKernelGGL((pa_reshape_and_cache_kernel<2, 128>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else
    hipLaunchKernelGGL((pa_reshape_and_cache_kernel<2, 64>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  return hip_check(hipGetLastError(), "pa_reshape_and_cache launch");
}

}  // extern "C"

namespace {

template <int FMT>
pa_status reshape_codes(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                        const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                        int32_t num_blocks, pa_dtype src_dtype, void *stream, const char *who) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return pa::fail(PA_ERR_INVALID_ARG, "%s: bad sizes", who);
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (src_dtype != PA_F16 && src_dtype != PA_BF16)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: rows must be F16 or BF16", who);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL device pointer", who);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(slot_mapping))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: device pointers must be 16-byte aligned", who);
  const int64_t rows = (int64_t)num_tokens * num_kv_heads;
  const dim3 grid((unsigned)((rows + 3) / 4));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto *kn = static_cast<const uint16_t *>(k_new);
  const auto *vn = static_cast<const uint16_t *>(v_new);
  auto *kc = static_cast<int8_t *>(k_cache);
  auto *vc = static_cast<int8_t *>(v_cache);
  const int64_t nslots = (int64_t)num_blocks * kBS;
  if (src_dtype == PA_BF16 && head_dim == 128)
    hipLaunchKernelGGL((pa_reshape_and_cache_i8_kernel<PA_BF16, 128, FMT>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else if (src_dtype == PA_BF16)
    hipLaunchKernelGGL((pa_reshape_and_cache_i8_kernel<PA_BF16, 64, FMT>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else if (head_dim == 128)
    hipLaunchKernelGGL((pa_reshape_and_cache_i8_kernel<PA_F16, 128, FMT>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  else
    hipLaunchKernelGGL((pa_reshape_and_cache_i8_kernel<PA_F16, 64, FMT>), grid, dim3(256), 0, hs, kn, vn, kc, vc, slot_mapping, num_tokens, num_kv_heads, nslots);
  return hip_check(hipGetLastError(), who);
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache_int8(const void *k_new, const void *v_new, int8_t *k_cache, int8_t *v_cache,
                                    const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t num_blocks, pa_dtype src_dtype, void *stream) {
  return reshape_codes<PA_I8>(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                              num_blocks, src_dtype, stream, "pa_reshape_and_cache_int8");
}

pa_status pa_reshape_and_cache_fp8(const void *k_new, const void *v_new, uint8_t *k_cache, uint8_t *v_cache,
                                   const int64_t *slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t num_blocks, pa_dtype src_dtype, void *stream) {
  return reshape_codes<PA_FP8>(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                               num_blocks, src_dtype, stream, "pa_reshape_and_cache_fp8");
}

pa_status pa_copy_blocks_int8(int8_t *k_cache, int8_t *v_cache, const int32_t *src_dst_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, void *stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks_int8: bad sizes");
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks_int8: head_dim must be 64 or 128");
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks_int8: NULL device pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks_int8: caches must be 16-byte aligned");
  // a block: every head's tile of codes and row scales
  hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3(num_pairs), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<uint8_t *>(k_cache), reinterpret_cast<uint8_t *>(v_cache), src_dst_pairs,
                     (int64_t)num_kv_heads * kBS * (head_dim + 4), num_blocks);
  return hip_check(hipGetLastError(), "pa_copy_blocks_int8 launch");
}

}  // extern "C"

namespace {

pa_status launch_swap(const void *src_k, const void *src_v, int32_t src_nb, void *dst_k, void *dst_v,
                      int32_t dst_nb, const int32_t *pairs, int32_t num_pairs, int64_t block_bytes,
                      hipStream_t hs, const char *who) {
  const int64_t chunks = (2 * block_bytes / 16 + kSwapVecs - 1) / kSwapVecs;
  hipLaunchKernelGGL(pa_swap_blocks_kernel, dim3(num_pairs, (unsigned)chunks), dim3(kSwapThreads), 0, hs,
                     static_cast<const uint8_t *>(src_k), static_cast<const uint8_t *>(src_v), src_nb,
                     static_cast<uint8_t *>(dst_k), static_cast<uint8_t *>(dst_v), dst_nb, pairs, block_bytes);
  return hip_check(hipGetLastError(), who);
}

// The address the GPU uses for p: device memory as it is, pinned host memory
// through its device mapping.  Anything else (pageable host memory, unknown
// pointers) is an error here rather than a memory fault in the kernel.
pa_status gpu_address(const void *p, const void **out, const char *who) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return pa::fail(PA_ERR_INVALID_ARG, "%s: %p is neither device memory nor pinned host memory", who, p);
  }
  if (attr.type == hipMemoryTypeDevice) {
    *out = p;
    return PA_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer && attr.hostPointer) {
    const char *hp = static_cast<const char *>(attr.hostPointer);
    *out = static_cast<const char *>(attr.devicePointer) + (static_cast<const char *>(p) - hp);
    return PA_OK;
  }
  return pa::fail(PA_ERR_INVALID_ARG, "%s: %p is neither device memory nor pinned host memory", who, p);
}

// Checks sizes and pointers; ptrs[] are replaced by their GPU addresses.
pa_status check_swap_args(int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t src_nb,
                          int32_t dst_nb, const void **ptrs, int nptr, const int32_t **pairs,
                          const char *who) {
  if (num_pairs < 0 || num_pairs > 65535 || num_kv_heads <= 0 || src_nb <= 0 || dst_nb <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: bad sizes (num_pairs must be in [0, 65535])", who);
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128", who);
  if (num_pairs == 0) return PA_OK;
  if (!*pairs) return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pairs", who);
  const void *pp = nullptr;
  pa_status st = gpu_address(*pairs, &pp, who);
  if (st != PA_OK) return st;
  *pairs = static_cast<const int32_t *>(pp);
  for (int i = 0; i < nptr; ++i) {
    if (!ptrs[i]) return pa::fail(PA_ERR_INVALID_ARG, "%s: NULL pool pointer", who);
    if (!aligned16(ptrs[i])) return pa::fail(PA_ERR_INVALID_ARG, "%s: pools must be 16-byte aligned", who);
    if ((st = gpu_address(ptrs[i], &ptrs[i], who)) != PA_OK) return st;
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_swap_blocks(const void *src_k, const void *src_v, int32_t src_num_blocks, void *dst_k,
                         void *dst_v, int32_t dst_num_blocks, const int32_t *src_dst_pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype, void *stream) {
  if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: unknown dtype");
  const void *ptrs[] = {src_k, src_v, dst_k, dst_v};
  const int32_t *pairs = src_dst_pairs;
  pa_status st = check_swap_args(num_pairs, num_kv_heads, head_dim, src_num_blocks, dst_num_blocks, ptrs, 4,
                                 &pairs, "pa_swap_blocks");
  if (st != PA_OK || num_pairs == 0) return st;
  return launch_swap(ptrs[0], ptrs[1], src_num_blocks, const_cast<void *>(ptrs[2]), const_cast<void *>(ptrs[3]),
                     dst_num_blocks, pairs, num_pairs, (int64_t)num_kv_heads * kBS * head_dim * elem_bytes(dtype),
                     static_cast<hipStream_t>(stream), "pa_swap_blocks launch");
}

pa_status pa_swap_blocks_int8(const int8_t *src_k, const int8_t *src_v, int32_t src_num_blocks, int8_t *dst_k,
                              int8_t *dst_v, int32_t dst_num_blocks, const int32_t *src_dst_pairs, int32_t num_pairs,
                              int32_t num_kv_heads, int32_t head_dim, void *stream) {
  const void *ptrs[] = {src_k, src_v, dst_k, dst_v};
  const int32_t *pairs = src_dst_pairs;
  pa_status st = check_swap_args(num_pairs, num_kv_heads, head_dim, src_num_blocks, dst_num_blocks, ptrs, 4,
                                 &pairs, "pa_swap_blocks_int8");
  if (st != PA_OK || num_pairs == 0) return st;
  // a block: every head's tile of codes and row scales
  return launch_swap(ptrs[0], ptrs[1], src_num_blocks, const_cast<void *>(ptrs[2]), const_cast<void *>(ptrs[3]),
                     dst_num_blocks, pairs, num_pairs, (int64_t)num_kv_heads * kBS * (head_dim + 4),
                     static_cast<hipStream_t>(stream), "pa_swap_blocks_int8 launch");
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *src_dst_pairs, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, pa_dtype dtype,
                         void *stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: bad sizes");
  if (head_dim != 64 && head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: head_dim must be 64 or 128");
  if (!valid_dtype(dtype)) return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: unknown dtype");
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: NULL device pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: caches must be 16-byte aligned");
  const int64_t block_bytes = (int64_t)num_kv_heads * kBS * head_dim * elem_bytes(dtype);
  hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3(num_pairs), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint8_t *>(k_cache), static_cast<uint8_t *>(v_cache), src_dst_pairs,
                     block_bytes, num_blocks);
  return hip_check(hipGetLastError(), "pa_copy_blocks launch");
}

}  // extern "C"

// ---------------------------------------------------------------- extend: host side
namespace {

struct ExtendShape {
  int nct, tpt, tpg, hparts, qgroups, pt, np;
};

pa_status validate_extend(const pa_extend_params *p) {
  if (!p) return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: params is NULL");
  // An array with no elements (no query rows; no sequences; no table columns) may be NULL.
  const bool rows = p->num_query_rows > 0, seqs = p->num_seqs > 0, cols = seqs && p->max_blocks_per_seq > 0;
  if ((rows && (!p->out || !p->q)) || (seqs && !p->context_lens) || (cols && !p->block_tables) ||
      !p->query_start || !p->k_cache || !p->v_cache)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: NULL device pointer");
  if (!aligned16(p->out) || !aligned16(p->q) || !aligned16(p->k_cache) || !aligned16(p->v_cache) ||
      !aligned16(p->block_tables) || !aligned16(p->context_lens) || !aligned16(p->query_start))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: device pointers must be 16-byte aligned");
  if (p->num_seqs < 0 || p->num_seqs > 65535 || p->num_query_rows < 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: num_seqs must be in [0, 65535], num_query_rows >= 0");
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads || p->num_kv_heads > 65535)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: num_q_heads must be a positive multiple of num_kv_heads");
  if (p->num_q_heads / p->num_kv_heads > kGMax)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_extend: at most %d query heads per KV head", kGMax);
  if (p->head_dim != 64 && p->head_dim != 128)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_extend: head_dim must be 64 or 128");
  if (p->kv_dtype != PA_F16 && p->kv_dtype != PA_BF16)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_extend: the cache must be fp16 or bf16");
  if (p->out_dtype != PA_F32 && p->out_dtype != p->kv_dtype)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_extend: out_dtype must be F32 or the cache type");
  if (p->max_blocks_per_seq < 0 || p->num_blocks <= 0 || p->max_context_len < 0 || p->max_query_len < 0)
    return pa::fail(PA_ERR_INVALID_ARG,
                    "pa_extend: num_blocks must be positive, the other sizes >= 0");
  if (p->partition_tokens < 0 || p->partition_tokens % kBS)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: partition_tokens must be 0 or a positive multiple of 16");
  if (!std::isfinite(p->scale)) return pa::fail(PA_ERR_INVALID_ARG, "pa_extend: scale must be finite");
  return PA_OK;
}

ExtendShape extend_shape(const pa_extend_params *p) {
  ExtendShape e;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int mq = std::max(p->max_query_len, 1);
  if (G > kTileCols) {  // a token's heads span tiles: NCT * 16 heads of one token per query group
    e.tpt = 1;
    e.nct = 2;
    e.tpg = 1;
    e.hparts = (G + e.nct * kTileCols - 1) / (e.nct * kTileCols);
  } else {
    e.tpt = kTileCols / G;
    const int64_t cols = (int64_t)mq * G;  // columns one sequence's new tokens need
    e.nct = cols > 2 * kTileCols ? kExtNctMax : cols > kTileCols ? 2 : 1;
    e.tpg = e.nct * e.tpt;
    e.hparts = 1;
  }
  e.qgroups = (mq + e.tpg - 1) / e.tpg * e.hparts;
  const int ctx = ((std::max(p->max_context_len, 1) + kBS - 1) / kBS) * kBS;
  if (p->partition_tokens > 0) {
    e.pt = p->partition_tokens;
  } else {
    // enough workgroups for about two per CU (one per CU with four tiles:
    // eight-wave workgroups), partitions of at least 64 tokens
    const int64_t base = (int64_t)std::max(p->num_seqs, 1) * p->num_kv_heads * e.qgroups;
    const int64_t want = (e.nct >= kExtNctMax ? 1LL : 2LL) * cu_count();
    const int64_t parts = base >= want ? 1 : (want + base - 1) / base;
    int64_t pt = (ctx + parts - 1) / parts;
    pt = std::max<int64_t>(64, (pt + kBS - 1) / kBS * kBS);
    e.pt = (int)std::min<int64_t>(pt, ctx);
  }
  e.np = (ctx + e.pt - 1) / e.pt;
  return e;
}

size_t extend_ws_bytes(const pa_extend_params *p, const ExtendShape &e) {
  if (e.np <= 1 || p->num_seqs == 0 || p->num_query_rows == 0) return 0;  // nothing split, or nothing to do
  return (size_t)p->num_query_rows * p->num_q_heads * e.np * (p->head_dim + 2) * sizeof(float);
}

template <int DT, int D>
const void *extend_kernel_nct(int nct) {
  switch (nct) {
    case 1: return reinterpret_cast<const void *>(&pa_extend_kernel<DT, D, 1>);
    case 2: return reinterpret_cast<const void *>(&pa_extend_kernel<DT, D, 2>);
    default: return reinterpret_cast<const void *>(&pa_extend_kernel<DT, D, kExtNctMax>);
  }
}

template <int D>
const void *extend_kernel(pa_dtype dt, int nct) {
  return dt == PA_BF16 ? extend_kernel_nct<PA_BF16, D>(nct) : extend_kernel_nct<PA_F16, D>(nct);
}

#ifdef PA_TRACE
// Read probe (traced build only): the balanced split's access pattern with
// none of its math.  A persistent grid of four-wave workgroups (one per CU)
// cuts a list of tile indices (block * num_kv_heads + head) into equal
// contiguous shares; each wave reads its units' K and V tiles (4 KiB each)
// through a 4-deep register ring of 16-byte non-temporal loads per lane and
// folds the data with XOR into one word, written per wave so that no load is
// dropped.  It shows what read rate that pattern reaches on the device.
__global__ __launch_bounds__(256, 1) void pa_read_probe_kernel(const uint8_t *k_cache, const uint8_t *v_cache,
                                                                const int32_t *tiles, int32_t n, uint32_t *sink) {
  constexpr int R = 4, NF = 4;  // ring depth; 1 KiB fragments per 4 KiB tile
  const int lane = threadIdx.x % 64;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int NW = gridDim.x * 4;
  const int C = (n + NW - 1) / NW, u0 = min(n, w * C), u1 = min(n, u0 + C);
  u32x4_t acc = {0, 0, 0, 0};
  for (int c0 = u0; c0 < u1; c0 += 64) {
    const int nc = min(64, u1 - c0);
    const int my = lane < nc ? tiles[c0 + lane] : 0;
    u32x4_t fr[R][2 * NF];
    auto load = [&](u32x4_t (&f)[2 * NF], int i) {
      const int64_t off = (int64_t)__builtin_amdgcn_readlane(my, min(i, nc - 1)) * 4096;
      const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(k_cache + off);
      const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(v_cache + off);
#pragma unroll
      for (int c = 0; c < NF; ++c) f[c] = __builtin_nontemporal_load(&kp[c * 64 + lane]);
#pragma unroll
      for (int c = 0; c < NF; ++c) f[NF + c] = __builtin_nontemporal_load(&vp[c * 64 + lane]);
    };
#pragma unroll
    for (int b = 0; b < R - 1; ++b) load(fr[b], b);
    for (int i0 = 0; i0 < nc; i0 += R) {
#pragma unroll
      for (int b = 0; b < R; ++b) {
        const int i = i0 + b;
        load(fr[(b + R - 1) % R], i + R - 1);  // (past the end: the last tile again)
        if (i < nc) {
#pragma unroll
          for (int c = 0; c < 2 * NF; ++c) acc ^= fr[b][c];
        }
      }
    }
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (lane == 0) sink[w] = x;
}
#endif

}  // namespace

#ifdef PA_TRACE
extern "C" {
// Traced build: copies the wave records of the last traced launch (8 uint64
// per wave: entry, inputs ready, first block, stream end, exit, XCD, blocks,
// written flag) to host memory; pa_trace_clear zeroes them.  Synchronous.
int pa_trace_read(void *host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(pa_trace_buf), std::min(bytes, sizeof(pa_trace_buf)), 0,
                                  hipMemcpyDeviceToHost);
}
int pa_trace_clear() {
  static uint64_t zeros[kTraceWaves * 8];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(pa_trace_buf), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice);
}
size_t pa_trace_bytes() { return sizeof(pa_trace_buf); }

// Read probe over n units of the tile list `tiles` (device, int32 tile
// indices of 4 KiB K and V tiles: a D = 128 16-bit cache), one workgroup per
// CU; sink (device) takes one word per wave (4 per CU).  Events as in
// pa_decode_params.  Returns a pa_status.
int pa_read_probe(const void *k_cache, const void *v_cache, const int32_t *tiles, int32_t n, uint32_t *sink,
                  size_t sink_words, void *start_event, void *stop_event, void *stream) {
  const int grid = cu_count();
  if (!k_cache || !v_cache || !tiles || !sink || n <= 0 || sink_words < (size_t)grid * 4)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_read_probe: null pointer, n <= 0 or a sink of fewer than %d words",
                    grid * 4);
  LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(start_event);
  ev.stop = static_cast<hipEvent_t>(stop_event);
  const uint8_t *k = static_cast<const uint8_t *>(k_cache), *v = static_cast<const uint8_t *>(v_cache);
  void *args[] = {&k, &v, &tiles, &n, &sink};
  const hipError_t err = launch_kernel(reinterpret_cast<const void *>(&pa_read_probe_kernel), dim3(grid),
                                       dim3(256), args, 0, static_cast<hipStream_t>(stream), ev);
  if (err != hipSuccess) return hip_check(err, "pa_read_probe launch");
  return hip_check(hipGetLastError(), "pa_read_probe launch");
}
}  // extern "C"
#endif

extern "C" {

int32_t pa_extend_partition_tokens(const pa_extend_params *p) {
  pa_status st = validate_extend(p);
  if (st != PA_OK) return -(int32_t)st;
  return extend_shape(p).pt;
}

size_t pa_extend_workspace_bytes(const pa_extend_params *p) {
  if (validate_extend(p) != PA_OK) return 0;
  return extend_ws_bytes(p, extend_shape(p));
}

pa_status pa_extend(const pa_extend_params *p, void *workspace, size_t workspace_bytes, void *stream) {
  pa_status st = validate_extend(p);
  if (st != PA_OK) return st;
  const ExtendShape e = extend_shape(p);
  const size_t need = extend_ws_bytes(p, e);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return pa::fail(PA_ERR_WORKSPACE, "pa_extend: workspace of %zu bytes (16-byte aligned) required, got %zu",
                    need, workspace ? workspace_bytes : (size_t)0);
  // (KV head, sequence, partition) triples in runs of 8, each run once per query group
  const int64_t grid = ((int64_t)p->num_kv_heads * p->num_seqs * e.np + 7) / 8 * 8 * e.qgroups;
  if (grid > INT32_MAX)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_extend: more than 2^31-1 workgroups (raise partition_tokens)");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  LaunchEvents ev;
  ev.start = static_cast<hipEvent_t>(p->start_event);
  ev.stop = static_cast<hipEvent_t>(p->stop_event);
  if (p->num_seqs == 0 || p->num_query_rows == 0) return record_events(ev, hs, "pa_extend events");
  ExtendArgs a;
  a.out = p->out;
  a.q = p->q;
  a.k_cache = static_cast<const uint8_t *>(p->k_cache);
  a.v_cache = static_cast<const uint8_t *>(p->v_cache);
  a.block_tables = p->block_tables;
  a.context_lens = p->context_lens;
  a.query_start = p->query_start;
  a.ws_ml = need ? static_cast<float *>(workspace) : nullptr;
  a.ws_acc = need ? static_cast<float *>(workspace) + (size_t)p->num_query_rows * p->num_q_heads * e.np * 2 : nullptr;
  a.num_seqs = p->num_seqs;
  a.num_q_heads = p->num_q_heads;
  a.num_kv_heads = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.max_blocks = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_ctx = p->max_context_len;
  a.max_q = p->max_query_len;
  a.num_rows = p->num_query_rows;
  a.max_parts = e.np;
  a.part_tokens = e.pt;
  a.out_dtype = p->out_dtype;
  a.qgroups = e.qgroups;
  a.tpt = e.tpt;
  a.tpg = e.tpg;
  a.hparts = e.hparts;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  const bool merge = e.np > 1;
  LaunchEvents first, second;
  first.start = ev.start;
  (merge ? second : first).stop = ev.stop;
  void *args[] = {&a};
  const void *fn = p->head_dim == 128 ? extend_kernel<128>(p->kv_dtype, e.nct) : extend_kernel<64>(p->kv_dtype, e.nct);
  const int threads = 64 * (e.nct >= kExtNctMax ? extend_waves<kExtNctMax>() : extend_waves<1>());
  hipError_t err = launch_kernel(fn, dim3((unsigned)grid), dim3(threads), args, 0, hs, first);
  if (err != hipSuccess) return hip_check(err, "pa_extend launch");
  if ((st = hip_check(hipGetLastError(), "pa_extend launch")) != PA_OK || !merge) return st;
  const int64_t rows = (int64_t)p->num_query_rows * p->num_q_heads;
  const void *mfn = p->head_dim == 128 ? reinterpret_cast<const void *>(&pa_extend_merge_kernel<128>)
                                       : reinterpret_cast<const void *>(&pa_extend_merge_kernel<64>);
  err = launch_kernel(mfn, dim3((unsigned)((rows + kMergeWaves - 1) / kMergeWaves)), dim3(kMergeWaves * 64), args,
                      0, hs, second);
  if (err != hipSuccess) return hip_check(err, "pa_extend merge launch");
  return hip_check(hipGetLastError(), "pa_extend merge launch");
}

}  // extern "C"
