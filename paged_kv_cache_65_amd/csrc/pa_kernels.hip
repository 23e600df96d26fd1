// Paged decode attention, KV append and block copy kernels for gfx950
// (CDNA4, wavefront 64), with their C-ABI entry points.
//
// Decode ("LLM Inference Optimization: KV-Cache, PagedAttention, and GPU
// Memory Efficiency", section "PagedAttention: OS Concepts Meet GPU Memory":
// walk the sequence's block table, load K and V of each physical block, score
// it and fold it in with an online softmax).  One workgroup of four waves
// takes one (context partition, KV head, sequence).  The waves split the
// partition's 16-token blocks round-robin; each wave keeps an online-softmax
// state (running max m, running sum l, weighted V sum) for all query heads of
// the KV head's group, so every K/V tile is read from HBM once and reused by
// the whole group.  The four wave states meet in LDS at the end; a partition
// either writes the final row (single-partition sequences) or an (m, l, acc)
// partial that the merge kernel folds with log-sum-exp rescaling.
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
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pa.h"
#include "pa_error.h"

namespace {

constexpr int kBS = 16;        // tokens per block
constexpr int kWaves = 4;      // waves per partition workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kGMax = 16;      // query heads per KV head (MFMA column tile)
constexpr int kDMax = 128;
constexpr float kLazyLog2 = 8.0f;  // MFMA path: softmax weights stay below 2^8

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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

__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

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
  int32_t num_seqs, num_q_heads, num_kv_heads, group, max_blocks, num_blocks, max_ctx, max_parts,
      part_tokens, out_dtype;
  float scale_log2;
};

__device__ inline bool ctx_valid(int L, const DecodeArgs &a) {
  return L >= 0 && L <= a.max_ctx && (int64_t)L <= (int64_t)a.max_blocks * kBS;
}

// Per-wave online-softmax states meet here at the end of a partition.
struct __align__(16) SmemBase {
  float acc[kWaves][kGMax][kDMax];
  float m[kWaves][kGMax];
  float l[kWaves][kGMax];
  uint32_t knew[kDMax];  // fused append: the new token's K and V rows (raw bits, up to 512 B)
  uint32_t vnew[kDMax];
};
struct __align__(16) SmemValu : SmemBase {
  float qs[kGMax][kDMax];        // q of the group in float32
  float ps[kWaves][kGMax][kBS];  // softmax weights of the current block
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

// ============================================================================
// MFMA wave: fp16 / bf16 caches.
//
// Lane l, with r = l % 16 and tq = l / 16:
//   K fragment c (c < D/32): the 16 bytes at tile + 1024c + 16l = token r,
//     dims 32c + 8tq .. +7  -> A operand of mfma_f32_16x16x32 (row = token).
//   q fragment c: head r of the group (zero when r >= G), same dims -> B operand.
//   score tile: sc[v] = s(token 4tq+v, head r).
//   V fragment m (m < D/32): 16 bytes at tile + 1024m + 16l = tokens
//     4tq..4tq+3 of dim 32m+r (first 8 bytes) and of dim 32m+16+r (last 8)
//     -> A operands of mfma_f32_16x16x16 for output tiles n = 2m, 2m+1
//     (row = dim, contraction = token).
//   P operand = the lane's own 4 weights (tokens 4tq..4tq+3, head r).
//   acc[n][v] = O(head r, dim 16n + 4tq + v).
// ============================================================================
template <int DT, int D>
struct MfmaWave {
  static constexpr int NC = D / 32;  // 16-byte fragments per tile
  static constexpr int NT = D / 16;  // output tiles
  static constexpr int TILE = kBS * D * 2;
#ifndef PA_MFMA_RING
#define PA_MFMA_RING 3
#endif
  static constexpr int kRing = PA_MFMA_RING;  // blocks held in registers per wave
  using v8 = typename std::conditional<DT == PA_BF16, bf16x8_t, f16x8_t>::type;

  struct Frag {
    u32x4_t k[NC];
    u32x4_t v[NC];
  };

  using Smem = SmemBase;

  v8 qB[NC];
  f32x4_t acc[NT];
  float m, l;

  __device__ void stage(const DecodeArgs &, Smem &, int, int, int) {}

  __device__ void init(const DecodeArgs &a, const Smem &, int s, int g, int lane) {
    const int r = lane % 16, tq = lane / 16;
    const int G = a.group;
    const int h = g * G + r;
    const u32x4_t *qrow =
        reinterpret_cast<const u32x4_t *>(static_cast<const uint8_t *>(a.q) +
                                          ((int64_t)s * a.num_q_heads + (r < G ? h : 0)) * D * 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4_t x = qrow[4 * c + tq];
      if (r >= G) x = u32x4_t{0, 0, 0, 0};
      qB[c] = __builtin_bit_cast(v8, x);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  __device__ static void load(Frag &f, const uint8_t *ktile, const uint8_t *vtile, int lane) {
    const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(ktile);
    const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vtile);
#pragma unroll
    for (int c = 0; c < NC; ++c) f.k[c] = __builtin_nontemporal_load(&kp[c * 64 + lane]);
#pragma unroll
    for (int c = 0; c < NC; ++c) f.v[c] = __builtin_nontemporal_load(&vp[c * 64 + lane]);
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

  // Splits p into hi + lo 16-bit values (hi = round(p), lo = round(p - hi)).
  __device__ static void split(const float p[4], u32x2_t &hi, u32x2_t &lo) {
    uint32_t h[4], w[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if constexpr (DT == PA_BF16) {
        __bf16 x = (__bf16)p[v];
        h[v] = __builtin_bit_cast(uint16_t, x);
        w[v] = __builtin_bit_cast(uint16_t, (__bf16)(p[v] - (float)x));
      } else {
        _Float16 x = (_Float16)p[v];
        h[v] = __builtin_bit_cast(uint16_t, x);
        w[v] = __builtin_bit_cast(uint16_t, (_Float16)(p[v] - (float)x));
      }
    }
    hi = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    lo = u32x2_t{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
  }

  // One block; `valid` = tokens of this block inside the context (1..16);
  // new_tok >= 0: that token's K/V come from the staged new row.
  __device__ void compute(Frag &f, int valid, float scale_log2, int lane, int new_tok,
                          const Smem &sm) {
    const int tq = lane / 16;
    if (new_tok >= 0) patch_new_token<2, NC>(f.k, f.v, new_tok, lane, sm.knew, sm.vnew);
    if (valid < kBS) {
      // Slots past the context may hold anything (NaN included): zero the V
      // elements so 0 * V stays 0; scores are masked below.
      const uint32_t lo = (4 * tq + 0 < valid ? 0x0000FFFFu : 0u) | (4 * tq + 1 < valid ? 0xFFFF0000u : 0u);
      const uint32_t hi = (4 * tq + 2 < valid ? 0x0000FFFFu : 0u) | (4 * tq + 3 < valid ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] &= u32x4_t{lo, hi, lo, hi};
    }
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = mma_qk(__builtin_bit_cast(v8, f.k[c]), qB[c], sc);
    float s[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) s[v] = sc[v] * scale_log2;
    if (valid < kBS) {
#pragma unroll
      for (int v = 0; v < 4; ++v) s[v] = (4 * tq + v < valid) ? s[v] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = max_xor32(max_xor16(mx));
    // Lazy reference max: the state is rescaled only when a head's block max
    // exceeds its reference by more than kLazyLog2, so weights stay below
    // 2^kLazyLog2 and most blocks skip the rescale (a wave-uniform branch).
    const bool bump = mx > m + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(bump)) {
      const float m_new = bump ? mx : m;
      const float alpha = exp2_neg(m - m_new);
      l *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[n] *= alpha;
      m = m_new;
    }
    float p[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(s[v] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    u32x2_t ph, pl;
    split(p, ph, pl);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const u32x2_t a0 = u32x2_t{f.v[c][0], f.v[c][1]};
      const u32x2_t a1 = u32x2_t{f.v[c][2], f.v[c][3]};
      acc[2 * c] = mma_pv(a0, ph, acc[2 * c]);
      acc[2 * c + 1] = mma_pv(a1, ph, acc[2 * c + 1]);
      acc[2 * c] = mma_pv(a0, pl, acc[2 * c]);
      acc[2 * c + 1] = mma_pv(a1, pl, acc[2 * c + 1]);
    }
  }

  // Publishes this wave's state for the group's heads into LDS.
  __device__ void finish(Smem &sm, int w, int lane, int G) {
    const int r = lane % 16, tq = lane / 16;
    const float lt = sum_xor32(sum_xor16(l));
    if (r < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<f32x4_t *>(&sm.acc[w][r][16 * n + 4 * tq]) = acc[n];
      if (tq == 0) {
        sm.m[w][r] = m;
        sm.l[w][r] = lt;
      }
    }
  }
};

// ============================================================================
// Vector-ALU wave: any cache type, GM = compile-time bound on the group size.
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

  __device__ void stage(const DecodeArgs &a, Smem &sm, int s, int g, int tid) {
    const int G = a.group;
    const uint8_t *qb = static_cast<const uint8_t *>(a.q);
    for (int i = tid; i < G * D; i += kThreads) {
      const int64_t e = ((int64_t)s * a.num_q_heads + g * G) * D + i;
      uint32_t bits;
      if constexpr (EB == 4)
        bits = reinterpret_cast<const uint32_t *>(qb)[e];
      else
        bits = reinterpret_cast<const uint16_t *>(qb)[e];
      sm.qs[i / D][i % D] = Ty<DT>::to_f32(bits);
    }
  }

  __device__ void init(const DecodeArgs &, const Smem &, int, int, int) {
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

  __device__ void compute(Frag &f, int valid, float scale_log2, int lane, int new_tok, Smem &sm,
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
        const float sv = (r < valid) ? part * scale_log2 : -INFINITY;
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
          vf[c * (X / 4) + sub][i] = (4 * tq + i < valid) ? x : 0.f;
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

// MFMA path: three 4-wave workgroups per CU (3 waves per SIMD, <= 168 VGPRs).
template <class W, int D, bool kMfma>
__global__ __launch_bounds__(kThreads, kMfma ? 3 : 1) void pa_partition_kernel(DecodeArgs a) {
  __shared__ typename W::Smem sm;
  // 1-D grid, KV head fastest, then sequence, then partition.  Workgroups are
  // dealt round-robin to the 8 XCDs by linear id, so this order spreads every
  // sequence's (unequal) partitions evenly over the XCDs; with the partition
  // index fastest, partition p of every sequence would land on the same XCD.
  const int g = blockIdx.x % a.num_kv_heads;
  const int s = (blockIdx.x / a.num_kv_heads) % a.num_seqs;
  const int p = blockIdx.x / (a.num_kv_heads * a.num_seqs);
  const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
  const int G = a.group;
  const int h0 = g * G;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // Loads that do not depend on the context length go out together with it:
  // the q fragments, and this wave's first 64 block ids (speculative: only
  // bounded by the table row; validated once the length is known).
  const int L = a.context_lens[s];
  const int blk0 = (int)((int64_t)p * a.part_tokens / kBS);
  const int32_t *trow = a.block_tables + (int64_t)s * a.max_blocks + blk0;
  const int ids_first = (int64_t)blk0 + wu + lane * kWaves < a.max_blocks ? trow[wu + lane * kWaves] : 0;
  W wave;
  wave.init(a, sm, s, g, lane);
  if (!ctx_valid(L, a)) {
    if (p == 0) write_rows<D>(a, s, h0, G, NAN);
    return;
  }
  if (L == 0) {
    if (p == 0) write_rows<D>(a, s, h0, G, 0.f);
    return;
  }
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (p >= nparts) return;
  const int tok0 = p * a.part_tokens;
  const int tok1 = min(L, tok0 + a.part_tokens);
  const int nblk = (tok1 - tok0 + kBS - 1) / kBS;
  const int last_valid = tok1 - (blk0 + nblk - 1) * kBS;

  wave.stage(a, sm, s, g, tid);
  if constexpr (!kMfma) __syncthreads();  // q staged in LDS
  int bad = 0;  // a block id outside the pool was seen (never dereferenced)
  // Fused append (one new token per sequence, at position L-1, in the last
  // block of the last partition): the wave that computes that block checks
  // the slot against the table, stages the token's K/V rows for head g in
  // LDS, stores them into the slot, and later takes the token from LDS.  A
  // slot that is not position L-1's slot marks the sequence bad: nothing is
  // written and the row is NaN.  Only that wave is involved (no barrier).
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
          const int valid = (j == nblk - 1) ? last_valid : kBS;
          const int nt = (j == nblk - 1) ? new_tok : -1;
          if constexpr (kMfma)
            wave.compute(fr[b], valid, a.scale_log2, lane, nt, sm);
          else
            wave.compute(fr[b], valid, a.scale_log2, lane, nt, sm, w, G);
        }
      }
    }
  }
  wave.finish(sm, w, lane, G);
  if (__syncthreads_or(bad)) {
    if (nparts == 1) {
      write_rows<D>(a, s, h0, G, NAN);
      return;
    }
    write_partial_nan<D>(a, s, h0, G, p);
  } else {
    // Fold the four wave states: M = max m_w, out = sum 2^(m_w-M) acc_w / sum 2^(m_w-M) l_w.
    for (int i = tid; i < G * D; i += kThreads) {
      const int h = i / D, d = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][h]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = exp2f(sm.m[ww][h] - M);  // 0 for a wave that saw no block
        num += f * sm.acc[ww][h][d];
        den += f * sm.l[ww][h];
      }
      const int64_t row = (int64_t)s * a.num_q_heads + h0 + h;
      if (nparts == 1) {
        store_out(a.out, row * D + d, num / den, a.out_dtype);
      } else {
        const int64_t prow = row * a.max_parts + p;
        a.ws_acc[prow * D + d] = num;
        if (d == 0) {
          a.ws_ml[prow * 2] = M;
          a.ws_ml[prow * 2 + 1] = den;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- merge kernel
// One wave per (sequence, query head) row with more than one partition:
//   M = max_p m_p,  out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.
// Each lane owns D/64 output dims and sums the partitions in order.  A NaN
// partial (bad table entry) makes the row NaN.
constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void pa_merge_kernel(DecodeArgs a, int32_t num_rows) {
  constexpr int PER = D / 64;  // output dims per lane
  const int lane = threadIdx.x % 64;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / 64;
  if (row >= num_rows) return;
  const int s = (int)(row / a.num_q_heads);
  const int L = a.context_lens[s];
  if (!ctx_valid(L, a)) return;
  const int np = (L + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  const float *ml = a.ws_ml + row * a.max_parts * 2;
  const float *acc = a.ws_acc + row * a.max_parts * D;
  // Same arithmetic, in the same order, as the merge inside pa_decode's
  // launch, so both paths give bit-identical rows.
  float M = -INFINITY;
  bool nan = false;
  for (int q = 0; q < np; ++q) {
    const float mq = ml[2 * q];
    nan |= mq != mq;
    M = fmaxf(M, mq);
  }
  float den = 0.f;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
#pragma unroll 4
  for (int q = 0; q < np; ++q) {
    const float f = exp2f(ml[2 * q] - M);
    den += f * ml[2 * q + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += f * acc[(int64_t)q * D + lane * PER + e];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    store_out(a.out, row * D + lane * PER + e, nan ? NAN : num[e] / den, a.out_dtype);
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

// ============================================================================
// Host side
// ============================================================================
int elem_bytes(pa_dtype d) { return d == PA_F32 ? 4 : 2; }
bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pa_status hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PA_OK;
}

pa_status validate(const pa_decode_params *p) {
  if (!p) return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: params is NULL");
  if (!p->out || !p->q || !p->k_cache || !p->v_cache || !p->block_tables || !p->context_lens)
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
  if (p->max_blocks_per_seq <= 0 || p->num_blocks <= 0 || p->max_context_len < 0)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: sizes must be positive");
  if (!valid_dtype(p->kv_dtype) || !valid_dtype(p->out_dtype))
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: unknown dtype");
  if (p->out_dtype != PA_F32 && p->out_dtype != p->kv_dtype)
    return pa::fail(PA_ERR_UNSUPPORTED, "pa_decode: out_dtype must be F32 or the cache type");
  if (p->partition_tokens < 0 || p->partition_tokens % kBS)
    return pa::fail(PA_ERR_INVALID_ARG, "pa_decode: partition_tokens must be 0 or a positive multiple of 16");
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
int32_t resolve_partition(const pa_decode_params *p) {
  if (p->partition_tokens > 0) return p->partition_tokens;
  const int32_t ctx = ((std::max(p->max_context_len, 1) + kBS - 1) / kBS) * kBS;
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

size_t partial_bytes(const pa_decode_params *p, int32_t np) {
  return (size_t)p->num_seqs * p->num_q_heads * np * (p->head_dim + 2) * sizeof(float);
}


int32_t num_partitions(const pa_decode_params *p, int32_t pt) {
  return std::max(1, (std::max(p->max_context_len, 1) + pt - 1) / pt);
}

template <int DT, int D>
void launch_valu(int G, dim3 grid, hipStream_t st, const DecodeArgs &a) {
  if (G <= 1)
    hipLaunchKernelGGL((pa_partition_kernel<ValuWave<DT, D, 1>, D, false>), grid, dim3(kThreads), 0, st, a);
  else if (G <= 2)
    hipLaunchKernelGGL((pa_partition_kernel<ValuWave<DT, D, 2>, D, false>), grid, dim3(kThreads), 0, st, a);
  else if (G <= 4)
    hipLaunchKernelGGL((pa_partition_kernel<ValuWave<DT, D, 4>, D, false>), grid, dim3(kThreads), 0, st, a);
  else if (G <= 8)
    hipLaunchKernelGGL((pa_partition_kernel<ValuWave<DT, D, 8>, D, false>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((pa_partition_kernel<ValuWave<DT, D, 16>, D, false>), grid, dim3(kThreads), 0, st, a);
}

template <int D>
void launch_partition(pa_dtype dt, bool mfma, int G, dim3 grid, hipStream_t st, const DecodeArgs &a) {
  if (mfma) {
    if (dt == PA_BF16)
      hipLaunchKernelGGL((pa_partition_kernel<MfmaWave<PA_BF16, D>, D, true>), grid, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((pa_partition_kernel<MfmaWave<PA_F16, D>, D, true>), grid, dim3(kThreads), 0, st, a);
  } else {
    if (dt == PA_BF16)
      launch_valu<PA_BF16, D>(G, grid, st, a);
    else if (dt == PA_F16)
      launch_valu<PA_F16, D>(G, grid, st, a);
    else
      launch_valu<PA_F32, D>(G, grid, st, a);
  }
}

}  // namespace

extern "C" {

int32_t pa_decode_partition_tokens(const pa_decode_params *p) {
  pa_status st = validate(p);
  if (st != PA_OK) return -(int32_t)st;
  return resolve_partition(p);
}

size_t pa_decode_workspace_bytes(const pa_decode_params *p) {
  if (validate(p) != PA_OK) return 0;
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
  pa_status st = validate(p);
  if (st != PA_OK) return st;
  const int32_t pt = resolve_partition(p);
  const int32_t np = num_partitions(p, pt);
  if ((int64_t)np * p->num_kv_heads * p->num_seqs > INT32_MAX)
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
  return PA_OK;
}

pa_status launch_partitions(const pa_decode_params *p, const DecodeArgs &a, hipStream_t hs) {
  const bool mfma = p->kernel == PA_KERNEL_MFMA || (p->kernel == PA_KERNEL_AUTO && p->kv_dtype != PA_F32);
  const dim3 grid((unsigned)((int64_t)a.max_parts * p->num_kv_heads * p->num_seqs));
  if (p->head_dim == 128)
    launch_partition<128>(p->kv_dtype, mfma, a.group, grid, hs, a);
  else
    launch_partition<64>(p->kv_dtype, mfma, a.group, grid, hs, a);
  return hip_check(hipGetLastError(), "pa_decode partition launch");
}

pa_status launch_merge(const pa_decode_params *p, const DecodeArgs &a, hipStream_t hs) {
  if (a.max_parts <= 1) return PA_OK;
  const int32_t rows = p->num_seqs * p->num_q_heads;
  const dim3 mgrid((rows + kMergeWaves - 1) / kMergeWaves);
  if (p->head_dim == 128)
    hipLaunchKernelGGL(pa_merge_kernel<128>, mgrid, dim3(kMergeWaves * 64), 0, hs, a, rows);
  else
    hipLaunchKernelGGL(pa_merge_kernel<64>, mgrid, dim3(kMergeWaves * 64), 0, hs, a, rows);
  return hip_check(hipGetLastError(), "pa_decode merge launch");
}

}  // namespace

extern "C" {

pa_status pa_decode(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                    void *stream) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, "pa_decode", a);
  if (st != PA_OK || p->num_seqs == 0) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = launch_partitions(p, a, hs)) != PA_OK) return st;
  return launch_merge(p, a, hs);
}

pa_status pa_decode_partitions(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                               void *stream) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, "pa_decode_partitions", a);
  if (st != PA_OK || p->num_seqs == 0) return st;
  return launch_partitions(p, a, static_cast<hipStream_t>(stream));
}

pa_status pa_decode_merge(const pa_decode_params *p, void *workspace, size_t workspace_bytes,
                          void *stream) {
  DecodeArgs a;
  pa_status st = prepare(p, workspace, workspace_bytes, "pa_decode_merge", a);
  if (st != PA_OK || p->num_seqs == 0) return st;
  return launch_merge(p, a, static_cast<hipStream_t>(stream));
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
