// Device helpers shared by the HIP kernels of libsa (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa.h"

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- storage

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;
};
template <>
struct Elt<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte vector load (global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte streaming load with the nontemporal hint: for data read once (a
// scan of the whole cache), so it does not displace reusable cache lines.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Unpack one 16-byte chunk into floats (8 bf16 or 4 fp32 values).
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& w, float* f);
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& w, float* f) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

// Read `n` consecutive query values of either storage type as fp32.
__device__ __forceinline__ float load_q(const void* q, sa_dtype dt, int64_t i) {
  if (dt == SA_BF16) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(q)[i];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  return reinterpret_cast<const float*>(q)[i];
}

// E (4 or 8) consecutive q values from element i with vector loads; the
// element offset i is a multiple of E and q is 16-byte aligned.
template <int E, bool BF16>
__device__ __forceinline__ void load_q_vec(const void* q, int64_t i, float (&v)[E]) {
  static_assert(E == 4 || E == 8, "E is 4 or 8");
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(q) + i;
    uint32_t w[E / 2];
    if constexpr (E == 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x;
      w[1] = x.y;
    }
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      v[2 * j] = bf16_lo(w[j]);
      v[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(q) + i;
#pragma unroll
    for (int j = 0; j < E; j += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + j);
      v[j] = x.x;
      v[j + 1] = x.y;
      v[j + 2] = x.z;
      v[j + 3] = x.w;
    }
  }
}

// The E-value slices at element offset `off` of the G (<= 8) query heads
// g0, g0 + 1, ... of a group (head stride D): every load is issued before
// any value is used; slices of heads g >= G repeat head g0 and are unused.
template <int E, int D>
__device__ __forceinline__ void load_q_group(const void* q, sa_dtype dt, int64_t g0, int G,
                                             int off, float (&v)[8][E]) {
  if (dt == SA_BF16) {
#pragma unroll
    for (int g = 0; g < 8; ++g) load_q_vec<E, true>(q, (g0 + (g < G ? g : 0)) * D + off, v[g]);
  } else {
#pragma unroll
    for (int g = 0; g < 8; ++g) load_q_vec<E, false>(q, (g0 + (g < G ? g : 0)) * D + off, v[g]);
  }
}

// ------------------------------------------------------ lane-group reductions
// A "lane group" is LPR consecutive lanes of a wave (LPR in {4, 8, 16, 32}) that
// together hold one cache row.  The first steps use DPP within a 16-lane DPP
// row; LPR = 32 adds one cross-row exchange.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xf, 0xf, false);
}

constexpr int kQuadXor1 = 0xb1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;    // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32, "lane group of 4 to 32");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp<kRowMirror>(x);
  if constexpr (LPR == 32) x += __shfl_xor(x, 16);
  return x;
}

template <int LPR>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  if constexpr (LPR >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (LPR >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (LPR == 32) x = fmaxf(x, __shfl_xor(x, 16));
  return x;
}

// Exact token score pieces shared by every kernel that scores tokens one by
// one (so their fp32 results agree bit for bit):
//  * group_query_sum: lane's E values of (sum over the G <= 8 query heads of
//    the group) * scale, all G loads issued before any add;
//  * row_dot: one 16-byte piece of a cache row dotted with those values (fma
//    chain from 0 in element order), summed over the row's LPR lanes.
template <int E, int D>
__device__ __forceinline__ void group_query_sum(const void* q, sa_dtype dt, int64_t g0, int G,
                                                int off, float scale, float (&qs)[E]) {
  float qv[8][E];
  load_q_group<E, D>(q, dt, g0, G, off, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float acc = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) acc += g < G ? qv[g][e] : 0.0f;
    qs[e] = acc * scale;
  }
}

template <typename KT, int LPR, int E>
__device__ __forceinline__ float row_dot(const uint4& w, const float (&qs)[E]) {
  float kf[E];
  unpack16<KT>(w, kf);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc = fmaf(qs[e], kf[e], acc);
  return group_sum<LPR>(acc);
}

// Indexer score of one token ("Flash Attention vs Sparse Attention", DSA
// Stage 1): sum_h w_h max(0, q_h . k), with the key's DI bf16 values spread
// over LPR lanes (16 bytes each) and this lane's 16 bytes of every indexer
// query packed in qv.  Each lane dots its 8 dims with v_dot2_f32_bf16 (both
// operands bf16, so the products are exact and the sums fp32), the head
// sums close over the lane group with DPP.  Shared by every kernel that
// scores with the indexer, so their fp32 results agree bit for bit.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot8_bf16(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                        __builtin_bit_cast(bf16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), acc, false);
  return acc;
}

template <int LPR, int HP>
__device__ __forceinline__ float indexer_token(const uint4& kw, const uint4 (&qv)[HP],
                                               const float (&wv)[HP]) {
  float sc = 0.0f;
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    const float acc = group_sum<LPR>(dot8_bf16(kw, qv[h], 0.0f));
    sc = fmaf(wv[h], fmaxf(acc, 0.0f), sc);
  }
  return sc;
}

// This lane's 16 bytes (dims [8 sl, 8 sl + 8)) of the H <= HP indexer queries
// of row `b` and their weights; heads >= H are zero.
template <int DI, int HP>
__device__ __forceinline__ void load_indexer_queries(const uint8_t* q_idx, const float* w, int64_t b,
                                                     int H, int sl, uint4 (&qv)[HP],
                                                     float (&wv)[HP]) {
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    const bool live = h < H;
    wv[h] = live ? w[b * H + h] : 0.0f;
    qv[h] = live ? *reinterpret_cast<const uint4*>(q_idx + ((b * H + h) * DI) * 2 + sl * 16)
                 : make_uint4(0, 0, 0, 0);
  }
}

// DPP move of a uint32 across lanes; lanes whose source lies outside the row
// read 0 (bound_ctrl), lanes of rows outside ROW_MASK get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, true);
}

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;  // lane 15 of each row into the next row
constexpr int kRowBcast31 = 0x143;  // lane 31 into rows 2 and 3

// Wave-wide inclusive prefix sum of a uint32 (64 lanes): shifted adds inside
// each 16-lane row, then the row totals carried across rows by broadcasts.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += dpp_u32<kRowShr1>(v);
  v += dpp_u32<kRowShr2>(v);
  v += dpp_u32<kRowShr4>(v);
  v += dpp_u32<kRowShr8>(v);
  v += dpp_u32<kRowBcast15, 0xa>(v);
  v += dpp_u32<kRowBcast31, 0xc>(v);
  return v;
}

// ------------------------------------------------------------ top-k keys
// Order-preserving map of fp32 bit patterns onto uint32: a larger float maps
// to a larger key; -0.0 maps like +0.0; every NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sa
