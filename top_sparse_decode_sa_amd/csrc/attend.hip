// Split-K online-softmax decode attention over a selected token set (or over
// the whole cache), and the log-sum-exp combine of the splits.
//
// What is computed ("Flash Attention vs Sparse Attention", DSA Stage 2 and
// the tiling + online-softmax section; "Inference-time context sparsity",
// section 3.C): for every query head of a (sequence, KV head) row, softmax
// attention restricted to the row's selected tokens, reading only those K/V
// rows from HBM.
//
// Two launches:
//   1. attend: grid (nsplit, rows).  A workgroup takes `chunk` consecutive
//      slots of its row's selection and writes one partial per query head:
//      (o = sum_t exp2(l_t - m) V_t, m, l = sum_t exp2(l_t - m)), logits in
//      base 2 (log2(e) folded into q).  With nsplit == 1 it writes o / l
//      directly and there is no second launch.
//   2. combine: grid (rows, G); merges the nsplit partials of a row with a
//      log-sum-exp combine and writes the fp32 output.
// The partials travel through the workspace between the two launches; the
// kernel boundary makes them visible, so no cross-workgroup synchronisation
// (and no zero-initialised counter) is needed.
//
// Kernels:
//   * attend_sparse_kernel (bf16, head_dim 128, G <= 4), for selected sets
//     and for dense decode alike: a workgroup of 1 to 12 waves; each wave
//     takes rounds of up to 64 slots.  Per round every index, key and value
//     load is issued before any is used (no load sits under a branch, so the
//     in-order load counter keeps them all in flight).  Lane l holds token
//     l%16's key dims [32c + 8(l/16), +8) -- the B operand of
//     v_mfma_f32_16x16x32_bf16 with the group's queries as the A operand --
//     so four MFMAs give the G logits of 16 tokens.  P.V also runs on MFMA
//     (P split into two bf16 parts).  Rounds merge online per wave; the
//     waves of a workgroup merge through LDS.  Dense decode walks contiguous
//     tokens without index loads.
//   * attend_kernel (any other dtype / head_dim / group): lane groups of LPR
//     lanes hold whole cache rows; logits reduce with DPP inside the group.
#include <math.h>

#include <algorithm>
#include <initializer_list>

#include "common.hpp"
#include "internal.hpp"
#include "topk_core.hpp"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // generic kernel: slots per lane group in flight

struct AttendArgs {
  const void* q;
  sa_dtype q_dtype;
  const uint8_t* k;
  const uint8_t* v;
  int64_t sb, sh, st;  // element strides
  int32_t Hq, Hkv;
  int32_t kv_div;  // row r reads KV head r / kv_div (1, or G for per-query-head rows)
  int64_t N;
  float qscale;  // softmax scale * log2(e)
  const int32_t* idx;
  int32_t n_idx;
  int32_t bs;
  int64_t n_slots;
  int32_t chunk;
  int32_t nsplit;
  int32_t rounds;  // gather kernel: slot rounds per wave
  float* scores;   // kIdxDenseScored: [rows, N] exact scores
  float sscale;    // softmax scale (the exact score's scale)
  float* out;
  float* part;  // [rows, nsplit, G, D + 2]: o[G][D], m[G], l[G]
  uint32_t row_span;  // pair kernel: bytes of one row's cache, N * st * 2 (< 2^32)
  int32_t rows;       // B * Hkv
};

// Buffer resource word 3 of a raw (stride 0) buffer of 32-bit data; loads
// past num_records return zeros.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy operand of a buffer load: nontemporal.
constexpr int kBufferNT = 2;

// 16-byte nontemporal buffer load: a gathered row is read once, so it is
// fetched without displacing reusable lines (on a cold cache this also keeps
// the gather from evicting, and writing back, other data).
__device__ __forceinline__ uint4 ld16_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kBufferNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kBufferNT);
  return make_uint2(v.x, v.y);
}

template <int MODE>
__device__ __forceinline__ int64_t resolve_slot(const AttendArgs& a, int row, int b, int64_t j,
                                                bool& ok) {
  // Out-of-range indices as in slot_token below: token N - 1, or masked.
  const uint32_t last = (uint32_t)(a.N - 1);
  if constexpr (MODE == kIdxDense) {
    return j;
  } else if constexpr (MODE == kIdxTokenPerHead) {
    return min((uint32_t)a.idx[(int64_t)row * a.n_idx + j], last);
  } else if constexpr (MODE == kIdxTokenShared) {
    return min((uint32_t)a.idx[(int64_t)b * a.n_idx + j], last);
  } else {
    const int64_t blk = a.idx[(int64_t)row * a.n_idx + j / a.bs];
    const int64_t t = blk * a.bs + j % a.bs;
    const bool in = t >= 0 && t < a.N;
    ok = ok && in;
    return in ? t : a.N - 1;
  }
}

// Write one workgroup's value for query head h, dimension dim: the final
// output when the row has one split, else the partial (o, and m/l once).
template <int G, int D>
__device__ __forceinline__ void write_result(const AttendArgs& a, int row, int split, int b, int r,
                                             int h, int dim, float O, float M, float L) {
  if (a.nsplit == 1) {
    a.out[((int64_t)b * a.Hq + (int64_t)r * G + h) * D + dim] = O / L;
  } else {
    float* p = a.part + ((int64_t)row * a.nsplit + split) * (G * (D + 2));
    p[h * D + dim] = O;
    if (dim == 0) {
      p[G * D + h] = M;
      p[G * D + G + h] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic kernel: lane groups hold whole rows, DPP reductions.
template <typename KT, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int NG = kThreads / LPR;
  constexpr int U = kUnroll;

  __shared__ float s_m[NG][G];
  __shared__ float s_l[NG][G];
  __shared__ float s_o[NG][G][D];

  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;

  float qv[G][E];
  {
    float q8[8][E];
    load_q_group<E, D>(a.q, a.q_dtype, (int64_t)b * a.Hq + (int64_t)r * G, G, sl * E, q8);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) qv[g][e] = q8[g][e] * a.qscale;
  }

  const int64_t kv_off = ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh) * EB + sl * 16;
  const uint8_t* kbase = a.k + kv_off;
  const uint8_t* vbase = a.v + kv_off;
  const int64_t row_bytes = a.st * EB;

  float m[G], l[G], o[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.0f;
  }

  const int64_t s0 = (int64_t)split * a.chunk;
  const int64_t s1 = min(s0 + (int64_t)a.chunk, a.n_slots);
  const int iters = (a.chunk + NG * U - 1) / (NG * U);

  for (int it = 0; it < iters; ++it) {
    bool ok[U];
    uint4 kw[U], vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = s0 + (int64_t)(it * U + u) * NG + grp;
      ok[u] = j < s1;
      int64_t t = 0;
      if (ok[u]) t = resolve_slot<MODE>(a, row, b, j, ok[u]);
      if (ok[u]) {
        kw[u] = ld16(kbase + t * row_bytes);
        vw[u] = ld16(vbase + t * row_bytes);
      } else {
        kw[u] = make_uint4(0, 0, 0, 0);
        vw[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float lg[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[E];
      unpack16<KT>(kw[u], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(qv[g][e], kf[e], acc);
        acc = group_sum<LPR>(acc);
        lg[u][g] = ok[u] ? acc : -INFINITY;
      }
    }
    float vf[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) unpack16<KT>(vw[u], vf[u]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float bm = lg[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, lg[u][g]);
      const float mn = fmaxf(m[g], bm);
      if (mn == -INFINITY) continue;  // nothing valid yet in this lane group
      const float alpha = exp2f(m[g] - mn);
      float ls = l[g] * alpha;
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = o[g][e] * alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = exp2f(lg[u][g] - mn);
        ls += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(p, vf[u][e], acc[e]);
      }
      l[g] = ls;
      m[g] = mn;
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] = acc[e];
    }
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (sl == 0) {
      s_m[grp][g] = m[g];
      s_l[grp][g] = l[g];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s_o[grp][g][sl * E + e] = o[g][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += kThreads) {
    const int g = x / D;
    const int dim = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < NG; ++q) M = fmaxf(M, s_m[q][g]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < NG; ++q) {
        const float w = exp2f(s_m[q][g] - M);
        L = fmaf(s_l[q][g], w, L);
        O = fmaf(s_o[q][g][dim], w, O);
      }
    }
    write_result<G, D>(a, row, split, b, r, g, dim, O, M, L);
  }
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128, G <= 4: MFMA logits, one wave per 16-token tile.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_bcast0(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Slot j of a row (s0 <= j < s1) -> token position, for a slot that may lie
// past the selection: the load is always made at an in-range position (the
// last slot, the last token) and `ok` reports whether the slot is real.  No
// load sits under a branch, so the wave's loads stay in flight together.
template <int MODE, bool LIDX = false>
__device__ __forceinline__ int32_t slot_token(const AttendArgs& a, int row, int b, int64_t j,
                                              int64_t s1, bool& ok, const int32_t* lidx = nullptr) {
  ok = j < s1;
  const int64_t jj = ok ? j : s1 - 1;
  // A token index outside [0, N) (a broken precondition) is read as token
  // N - 1, so no load leaves the row's cache; block tokens past the end are
  // masked out.
  const uint32_t last = (uint32_t)(a.N - 1);
  if constexpr (LIDX) {
    return (int32_t)min((uint32_t)lidx[jj], last);  // the row's index list, already in LDS
  } else if constexpr (MODE == kIdxDense || MODE == kIdxDenseScored) {
    return (int32_t)jj;
  } else if constexpr (MODE == kIdxTokenPerHead) {
    return (int32_t)min((uint32_t)a.idx[(int64_t)row * a.n_idx + jj], last);
  } else if constexpr (MODE == kIdxTokenShared) {
    return (int32_t)min((uint32_t)a.idx[(int64_t)b * a.n_idx + jj], last);
  } else {
    const int64_t t = (int64_t)a.idx[(int64_t)row * a.n_idx + jj / a.bs] * a.bs + jj % a.bs;
    const bool in = t >= 0 && t < a.N;
    ok = ok && in;
    return (int32_t)(in ? t : a.N - 1);
  }
}

// K/V row pieces: a dense scan, and the 128-token runs of selected blocks,
// read every row once in long contiguous runs, so their loads are
// nontemporal (streaming); gathered token rows use ordinary loads.
template <int MODE>
__device__ __forceinline__ uint4 ld_kv(const uint8_t* p) {
  if constexpr (MODE == kIdxDense || MODE == kIdxDenseScored || MODE == kIdxBlockPerHead)
    return ld16_nt(p);
  else return ld16(p);
}

// Gather-attend over selected slots (or all tokens): 1 to kMaxSparseWaves
// waves per workgroup (the block size says how many), `rounds` rounds of up
// to 16 * TILES slots per wave.  Within a round the memory operations are
// ordered for the in-order load counter: one index load per lane per tile
// (lane l reads the token of slot l % 16), then every key row piece of every
// tile, then every value row piece (value-row token ids come from the owning
// lane by a shuffle), then the compute.  Q.K and P.V run on MFMA; a round's
// softmax takes two passes over its tokens (one max, one sum per head), and
// rounds merge into a running (max, sum, o) per head.  The waves of a
// workgroup merge in LDS and write one result.
constexpr int kMaxSparseWaves = 12;
// The scored dense scan keeps a few more values live per round; at most 4
// waves per workgroup give it the registers to do so without spilling.
constexpr int kMaxScoredWaves = 4;

template <int MODE>
constexpr int max_waves() {
  return MODE == kIdxDenseScored ? kMaxScoredWaves : kMaxSparseWaves;
}

// LDS of one gather-attend workgroup: p of slot 16i + 4u + g for head h at
// s_pa[wave][h][i][g][u] (the MFMA A-fragment order of the P.V product), and
// each wave's (o, m, l) for the merge of the waves.
template <int G, int TILES>
struct AttendLds {
  alignas(16) float s_pa[kMaxSparseWaves][G][TILES][4][4];
  alignas(16) float s_o[kMaxSparseWaves][G][128];
  float s_ml[kMaxSparseWaves][2][G];
};

// The workgroup's share of the gather-attend (the kernel below, and the
// merge-then-attend kernel, which passes the row's index list in LDS as
// `lidx` with LIDX set).
template <int G, int MODE, int TILES, bool LIDX>
__device__ __forceinline__ void attend_sparse_body(const AttendArgs& a, const int32_t* lidx,
                                                   AttendLds<G, TILES>& lds) {
  static_assert(G >= 1 && G <= 4, "query heads of a group fit MFMA rows 0..3");
  constexpr int D = 128;
  auto& s_pa = lds.s_pa;
  auto& s_o = lds.s_o;
  auto& s_ml = lds.s_ml;
  const int nw = blockDim.x >> 6;  // waves in this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int rq = lane >> 4;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const int64_t wg0 = (int64_t)split * a.chunk;
  const int64_t wg1 = min(wg0 + (int64_t)a.chunk, a.n_slots);

  // q of head n (lanes n >= G carry zeros): MFMA A fragments, dims [32c + 8rq, +8)
  bf16x8_t qa[4];
  {
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) +
                        (((int64_t)b * a.Hq + (int64_t)r * G + (n < G ? n : 0)) * D + 8 * rq) * 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 w = ld16(qb + 64 * c);
      if (n >= G) w = make_uint4(0, 0, 0, 0);
      __builtin_memcpy(&qa[c], &w, 16);
    }
  }

  const int64_t kv_off = ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh) * 2;
  const uint8_t* kbase = a.k + kv_off + 16 * rq;
  const uint8_t* vbase = a.v + kv_off + 16 * n;
  const int64_t row_bytes = a.st * 2;

  // running (max, sum, o) of head rq over this wave's rounds; lane (n, rq)
  // holds o for dims [8n, 8n + 8)
  float m_me = -INFINITY, l_me = 0.0f;
  float mine[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int rd = 0; rd < a.rounds; ++rd) {
    // this wave's slots of round rd: [s0, s1), 16 * TILES of them; a wave with
    // none skips the round whole (a uniform branch around it, not around loads)
    const int64_t s0 = wg0 + ((int64_t)rd * nw + wave) * 16 * TILES;
    const int64_t s1 = min(s0 + 16 * TILES, wg1);
    if (s0 >= wg1) break;

    // 1. token of slot 16i + n of every tile
    int32_t tok[TILES];
    bool ok[TILES];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
      tok[i] = slot_token<MODE, LIDX>(a, row, b, s0 + 16 * i + n, s1, ok[i], lidx);

    // 2. key pieces of every tile, then value rows (token 4u + rq of each tile)
    uint4 kw[TILES][4], vw[TILES][4];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) kw[i][c] = ld_kv<MODE>(kbase + (int64_t)tok[i] * row_bytes + 64 * c);
    int32_t tv[TILES][4];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) tv[i][u] = __shfl(tok[i], 4 * u + rq);
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) vw[i][u] = ld_kv<MODE>(vbase + (int64_t)tv[i][u] * row_bytes);
    // keep every load above this point: all rows of the wave are requested
    // before the first logit is computed
    __builtin_amdgcn_sched_barrier(0);

    // 3. logits of every tile: rows 0..G-1 of the MFMA results, in lanes 0..15
    float lg[TILES][G];
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8_t kb;
        __builtin_memcpy(&kb, &kw[i][c], 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) lg[i][h] = (rq == 0 && ok[i]) ? acc[h] * a.qscale : -INFINITY;
      if constexpr (MODE == kIdxDenseScored) {
        // the token's exact score from the same logits; in a dense scan slot
        // j is token j (recomputed here, so the token ids need not stay live
        // in registers)
        if (rq == 0 && ok[i]) {
          float sc = 0.0f;
#pragma unroll
          for (int h = 0; h < G; ++h) sc += acc[h];
          __builtin_nontemporal_store(sc * a.sscale, a.scores + (int64_t)row * a.N + s0 + 16 * i + n);
        }
      }
    }
    // 4. one max per head over the wave's tokens (valid in lanes 0..15), then
    //    p = 2^(logit - max) and its sum
    float M[G], Lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = lg[0][h];
#pragma unroll
      for (int i = 1; i < TILES; ++i) mx = fmaxf(mx, lg[i][h]);
      M[h] = group_max<16>(mx);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float ls = 0.0f;
#pragma unroll
      for (int i = 0; i < TILES; ++i) {
        const float pv = M[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lg[i][h] - M[h]);
        lg[i][h] = pv;
        ls += pv;
      }
      Lsum[h] = group_sum<16>(ls);
    }
    // 5. O = P.V on MFMA.  K-step t covers tiles 2t and 2t+1; its k index
    //    8g + j stands for slot 16(2t + j/4) + 4(j%4) + g.  B fragment of lane
    //    (n, g): value dim 8n + e of those 8 slots, which this lane loaded as
    //    vw[2t + j/4][j%4] (MFMA e takes the dims 8n + e, n = 0..15).  A
    //    fragment: P enters as two bf16 parts, p = hi + lo to 2^-16 relative
    //    (hi: p truncated to bf16; lo: the rest, rounded), so the product keeps
    //    fp32 accuracy: row 4h carries head h's hi part, row 4h + 1 its lo part.
    //    Lane (n, h) ends with O[h][8n + e] = acc[e][0] + acc[e][1].
    if (rq == 0) {
#pragma unroll
      for (int i = 0; i < TILES; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) s_pa[wave][h][i][n & 3][n >> 2] = lg[i][h];
    }
    __builtin_amdgcn_wave_barrier();
    const int ha = n >> 2;
    const bool arow = (n & 3) < 2 && ha < G;
    const bool lo_row = (n & 1) != 0;
    const int hc = ha < G ? ha : G - 1;
    f32x4_t acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < (TILES + 1) / 2; ++t) {
      float pj[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int i = 2 * t + half;
        float4 q4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (i < TILES)
          q4 = *reinterpret_cast<const float4*>(&s_pa[wave][hc][i < TILES ? i : 0][rq][0]);
        pj[4 * half + 0] = arow ? q4.x : 0.0f;
        pj[4 * half + 1] = arow ? q4.y : 0.0f;
        pj[4 * half + 2] = arow ? q4.z : 0.0f;
        pj[4 * half + 3] = arow ? q4.w : 0.0f;
      }
      uint32_t af[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t b0 = __float_as_uint(pj[2 * d]);
        const uint32_t b1 = __float_as_uint(pj[2 * d + 1]);
        const uint32_t hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // truncated bf16 pair
        f32x2_t rest = {pj[2 * d] - __uint_as_float(b0 & 0xffff0000u),
                        pj[2 * d + 1] - __uint_as_float(b1 & 0xffff0000u)};
        bf16x2_t lo2 = __builtin_convertvector(rest, bf16x2_t);
        uint32_t lo;
        __builtin_memcpy(&lo, &lo2, 4);
        af[d] = lo_row ? lo : hi;
      }
      bf16x8_t a_p;
      __builtin_memcpy(&a_p, af, 16);
    const uint4 z = make_uint4(0, 0, 0, 0);
      const uint4 v0 = vw[2 * t][0], v1 = vw[2 * t][1], v2 = vw[2 * t][2], v3 = vw[2 * t][3];
      const uint4 v4 = 2 * t + 1 < TILES ? vw[2 * t + 1 < TILES ? 2 * t + 1 : 0][0] : z;
      const uint4 v5 = 2 * t + 1 < TILES ? vw[2 * t + 1 < TILES ? 2 * t + 1 : 0][1] : z;
      const uint4 v6 = 2 * t + 1 < TILES ? vw[2 * t + 1 < TILES ? 2 * t + 1 : 0][2] : z;
      const uint4 v7 = 2 * t + 1 < TILES ? vw[2 * t + 1 < TILES ? 2 * t + 1 : 0][3] : z;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // word e/2 of each row holds dims 8n + 2(e/2) (low half) and +1 (high)
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        auto word = [&](const uint4& x) -> uint32_t {
          return (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
        };
        uint32_t bw[4];
        bw[0] = __builtin_amdgcn_perm(word(v1), word(v0), sel);
        bw[1] = __builtin_amdgcn_perm(word(v3), word(v2), sel);
        bw[2] = __builtin_amdgcn_perm(word(v5), word(v4), sel);
        bw[3] = __builtin_amdgcn_perm(word(v7), word(v6), sel);
        bf16x8_t bv;
        __builtin_memcpy(&bv, bw, 16);
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_p, bv, acc[e], 0, 0, 0);
      }
    }

    // M and Lsum hold the row-0 reductions (valid in lanes 0..15): broadcast
    // them from lane 0; row rq keeps head rq and merges the round into its
    // running (max, sum, o)
    float m_r = wave_bcast0(M[0]), l_r = wave_bcast0(Lsum[0]);
#pragma unroll
    for (int h = 1; h < G; ++h) {
      const float mh = wave_bcast0(M[h]);
      const float lh = wave_bcast0(Lsum[h]);
      if (rq == h) {
        m_r = mh;
        l_r = lh;
      }
    }
    const float m_new = fmaxf(m_me, m_r);
    if (m_new != -INFINITY) {
      const float so = __builtin_amdgcn_exp2f(m_me - m_new);
      const float sr = __builtin_amdgcn_exp2f(m_r - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) mine[e] = mine[e] * so + (acc[e][0] + acc[e][1]) * sr;
      l_me = l_me * so + l_r * sr;
      m_me = m_new;
    }
  }  // rounds
  if (nw > 1) {
    // merge the workgroup's waves in LDS (log-sum-exp); thread t of the
    // workgroup then owns output (head t / D, dim t % D)
    if (rq < G) {
      float* so = &s_o[wave][rq][8 * n];
      *reinterpret_cast<float4*>(so) = make_float4(mine[0], mine[1], mine[2], mine[3]);
      *reinterpret_cast<float4*>(so + 4) = make_float4(mine[4], mine[5], mine[6], mine[7]);
      if (n == 0) {
        s_ml[wave][0][rq] = m_me;
        s_ml[wave][1][rq] = l_me;
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * D; t += 64 * nw) {
      const int h = t / D;
      const int dim = t % D;
      float Mx = -INFINITY;
      for (int w = 0; w < nw; ++w) Mx = fmaxf(Mx, s_ml[w][0][h]);
      float Lx = 0.0f, Ox = 0.0f;
      if (Mx != -INFINITY) {
        for (int w = 0; w < nw; ++w) {
          const float wt = __builtin_amdgcn_exp2f(s_ml[w][0][h] - Mx);
          Lx = fmaf(s_ml[w][1][h], wt, Lx);
          Ox = fmaf(s_o[w][h][dim], wt, Ox);
        }
      }
      if (a.nsplit == 1) {
        a.out[((int64_t)b * a.Hq + (int64_t)r * G + h) * D + dim] = Ox / Lx;
      } else {
        float* p = a.part + ((int64_t)row * a.nsplit + split) * (G * (D + 2));
        p[h * D + dim] = Ox;
        if (dim == 0) {
          p[G * D + h] = Mx;
          p[G * D + G + h] = Lx;
        }
      }
    }
    return;
  }
  if (rq < G) {
    if (a.nsplit == 1) {
      float* dst = a.out + ((int64_t)b * a.Hq + (int64_t)r * G + rq) * D + 8 * n;
      const float inv = 1.0f / l_me;
      *reinterpret_cast<float4*>(dst) =
          make_float4(mine[0] * inv, mine[1] * inv, mine[2] * inv, mine[3] * inv);
      *reinterpret_cast<float4*>(dst + 4) =
          make_float4(mine[4] * inv, mine[5] * inv, mine[6] * inv, mine[7] * inv);
    } else {
      // partial layout per head: [half][n][4] -> dims 8n + 4*half + j
      float* p = a.part + ((int64_t)row * a.nsplit + split) * (G * (D + 2));
      float* ph = p + rq * D + 4 * n;
      *reinterpret_cast<float4*>(ph) = make_float4(mine[0], mine[1], mine[2], mine[3]);
      *reinterpret_cast<float4*>(ph + 64) = make_float4(mine[4], mine[5], mine[6], mine[7]);
      if (n == 0) {
        p[G * D + rq] = m_me;
        p[G * D + G + rq] = l_me;
      }
    }
  }
}


template <int G, int MODE, int TILES>
__global__ __launch_bounds__(64 * max_waves<MODE>()) void attend_sparse_kernel(AttendArgs a) {
  __shared__ __align__(16) AttendLds<G, TILES> lds;
  attend_sparse_body<G, MODE, TILES, false>(a, nullptr, lds);
}

// ---------------------------------------------------------------------------
// Selected-token gather-attend, pipelined by pairs of 16-slot tiles.
//
// A wave owns up to 32 * PAIRS consecutive slots.  It requests every index,
// then the key rows of all its slots, then their value rows, all at once,
// and consumes them in that order: the logits of every pair as its keys
// arrive, one softmax over all of the wave's slots, then P.V pair by pair as
// the values arrive -- so only P.V follows the last row's arrival.
//
// Per pair, Q.K gives each tile's logits in MFMA rows 0..3 (lanes 0..15);
// one lane-row swap then puts the second tile's in lanes 16..31, so the
// softmax runs on 32 lanes.  Its reference per head is the maximum of the
// wave's logits, so exp2(logit - reference) <= 1 and nothing is rescaled.
// P.V runs on MFMA as in the kernel above (P as a truncated bf16 pair hi +
// lo, V columns assembled from the lane's own value rows by byte permutes),
// and the row sums are one more MFMA of the same P against a B of ones.
constexpr int kMaxPairWaves = 12;
constexpr int kChipCUs = 256;  // MI355X compute units

// Position of 16-byte chunk x (dims [8x, 8x + 8)) of token t in a wave's
// key tile: one row of the 16 tokens per chunk, rows padded to 272 bytes, so
// the 16 lanes that store chunk n of one token each (row stride 272 = 16 mod
// 256) and the 16 lanes that load one chunk of 16 tokens (consecutive) both
// touch 16 different bank groups, and every store and load of a lane is one
// base address plus a constant.
constexpr int kKtRow = 16 * 16 + 16;
__device__ __forceinline__ int kt_pos(int t, int x) { return x * kKtRow + 16 * t; }

template <int G>
struct PairLds {
  // per wave: one tile of keys on its way to the MFMA layout (kt_pos),
  // later the wave's O rows for the merge of the waves
  union Wave {
    alignas(16) uint8_t kt[16 * kKtRow];
    alignas(16) float o[G][128];
  };
  Wave w[kMaxPairWaves];
  alignas(16) uint8_t q[4 * 256];                     // the row's G query heads, bf16
  alignas(16) float s_p[kMaxPairWaves][G][2][4][4];  // p of head h, tile, g, u (token 4u + g)
  alignas(16) float s_zero[8];                        // A rows that carry no head
  float s_m[4][kMaxPairWaves];                        // merge: reference of head h, wave w
  float s_l[4][kMaxPairWaves];                        // merge: sum of head h, wave w
};


__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Order-preserving integer key of a float that is not NaN (a larger float
// has a larger key, -0 just below +0), and back: a max over lanes then runs
// as integer DPP maxes, which need no quieting of their float operands.
__device__ __forceinline__ int ordered_key(float f) {
  const int s = __float_as_int(f);
  return s ^ ((s >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float ordered_float(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}

// Maximum of x over lanes 0..31 (two rows of 16), x finite or -inf.
__device__ __forceinline__ float max_lanes32(float x) {
  int k = ordered_key(x);
  k = max(k, dpp_i<kQuadXor1>(k));
  k = max(k, dpp_i<kQuadXor2>(k));
  k = max(k, dpp_i<kRowHalfMirror>(k));
  k = max(k, dpp_i<kRowMirror>(k));
  return ordered_float(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)));
}

// VH = 1: the workgroup computes all head_dim output dimensions of its slot
// range.  VH = 2: two workgroups share a whole row, each computing the
// output of one half of the value dimensions over all of the row's slots:
// both read every selected key row and the half of every value row they
// need, compute the same softmax, and write disjoint halves of the output --
// no partial results cross workgroups.
template <int G, int MODE, int PAIRS, bool LIDX, int VH>
__device__ __forceinline__ void attend_pairs_body(const AttendArgs& a, const int32_t* lidx,
                                                  PairLds<G>& lds, int row, int split, int half) {
  static_assert(G >= 1 && G <= 4, "query heads of a group fit MFMA rows 0..3");
  static_assert(VH == 1 || VH == 2, "whole rows or value halves");
  constexpr int D = 128;
  constexpr int DV = D / VH;    // value dimensions of this workgroup
  constexpr int NE = 8 / VH;    // P.V MFMAs per pair (16 dimensions each)
  constexpr int VW = 4 / VH;    // 32-bit words of a lane's value piece
  constexpr int TILES = 2 * PAIRS;
  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int rq = lane >> 4;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const int64_t wg0 = (int64_t)split * a.chunk;
  const int64_t wg1 = min(wg0 + (int64_t)a.chunk, a.n_slots);
  const int64_t s0 = wg0 + (int64_t)wave * 32 * PAIRS;
  const int64_t s1 = min(s0 + 32 * PAIRS, wg1);

  float m_me = -INFINITY, l_me = 0.0f;
  float mine[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) mine[e] = 0.0f;
  if (lane < 8) lds.s_zero[lane] = 0.0f;
  // Where this workgroup writes its result (head 0); a word of it is read
  // early (see below), so the page's address translation is in place when
  // the result is stored at the very end (a translation miss there would
  // follow the last row's arrival).  The value read is never used.
  float* const dst_row = a.nsplit == 1
                             ? a.out + ((int64_t)b * a.Hq + (int64_t)r * G) * D + half * DV
                             : a.part + ((int64_t)row * a.nsplit + split) * (G * (D + 2));
  float touch = 0.0f;
  if (s0 < wg1) {  // uniform: the wave has slots
    // the row's G query heads (G * 256 bytes) straight into LDS, first of
    // all loads, so any later wait for key rows covers it; every wave of the
    // workgroup writes the same bytes.  Lane l copies bytes [16l, +16)
    // (lanes past the heads copy the last 16 bytes again).
    {
      const int qb = min(16 * lane, G * 256 - 16);
      __builtin_amdgcn_global_load_lds(
          static_cast<const uint8_t*>(a.q) + ((int64_t)b * a.Hq + (int64_t)r * G) * D * 2 + qb,
          reinterpret_cast<__attribute__((address_space(3))) void*>(
              reinterpret_cast<uintptr_t>(lds.q)),
          16, 0, 0);
    }
    // the row's keys and values as buffer resources over its N tokens: a
    // token's rows sit at byte offset token * row_bytes, and an offset past
    // the row reads zeros instead of leaving the cache
    const int64_t kv_off = ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh) * 2;
    const uint32_t row_bytes = (uint32_t)(a.st * 2);
    const uint32_t nrec = a.row_span;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.k + kv_off), (short)0, nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.v + kv_off), (short)0, nrec, kBufferFlags);

    // 1. token of slot 16i + n of every tile, as a byte offset
    uint32_t toff[TILES];
#pragma unroll
    for (int i = 0; i < TILES; ++i) {
      bool ok_unused;
      toff[i] = (uint32_t)slot_token<MODE, LIDX>(a, row, b, s0 + 16 * i + n, s1, ok_unused, lidx) *
                row_bytes;
    }
    // 2. the key row pieces of every tile, then the value row pieces of every
    //    tile, of token 4u + rq of the tile (load u): lane (n, rq) reads key
    //    bytes [16n, +16) and value bytes [DV*2*half + 16n/VH, +16/VH), so
    //    every 8 (values of a half: 16) lanes read one whole 128-byte line.
    //    Keys first: the logits and the softmax of all pairs need only keys,
    //    so they run while the values arrive, and only P.V follows them.
    uint32_t base[TILES][4];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) base[i][u] = (uint32_t)__shfl((int)toff[i], 4 * u + rq);
    uint4 kl[TILES][4];
    uint32_t vw[TILES][4][VW];
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) kl[i][u] = ld16_buf(rk, base[i][u] + 16 * n);
#pragma unroll
    for (int i = 0; i < TILES; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (VH == 1) {
          const uint4 x = ld16_buf(rv, base[i][u] + 16 * n);
          vw[i][u][0] = x.x;
          vw[i][u][1] = x.y;
          vw[i][u][2] = x.z;
          vw[i][u][3] = x.w;
        } else {
          const uint2 x = ld8_buf(rv, base[i][u] + DV * 2 * half + 8 * n);
          vw[i][u][0] = x.x;
          vw[i][u][1] = x.y;
        }
      }
    // after the rows, so no wait for a row waits for it (a per-lane address:
    // a vector load, counted with the rows)
    touch = dst_row[lane];
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const kt = lds.w[wave].kt;

    float mref[G];
    f32x4_t oacc[NE];
    // row sums on the matrix cores: P times a B of ones gives, in lane
    // (n, rq), the sums of A rows 4rq (hi) and 4rq + 1 (lo) of head rq
    f32x4_t lacc = {0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8_t ones;
    {
      const uint32_t o1[4] = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
      __builtin_memcpy(&ones, o1, 16);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) oacc[e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int ha = n >> 2;  // A row n of P.V: head n / 4, part n % 4 (0 hi, 1 lo)
    const bool arow = (n & 3) < 2 && ha < G;
    const uint32_t lo_mask = (n & 3) == 1 ? 0xffff0000u : 0u;
    const float* pa0 = arow ? &lds.s_p[wave][ha < G ? ha : 0][0][rq][0] : lds.s_zero;
    const float* pa1 = arow ? pa0 + 16 : lds.s_zero + 4;

    // 3. logits of every pair: both tiles' (rows 0..G-1, lanes 0..15 of
    //    each result), then the second tile's rows moved to lanes 16..31:
    //    lanes 0..15 hold tile 2p, lanes 16..31 tile 2p + 1.
    //    Each tile goes through the wave's LDS tile: stored as loaded, read
    //    back as MFMA B fragments (lane (n, rq) of fragment c: token n, dims
    //    [32c + 8rq, +8), i.e. chunk 4c + rq).
    float xl[PAIRS][G];  // lane (n, rq < 2): logit of slot 32p + 16rq + n
    bf16x8_t qa[4];      // A fragments: q of head n % G, dims [32c + 8rq, +8)
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      // each pair's work stays after the previous pair's (it waits only for
      // its own keys)
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          *reinterpret_cast<uint4*>(kt + kt_pos(4 * u + rq, n)) = kl[2 * p + i][u];
        __builtin_amdgcn_wave_barrier();
        // lanes n >= G repeat a head; the result rows they produce, G..15,
        // are never read
        bf16x8_t kf[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 w = *reinterpret_cast<const uint4*>(kt + kt_pos(n, 4 * c + rq));
          __builtin_memcpy(&kf[c], &w, 16);
          if (p == 0 && i == 0) {  // the query fragments are the same for every tile
            const uint4 x = *reinterpret_cast<const uint4*>(lds.q + (n % G) * 256 + 64 * c + 16 * rq);
            __builtin_memcpy(&qa[c], &x, 16);
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (i == 0)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kf[c], acc, 0, 0, 0);
          else
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kf[c], acc1, 0, 0, 0);
        }
      }
      const bool vld = rq < 2 && s0 + 32 * p + 16 * rq + n < s1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // odd 16-lane rows of the first operand trade with even rows of the second
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[h]),
                                                         __float_as_uint(acc1[h]), false, false);
        xl[p][h] = vld ? __uint_as_float(sw[0]) * a.qscale : -INFINITY;
      }
    }
    // 4. the wave's reference per head: the maximum of its logits (finite:
    //    the wave has at least one slot), and the exponents against it
    float pv[PAIRS][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float x = xl[0][h];
#pragma unroll
      for (int p = 1; p < PAIRS; ++p) x = fmaxf(x, xl[p][h]);
      mref[h] = max_lanes32(x);
#pragma unroll
      for (int p = 0; p < PAIRS; ++p)
        pv[p][h] = __builtin_amdgcn_exp2f(xl[p][h] - mref[h]);  // exp2(-inf) = 0 for empty slots
    }
    // 5. P to the A fragments of P.V (slot 4u + g of tile j/4 is k index
    //    8g + 4(j/4) + u), every pair's before any P.V, so that only the
    //    value permutes and the P.V products wait for the values
    bf16x8_t a_p[PAIRS];
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      if (rq < 2) {
#pragma unroll
        for (int h = 0; h < G; ++h) lds.s_p[wave][h][rq][n & 3][n >> 2] = pv[p][h];
      }
      __builtin_amdgcn_wave_barrier();
      const float4 x0 = *reinterpret_cast<const float4*>(pa0);
      const float4 x1 = *reinterpret_cast<const float4*>(pa1);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t af[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // hi rows: p truncated to bf16; lo rows: the rest, truncated
        const uint32_t u0 = __float_as_uint(xs[2 * d]), u1 = __float_as_uint(xs[2 * d + 1]);
        const float w0 = xs[2 * d] - __uint_as_float(u0 & lo_mask);
        const float w1 = xs[2 * d + 1] - __uint_as_float(u1 & lo_mask);
        af[d] = __builtin_amdgcn_perm(__float_as_uint(w1), __float_as_uint(w0), 0x07060302u);
      }
      __builtin_memcpy(&a_p[p], af, 16);
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_p[p], ones, lacc, 0, 0, 0);
      // the next pair's P overwrites s_p: every lane has read this pair's
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int p = 0; p < PAIRS; ++p) {
      // each pair's P.V stays after the previous pair's (it waits only for
      // its own values)
      __builtin_amdgcn_sched_barrier(0);
      // 6. O += P.V: B fragment of lane (n, g) = value dim NE*n + e of the
      //    pair's slots 4u + g of both tiles, from this lane's own rows
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int wi = e >> 1;
        uint32_t bw[4];
        bw[0] = __builtin_amdgcn_perm(vw[2 * p][1][wi], vw[2 * p][0][wi], sel);
        bw[1] = __builtin_amdgcn_perm(vw[2 * p][3][wi], vw[2 * p][2][wi], sel);
        bw[2] = __builtin_amdgcn_perm(vw[2 * p + 1][1][wi], vw[2 * p + 1][0][wi], sel);
        bw[3] = __builtin_amdgcn_perm(vw[2 * p + 1][3][wi], vw[2 * p + 1][2][wi], sel);
        bf16x8_t bv;
        __builtin_memcpy(&bv, bw, 16);
        oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_p[p], bv, oacc[e], 0, 0, 0);
      }
    }
    // the wave's (reference, sum) of head rq and its O rows
    float m_r = mref[0];
#pragma unroll
    for (int h = 1; h < G; ++h)
      if (rq == h) m_r = mref[h];
    m_me = m_r;
    l_me = lacc[0] + lacc[1];
#pragma unroll
    for (int e = 0; e < NE; ++e) mine[e] = oacc[e][0] + oacc[e][1];
  }
  if (nw > 1) {
    // merge of the waves: every wave's O rows, reference and sum to LDS;
    // then wave h merges head h: lane j < nw takes wave j's reference and
    // sum, the head's reference M = their maximum, wave j's weight
    // 2^(m_j - M) (over L = the weighted sum of the sums when the result is
    // final), and lane d sums value dimension d of the rows, weighted
    __builtin_amdgcn_wave_barrier();  // the wave's key-tile reads are done
    if (rq < G) {
      float* so = &lds.w[wave].o[rq][NE * n];
#pragma unroll
      for (int e = 0; e < NE; e += 4)
        *reinterpret_cast<float4*>(so + e) = make_float4(mine[e], mine[e + 1], mine[e + 2], mine[e + 3]);
      if (n == 0) {
        lds.s_m[rq][wave] = m_me;
        lds.s_l[rq][wave] = l_me;
      }
    }
    __syncthreads();
    for (int h = wave; h < G; h += nw) {
      const bool in = lane < nw;
      const float mj = in ? lds.s_m[h][in ? lane : 0] : -INFINITY;
      const float lj = in ? lds.s_l[h][in ? lane : 0] : 0.0f;
      // lanes 0..15 hold every wave (nw <= 12): row 0's maximum and sum
      int kx = ordered_key(mj);
      kx = max(kx, dpp_i<kQuadXor1>(kx));
      kx = max(kx, dpp_i<kQuadXor2>(kx));
      kx = max(kx, dpp_i<kRowHalfMirror>(kx));
      kx = max(kx, dpp_i<kRowMirror>(kx));
      const float M = ordered_float(__builtin_amdgcn_readlane(kx, 0));  // finite: wave 0 has slots
      const float wt = mj == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mj - M);
      const float L = lane_f(group_sum<16>(wt * lj), 0);
      const float wn = a.nsplit == 1 ? wt / L : wt;
      float wj[kMaxPairWaves];
#pragma unroll
      for (int j = 0; j < kMaxPairWaves; ++j) wj[j] = lane_f(wn, j);
      for (int d = lane; d < DV; d += 64) {
        float Ox = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxPairWaves; ++j) {
          const float o = lds.w[j].o[h][d];  // slots past the waves: dropped
          Ox = fmaf(j < nw ? o : 0.0f, wj[j], Ox);
        }
        dst_row[h * D + d] = Ox;
      }
      if (a.nsplit > 1 && lane == 0) {
        dst_row[G * D + h] = M;
        dst_row[G * D + G + h] = L;
      }
    }
    if (touch == 1.0f && a.n_slots < 0) dst_row[1] = 0.0f;  // never true: keeps the read
    return;
  }
  if (rq < G) {
    float* dst = dst_row + rq * D + NE * n;
    if (a.nsplit == 1) {
      const float inv = 1.0f / l_me;
#pragma unroll
      for (int e = 0; e < NE; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(mine[e] * inv, mine[e + 1] * inv, mine[e + 2] * inv, mine[e + 3] * inv);
    } else {
#pragma unroll
      for (int e = 0; e < NE; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(mine[e], mine[e + 1], mine[e + 2], mine[e + 3]);
      if (n == 0) {
        dst_row[G * D + rq] = m_me;
        dst_row[G * D + G + rq] = l_me;
      }
    }
  }
  if (touch == 1.0f && a.n_slots < 0) dst_row[1] = 0.0f;  // never true: keeps the read
}

// Workgroup -> (row, split, value half).  With value halves the grid is 1-D
// and the two halves of a row are workgroups id and id + 8 of each group of
// 16: workgroups are dispatched to the chip's 8 XCDs in turn, so both land on
// the same XCD and the second reading of a key row finds it in that XCD's L2
// (only a matter of speed: the halves exchange nothing).
template <int VH>
__device__ __forceinline__ bool pairs_coords(const AttendArgs& a, int& row, int& split, int& half) {
  if constexpr (VH == 2) {
    const int id = blockIdx.x;
    half = (id >> 3) & 1;
    row = (id >> 4) * 8 + (id & 7);
    split = 0;
    return row < a.rows;
  } else {
    row = blockIdx.y;
    split = blockIdx.x;
    half = 0;
    return true;
  }
}

template <int G, int MODE, int PAIRS, int VH>
__global__ __launch_bounds__(64 * kMaxPairWaves) void attend_pairs_kernel(AttendArgs a) {
  __shared__ __align__(16) PairLds<G> lds;
  int row, split, half;
  if (!pairs_coords<VH>(a, row, split, half)) return;
  attend_pairs_body<G, MODE, PAIRS, false, VH>(a, nullptr, lds, row, split, half);
}

// The reads of attend_pairs_kernel without its arithmetic (a measurement
// reference, not a step of the method): the same grid, the same slots per
// wave, the same index loads and the same key and value row loads in the
// same order (whole 128-byte lines, nontemporal buffer loads, every key row
// before the value rows), folded with XOR; the fold is
// stored only if it equals a constant it practically never equals.  Its
// duration is what reading the selected rows alone takes on this device.
template <int MODE, int PAIRS, int VH>
__global__ __launch_bounds__(64 * kMaxPairWaves) void gather_read_kernel(AttendArgs a,
                                                                         uint32_t* sink) {
  constexpr int D = 128;
  constexpr int DV = D / VH;
  constexpr int TILES = 2 * PAIRS;
  int row, split, half;
  if (!pairs_coords<VH>(a, row, split, half)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int rq = lane >> 4;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const int64_t wg0 = (int64_t)split * a.chunk;
  const int64_t wg1 = min(wg0 + (int64_t)a.chunk, a.n_slots);
  const int64_t s0 = wg0 + (int64_t)wave * 32 * PAIRS;
  const int64_t s1 = min(s0 + 32 * PAIRS, wg1);
  if (s0 >= wg1) return;
  const int64_t kv_off = ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh) * 2;
  const uint32_t row_bytes = (uint32_t)(a.st * 2);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.k + kv_off), (short)0, a.row_span, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.v + kv_off), (short)0, a.row_span, kBufferFlags);
  uint32_t toff[TILES];
#pragma unroll
  for (int i = 0; i < TILES; ++i) {
    bool ok_unused;
    toff[i] = (uint32_t)slot_token<MODE, false>(a, row, b, s0 + 16 * i + n, s1, ok_unused) *
              row_bytes;
  }
  // the key rows of every tile, then the value rows, as the attend requests them
  uint32_t base[TILES][4];
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) base[i][u] = (uint32_t)__shfl((int)toff[i], 4 * u + rq);
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 k = ld16_buf(rk, base[i][u] + 16 * n);
      acc ^= k.x ^ k.y ^ k.z ^ k.w;
    }
#pragma unroll
  for (int i = 0; i < TILES; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (VH == 1) {
        const uint4 x = ld16_buf(rv, base[i][u] + 16 * n);
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
      } else {
        const uint2 x = ld8_buf(rv, base[i][u] + DV * 2 * half + 8 * n);
        acc ^= x.x ^ x.y;
      }
    }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <int PAIRS, int VH>
hipError_t dispatch_gather_read(int mode, dim3 grid, dim3 block, const AttendArgs& a, uint32_t* sink,
                                hipStream_t s) {
  if (mode == kIdxTokenShared)
    hipLaunchKernelGGL((gather_read_kernel<kIdxTokenShared, PAIRS, VH>), grid, block, 0, s, a, sink);
  else if (mode == kIdxBlockPerHead)
    hipLaunchKernelGGL((gather_read_kernel<kIdxBlockPerHead, PAIRS, VH>), grid, block, 0, s, a, sink);
  else
    hipLaunchKernelGGL((gather_read_kernel<kIdxTokenPerHead, PAIRS, VH>), grid, block, 0, s, a, sink);
  return hipGetLastError();
}

// Merge, then gather-attend, in one workgroup of kMaxSparseWaves waves per
// row: the register top-k of the selection's merge picks the row's k tokens
// from its parts' (score, position) candidates, writes them to the index
// list and to LDS, and the waves attend over them from LDS -- the same
// index list and the same per-wave work as the merge launch followed by the
// whole-row pair-pipelined gather-attend launch, without the launch between
// them and without reading the index list back from memory.
template <int G, int PAIRS, int GK, int VH>
__global__ __launch_bounds__(64 * kMaxSparseWaves) void merge_attend_kernel(
    AttendArgs a, const float* __restrict__ cand_val, const int32_t* __restrict__ cand_pos,
    int n_cand, int64_t cstride, bool vec4, int32_t* __restrict__ idx_out) {
  constexpr int NT = 64 * kMaxSparseWaves;
  __shared__ SharedT<NT> sh;
  __shared__ __align__(16) uint2 cand[kRankMax + 8];
  __shared__ uint32_t s_wave[NT / 64];
  __shared__ __align__(16) int32_t s_map[4 * GK * NT];
  __shared__ int32_t s_idx[64 * kMaxSparseWaves];
  __shared__ __align__(16) PairLds<G> lds;
  int row, split, half;
  if (!pairs_coords<VH>(a, row, split, half)) return;
  const int n = n_cand;  // <= 4 * GK * NT
  const int32_t k = a.n_idx;
  const float* __restrict__ sv = cand_val + (int64_t)row * cstride;
  const int32_t* __restrict__ map = cand_pos + (int64_t)row * cstride;
  int32_t* __restrict__ out = idx_out + (int64_t)row * k;
  auto load = [&](int p0, float (&v)[GK][4]) {
    if (vec4 && n % 4 == 0) {
      // a group of four lies wholly inside or wholly outside the row
      const float4* s4 = reinterpret_cast<const float4*>(sv + p0);
      int4 m[GK];
#pragma unroll
      for (int j = 0; j < GK; ++j) {
        const bool in = p0 + 256 * j < n;
        const float4 f = in ? s4[64 * j] : make_float4(0.f, 0.f, 0.f, 0.f);
        m[j] = in ? reinterpret_cast<const int4*>(map + p0)[64 * j] : make_int4(0, 0, 0, 0);
        v[j][0] = f.x;
        v[j][1] = f.y;
        v[j][2] = f.z;
        v[j][3] = f.w;
      }
#pragma unroll
      for (int j = 0; j < GK; ++j) *reinterpret_cast<int4*>(&s_map[p0 + 256 * j]) = m[j];
    } else {
#pragma unroll
      for (int j = 0; j < GK; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = p0 + 256 * j + e;
          const bool in = i < n;
          v[j][e] = in ? sv[i] : 0.0f;
          if (in) s_map[i] = map[i];
        }
    }
  };
  // s_map is complete before the ordered write: reg_row_topk passes several
  // barriers between the load and the write
  // with value halves both workgroups of a row select (the same list);
  // half 0 writes it
  auto emit = [&](uint32_t slot, int32_t p) {
    const int32_t t = s_map[p];
    if (half == 0) out[slot] = t;
    s_idx[slot] = t;
  };
  reg_row_topk<NT, GK, false>(load, n, k, emit, sh, cand, s_wave);
  __syncthreads();
  attend_pairs_body<G, kIdxTokenPerHead, PAIRS, true, VH>(a, s_idx, lds, row, split, half);
}

// ---------------------------------------------------------------------------
// Combine: the nsplit partials (o, m, l) of one (row, query head) merged
// with a log-sum-exp.  A workgroup covers 32 output dimensions of one
// (row, head) with SL lanes per dimension: lane j merges splits j, j + SL,
// j + 2 SL, ..., sixteen at a time with all their loads independent, so a
// row of 512 splits is one round of loads at SL = 32 instead of 32 rounds
// one after another; the SL running (m, l, o) are then merged in LDS.
template <int SL>
__global__ __launch_bounds__(32 * SL) void combine_kernel(const float* __restrict__ part, int nsplit,
                                                         int G, int D, int Hq, int Hkv,
                                                         float* __restrict__ out, bool vec_layout) {
  constexpr int K = 16;
  __shared__ float s_m[SL][32], s_l[SL][32], s_o[SL][32];
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 31;
  const int j = threadIdx.x >> 5;
  const int dim = blockIdx.z * 32 + lane;
  const int PS = G * (D + 2);
  const float* pr = part + (int64_t)row * nsplit * PS;
  // where dim lives inside a partial's head block: dim itself, or (sparse
  // one-wave kernel) [half][n][4] with dim = 8n + 4 half + j
  const int pos = vec_layout ? ((dim & 7) >> 2) * 64 + (dim >> 3) * 4 + (dim & 3) : dim;
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int s0 = j; s0 < nsplit; s0 += K * SL) {
    float ov[K], mv[K], lv[K];
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const int sp = s0 + u * SL;
      const bool ok = sp < nsplit;
      const float* ps = pr + (int64_t)sp * PS;
      ov[u] = ok ? ps[h * D + pos] : 0.0f;
      mv[u] = ok ? ps[G * D + h] : -INFINITY;
      lv[u] = ok ? ps[G * D + G + h] : 0.0f;
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < K; ++u) mn = fmaxf(mn, mv[u]);
    if (mn == -INFINITY) continue;
    const float alpha = exp2f(M - mn);
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const float w = exp2f(mv[u] - mn);
      L = fmaf(lv[u], w, L);
      O = fmaf(ov[u], w, O);
    }
    M = mn;
  }
  s_m[j][lane] = M;
  s_l[j][lane] = L;
  s_o[j][lane] = O;
  __syncthreads();
  if (j != 0) return;
  float mn = -INFINITY;
#pragma unroll
  for (int i = 0; i < SL; ++i) mn = fmaxf(mn, s_m[i][lane]);
  float Lt = 0.0f, Ot = 0.0f;
  if (mn != -INFINITY) {
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const float w = exp2f(s_m[i][lane] - mn);
      Lt = fmaf(s_l[i][lane], w, Lt);
      Ot = fmaf(s_o[i][lane], w, Ot);
    }
  }
  const int b = row / Hkv;
  const int r = row % Hkv;
  out[((int64_t)b * Hq + (int64_t)r * G + h) * D + dim] = Ot / Lt;
}

// ---------------------------------------------------------------------------
template <typename KT, int D, int G>
hipError_t dispatch_mode(int mode, dim3 grid, const AttendArgs& a, hipStream_t s) {
  switch (mode) {
    case kIdxTokenPerHead:
      hipLaunchKernelGGL((attend_kernel<KT, D, G, kIdxTokenPerHead>), grid, dim3(kThreads), 0, s, a);
      break;
    case kIdxTokenShared:
      hipLaunchKernelGGL((attend_kernel<KT, D, G, kIdxTokenShared>), grid, dim3(kThreads), 0, s, a);
      break;
    case kIdxBlockPerHead:
      hipLaunchKernelGGL((attend_kernel<KT, D, G, kIdxBlockPerHead>), grid, dim3(kThreads), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((attend_kernel<KT, D, G, kIdxDense>), grid, dim3(kThreads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

template <typename KT, int D>
hipError_t dispatch_group(int G, int mode, dim3 grid, const AttendArgs& a, hipStream_t s) {
  switch (G) {
    case 1: return dispatch_mode<KT, D, 1>(mode, grid, a, s);
    case 2: return dispatch_mode<KT, D, 2>(mode, grid, a, s);
    case 4: return dispatch_mode<KT, D, 4>(mode, grid, a, s);
    default: return dispatch_mode<KT, D, 8>(mode, grid, a, s);
  }
}

template <int G, int TILES>
hipError_t dispatch_sparse(int waves, int mode, dim3 grid, const AttendArgs& a, hipStream_t s) {
  const dim3 block(64 * waves);
  switch (mode) {
    case kIdxTokenPerHead:
      hipLaunchKernelGGL((attend_sparse_kernel<G, kIdxTokenPerHead, TILES>), grid, block, 0, s, a);
      break;
    case kIdxTokenShared:
      hipLaunchKernelGGL((attend_sparse_kernel<G, kIdxTokenShared, TILES>), grid, block, 0, s, a);
      break;
    case kIdxBlockPerHead:
      hipLaunchKernelGGL((attend_sparse_kernel<G, kIdxBlockPerHead, TILES>), grid, block, 0, s, a);
      break;
    case kIdxDenseScored:
      hipLaunchKernelGGL((attend_sparse_kernel<G, kIdxDenseScored, TILES>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((attend_sparse_kernel<G, kIdxDense, TILES>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

// The gather kernel with `waves` waves of chunk / (waves * rounds) slots per
// round.
template <int G>
hipError_t dispatch_wave(int waves, int rounds, int chunk, int mode, dim3 grid,
                         const AttendArgs& a, hipStream_t s) {
  const int per_wave = chunk / (waves * rounds);
  if (per_wave <= 16) return dispatch_sparse<G, 1>(waves, mode, grid, a, s);
  if (per_wave <= 32) return dispatch_sparse<G, 2>(waves, mode, grid, a, s);
  if (per_wave <= 48) return dispatch_sparse<G, 3>(waves, mode, grid, a, s);
  return dispatch_sparse<G, 4>(waves, mode, grid, a, s);
}

template <int G, int PAIRS, int VH>
hipError_t dispatch_pairs_mode(int mode, dim3 grid, dim3 block, const AttendArgs& a,
                               hipStream_t s) {
  if (mode == kIdxTokenShared)
    hipLaunchKernelGGL((attend_pairs_kernel<G, kIdxTokenShared, PAIRS, VH>), grid, block, 0, s, a);
  else if (mode == kIdxBlockPerHead)
    hipLaunchKernelGGL((attend_pairs_kernel<G, kIdxBlockPerHead, PAIRS, VH>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attend_pairs_kernel<G, kIdxTokenPerHead, PAIRS, VH>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Grid of a pair plan: (nsplit, rows), or with value halves one workgroup
// per (row, half) in groups of 16 (8 rows, both halves; pairs_coords).
dim3 pairs_grid(const AttendPlan& p, int64_t rows) {
  if (p.vhalves == 2) return dim3((unsigned)(16 * ((rows + 7) / 8)));
  return dim3((unsigned)p.nsplit, (unsigned)rows);
}

template <int G>
hipError_t dispatch_pairs(const AttendPlan& p, int64_t rows, const AttendArgs& a, hipStream_t s) {
  const dim3 block(64 * p.waves), grid = pairs_grid(p, rows);
  if (p.vhalves == 2)
    return p.pairs == 1 ? dispatch_pairs_mode<G, 1, 2>(p.mode, grid, block, a, s)
                        : dispatch_pairs_mode<G, 2, 2>(p.mode, grid, block, a, s);
  return p.pairs == 1 ? dispatch_pairs_mode<G, 1, 1>(p.mode, grid, block, a, s)
                      : dispatch_pairs_mode<G, 2, 1>(p.mode, grid, block, a, s);
}

bool use_wave_kernel(const Cache& c) {
  return c.kv_dtype == SA_BF16 && c.q_dtype == SA_BF16 && c.D == 128 && c.G <= 4;
}

// Bytes from a row's first token to the end of its last one: the range its
// gathered K/V rows lie in.
int64_t row_span_bytes(const Cache& c) {
  return ((c.N - 1) * c.st + c.D) * (c.kv_dtype == SA_BF16 ? 2 : 4);
}

int lanes_per_row(const Cache& c) { return c.D * (c.kv_dtype == SA_BF16 ? 2 : 4) / 16; }

}  // namespace

AttendPlan plan_attend(const Cache& c, int mode, int32_t n_idx, int32_t bs) {
  AttendPlan p{};
  p.mode = mode;
  if (is_dense_mode(mode)) {
    p.n_slots = c.N;
  } else if (mode == kIdxBlockPerHead) {
    p.n_slots = (int64_t)n_idx * bs;
  } else {
    p.n_slots = n_idx;
  }
  const int64_t rows = (int64_t)c.B * c.Hkv;
  int64_t chunk;
  p.pairs = 0;
  // (selected blocks: only when every block is whole, as the pair kernel
  // masks slots, not tokens past the end)
  const bool pair_mode = mode == kIdxTokenPerHead || mode == kIdxTokenShared ||
                         (mode == kIdxBlockPerHead && c.N % bs == 0);
  if (use_wave_kernel(c) && pair_mode && row_span_bytes(c) < (int64_t(1) << 32)) {
    // Selected tokens: waves of one or two pairs of 16-slot tiles.  At least
    // 128 rows (half the chip's CUs at one workgroup each) and at most 24
    // pairs: one workgroup takes a whole row, so no split partials and no
    // combine launch; one pair per wave while 12 waves hold the row, else
    // two.  Otherwise rows split so that about 512 workgroups run, and a
    // combine launch merges the splits.
    p.kernel = kKernPairs;
    p.rounds = 1;
    const int64_t np = (p.n_slots + 31) / 32;
    int waves, pairs;
    if (rows >= 128 && np <= 2 * kMaxPairWaves) {
      pairs = np <= kMaxPairWaves ? 1 : 2;
      waves = (int)((np + pairs - 1) / pairs);
    } else {
      pairs = 2;
      waves = 0;
      // The widest workgroups whose splits run in one round that fills at
      // least 3/4 of the chip's wave slots (at two pairs per wave a CU holds
      // 12 waves): fewest splits for the combine, no second round
      // (block61k's 64 rows of 96 pairs: 256 workgroups of 12 waves, 23.5 us
      // against 24.2 us for 768 of 4).
      for (int w : {12, 8, 4, 2, 1}) {
        const int64_t wgs = rows * ((np + 2 * w - 1) / (2 * w));
        if (4 * wgs * w >= 3 * (int64_t)kChipCUs * kMaxPairWaves &&
            wgs <= (int64_t)kChipCUs * (kMaxPairWaves / w)) {
          waves = w;
          break;
        }
      }
      // else about 512 workgroups
      for (int w : {12, 8, 4, 2, 1}) {
        if (waves != 0) break;
        if (rows * ((np + 2 * w - 1) / (2 * w)) >= 512) waves = w;
      }
      if (waves == 0) {
        waves = 1;
        pairs = 1;
      }
      // no more waves than the row has pairs for
      while (waves > 1 && (int64_t)(waves - 1) * pairs >= np) --waves;
    }
    p.waves = waves;
    p.pairs = pairs;
    chunk = (int64_t)waves * pairs * 32;
    // Fewer whole rows than the chip has CUs: two workgroups per row, each
    // reading all the row's keys and half of each value row (the keys' second
    // reading is served by the XCD's L2), so twice as many CUs request the
    // rows.  On 128 rows of 655 slots the gather alone takes 9.0 us against
    // 9.7 us with one workgroup per row (cache-cold).
    p.vhalves = (chunk >= p.n_slots && rows < 256) ? 2 : 1;
  } else if (use_wave_kernel(c)) {
    p.kernel = kKernWave;
    // Each wave takes rounds of up to 64 slots with every load of a round in
    // flight at once; the waves of a workgroup merge in LDS.
    const int64_t wn = (p.n_slots + 63) / 64;
    int waves = 1, rounds = 1;
    int64_t per_wave = 64;
    if (rows >= 128 && wn <= kMaxSparseWaves && mode != kIdxDenseScored) {
      // At least 128 rows (half the chip's CUs at one workgroup each) and at
      // most 12 waves' worth of slots: one workgroup takes a whole row in one
      // round, so no split partials and no combine launch (on 128 rows of
      // 655 slots, 14.6 us against 14.2 us + 4.5 us for one-wave splits and
      // their combine).  The fewest slots per wave (32, 48 or 64) that still
      // fit: more, shorter waves finish sooner (on 1024 rows of 262 slots,
      // 9 x 32 beats 5 x 64 by 10 %).
      for (int pw : {32, 48, 64}) {
        if ((p.n_slots + pw - 1) / pw <= kMaxSparseWaves) {
          per_wave = pw;
          break;
        }
      }
      waves = (int)((p.n_slots + per_wave - 1) / per_wave);
    } else if (is_dense_mode(mode)) {
      // long contiguous scans: several rounds per wave merged online, so a
      // workgroup covers waves * rounds * 64 tokens and few split partials
      // are written.  4 waves, and the most rounds (at most 32) that still
      // give about 1024 workgroups: on 128 rows of 32768 tokens 16 rounds
      // (8 splits) take 320 us against 324.5 us for 8 rounds; on 8 rows of
      // 1M tokens 32 rounds (128 splits) 626 us against 649 us for 8 rounds
      // and 638 us for 64; 8 waves were no faster on either
      waves = 4;
      rounds = 32;
      // fewer rounds per wave until about 1024 workgroups run (64 rows of
      // 3072 tokens: 12 splits of 256 tokens, not 1 of 3072)
      while (rounds > 1 && rows * ((p.n_slots + 64 * waves * rounds - 1) / (64 * waves * rounds)) < 1024)
        rounds /= 2;
    } else {
      // selections split so that about 512 workgroups (two per CU) run; a
      // combine pass merges the splits
      for (int w : {12, 8, 4}) {
        if (rows * ((wn + w - 1) / w) >= 512) {
          waves = w;
          break;
        }
      }
      if (waves == 1)
        while (per_wave > 16 && rows * ((p.n_slots + per_wave - 1) / per_wave) < 512) per_wave /= 2;
    }
    p.waves = waves;
    p.rounds = rounds;
    chunk = per_wave * waves * rounds;
  } else {
    p.kernel = kKernGeneric;
    p.waves = 4;
    p.rounds = 1;
    const int64_t unit = (int64_t)(kThreads / lanes_per_row(c)) * kUnroll;
    chunk = (rows * p.n_slots + 4095) / 4096;
    chunk = (chunk + unit - 1) / unit * unit;
    chunk = std::max<int64_t>(unit, std::min<int64_t>(chunk, 256 * unit));
    while ((p.n_slots + chunk - 1) / chunk > 1024) chunk *= 2;
  }
  p.chunk = (int32_t)chunk;
  p.nsplit = (int32_t)((p.n_slots + chunk - 1) / chunk);
  p.ws_bytes = p.nsplit > 1 ? (size_t)rows * p.nsplit * c.G * (c.D + 2) * sizeof(float) : 0;
  return p;
}

bool fused_scores_supported(const Cache& c) { return use_wave_kernel(c); }

namespace {

AttendArgs attend_args(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                       const void* v, const int32_t* idx, int32_t n_idx, int32_t bs, float* out,
                       void* ws, float* scores) {
  AttendArgs a{};
  a.scores = scores;
  a.sscale = c.scale;
  a.q = q;
  a.q_dtype = c.q_dtype;
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.sb = c.sb;
  a.sh = c.sh;
  a.st = c.st;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.kv_div = c.kv_div;
  a.N = c.N;
  a.qscale = c.scale * kLog2e;
  a.idx = idx;
  a.n_idx = n_idx;
  a.bs = bs;
  a.n_slots = p.n_slots;
  a.chunk = p.chunk;
  a.nsplit = p.nsplit;
  a.rounds = p.rounds;
  a.out = out;
  a.part = static_cast<float*>(ws);
  a.row_span = p.kernel == kKernPairs ? (uint32_t)row_span_bytes(c) : 0u;
  a.rows = c.B * c.Hkv;
  return a;
}

}  // namespace

hipError_t launch_gather_read(const Cache& c, const AttendPlan& p, const void* k, const void* v,
                              const int32_t* idx, int32_t n_idx, int32_t bs, uint32_t* sink,
                              hipStream_t s) {
  const AttendArgs a = attend_args(c, p, nullptr, k, v, idx, n_idx, bs, nullptr, nullptr, nullptr);
  const int64_t rows = (int64_t)c.B * c.Hkv;
  const dim3 block(64 * p.waves), grid = pairs_grid(p, rows);
  if (p.vhalves == 2)
    return p.pairs == 1 ? dispatch_gather_read<1, 2>(p.mode, grid, block, a, sink, s)
                        : dispatch_gather_read<2, 2>(p.mode, grid, block, a, sink, s);
  return p.pairs == 1 ? dispatch_gather_read<1, 1>(p.mode, grid, block, a, sink, s)
                      : dispatch_gather_read<2, 1>(p.mode, grid, block, a, sink, s);
}

hipError_t launch_attend(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                         const void* v, const int32_t* idx, int32_t n_idx, int32_t bs, float* out,
                         void* ws, hipStream_t s, float* scores) {
  const AttendArgs a = attend_args(c, p, q, k, v, idx, n_idx, bs, out, ws, scores);
  const int64_t rows = (int64_t)c.B * c.Hkv;
  const dim3 grid(p.nsplit, (unsigned)rows);
  hipError_t e;
  if (p.kernel == kKernPairs) {
    switch (c.G) {
      case 1: e = dispatch_pairs<1>(p, rows, a, s); break;
      case 2: e = dispatch_pairs<2>(p, rows, a, s); break;
      default: e = dispatch_pairs<4>(p, rows, a, s); break;
    }
  } else if (p.kernel == kKernWave) {
    switch (c.G) {
      case 1: e = dispatch_wave<1>(p.waves, p.rounds, p.chunk, p.mode, grid, a, s); break;
      case 2: e = dispatch_wave<2>(p.waves, p.rounds, p.chunk, p.mode, grid, a, s); break;
      default: e = dispatch_wave<4>(p.waves, p.rounds, p.chunk, p.mode, grid, a, s); break;
    }
  } else if (c.kv_dtype == SA_BF16) {
    e = c.D == 64 ? dispatch_group<bf16_t, 64>(c.G, p.mode, grid, a, s)
                  : dispatch_group<bf16_t, 128>(c.G, p.mode, grid, a, s);
  } else {
    e = c.D == 64 ? dispatch_group<float, 64>(c.G, p.mode, grid, a, s)
                  : dispatch_group<float, 128>(c.G, p.mode, grid, a, s);
  }
  if (e != hipSuccess || p.nsplit == 1) return e;
  const dim3 cgrid((unsigned)rows, (unsigned)c.G, (unsigned)(c.D / 32));
  // one-wave workgroups of the round kernel write the interleaved partial
  // layout
  const bool vec_layout = p.kernel == kKernWave && p.waves == 1;
  // the fewest lanes per dimension that cover the splits in one round of
  // sixteen loads (at most 32)
  if (p.nsplit <= 64)
    hipLaunchKernelGGL(combine_kernel<4>, cgrid, dim3(128), 0, s, a.part, p.nsplit, c.G, c.D, c.Hq,
                       c.Hkv, out, vec_layout);
  else if (p.nsplit <= 128)
    hipLaunchKernelGGL(combine_kernel<8>, cgrid, dim3(256), 0, s, a.part, p.nsplit, c.G, c.D, c.Hq,
                       c.Hkv, out, vec_layout);
  else if (p.nsplit <= 256)
    hipLaunchKernelGGL(combine_kernel<16>, cgrid, dim3(512), 0, s, a.part, p.nsplit, c.G, c.D, c.Hq,
                       c.Hkv, out, vec_layout);
  else
    hipLaunchKernelGGL(combine_kernel<32>, cgrid, dim3(1024), 0, s, a.part, p.nsplit, c.G, c.D,
                       c.Hq, c.Hkv, out, vec_layout);
  return hipGetLastError();
}

namespace {

template <int G, int PAIRS, int VH>
hipError_t launch_merge_attend_g(const AttendArgs& a, const AttendPlan& p, int64_t rows,
                                 const float* cand_val, const int32_t* cand_pos, int64_t n_cand,
                                 int64_t cstride, bool vec4, int32_t* idx, hipStream_t s) {
  const dim3 grid = pairs_grid(p, rows), block(64 * kMaxSparseWaves);
  if (n_cand <= 4 * 64 * kMaxSparseWaves)
    hipLaunchKernelGGL((merge_attend_kernel<G, PAIRS, 1, VH>), grid, block, 0, s, a, cand_val,
                       cand_pos, (int)n_cand, cstride, vec4, idx);
  else
    hipLaunchKernelGGL((merge_attend_kernel<G, PAIRS, 2, VH>), grid, block, 0, s, a, cand_val,
                       cand_pos, (int)n_cand, cstride, vec4, idx);
  return hipGetLastError();
}

template <int G>
hipError_t launch_merge_attend_t(const AttendPlan& p, const AttendArgs& a, int64_t rows,
                                 const float* cand_val, const int32_t* cand_pos, int64_t n_cand,
                                 int64_t cstride, bool vec4, int32_t* idx, hipStream_t s) {
  if (p.vhalves == 2)
    return p.pairs == 1
               ? launch_merge_attend_g<G, 1, 2>(a, p, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s)
               : launch_merge_attend_g<G, 2, 2>(a, p, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s);
  return p.pairs == 1
             ? launch_merge_attend_g<G, 1, 1>(a, p, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s)
             : launch_merge_attend_g<G, 2, 1>(a, p, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s);
}

}  // namespace

bool merge_attend_ok(const Cache& c, const AttendPlan& p, int64_t n_cand, int32_t k) {
  // the merge's workgroup (kMaxSparseWaves waves) attends over the row as one
  // whole-row pair plan
  static_assert(kMaxSparseWaves == kMaxPairWaves, "merge and attend share the workgroup");
  return p.kernel == kKernPairs && p.mode == kIdxTokenPerHead && p.nsplit == 1 &&
         p.waves <= kMaxPairWaves && p.n_slots == k && k >= 1 && n_cand >= k &&
         n_cand <= 2 * 4 * 64 * kMaxSparseWaves && c.G <= 4;
}

hipError_t launch_merge_attend(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                               const void* v, float* out, const float* cand_val,
                               const int32_t* cand_pos, int64_t n_cand, int64_t cstride, int32_t kk,
                               int32_t* idx, hipStream_t s) {
  const AttendArgs a = attend_args(c, p, q, k, v, nullptr, kk, 0, out, nullptr, nullptr);
  const int64_t rows = (int64_t)c.B * c.Hkv;
  const bool vec4 = (reinterpret_cast<uintptr_t>(cand_val) % 16 == 0) && (cstride % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(cand_pos) % 16 == 0);
  switch (c.G) {
    case 1: return launch_merge_attend_t<1>(p, a, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s);
    case 2: return launch_merge_attend_t<2>(p, a, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s);
    default: return launch_merge_attend_t<4>(p, a, rows, cand_val, cand_pos, n_cand, cstride, vec4, idx, s);
  }
}

}  // namespace sa
