// Token and block scoring kernels.
//
//  * score_exact: exact score of every cached token of every (sequence, KV
//    head) row -- the "oracle top-k" selection criterion of "Inference-time
//    context sparsity: illusion or opportunity?" (section 2).  The G query
//    heads of a row are summed first (sum_g q_g . k = (sum_g q_g) . k), kept in
//    fp32, so one dot product per token streams the key cache once.
//  * block_summarize / score_block: per-128-token-block elementwise key
//    min/max and the block upper bound sum_i max(q_i kmin_i, q_i kmax_i),
//    summed over the group ("HyLRA" summary, section 2.4).  The kernel uses
//    max(q kmin, q kmax) = q+ kmax + q- kmin with q+ = max(q, 0), q- =
//    min(q, 0), which holds because kmin <= kmax, and folds the group sum into
//    Q+ = sum_g q_g+ and Q- = sum_g q_g-.
//  * score_indexer: the low-dimensional indexer of "Flash Attention vs Sparse
//    Attention" (DSA, Stage 1): sum_h w_h max(0, q_idx_h . k_idx_t).
//
// All kernels are HBM-streaming: a lane group of LPR lanes reads one cache row
// with 16-byte loads, reduces its dot product with DPP inside the group, and
// each wave covers a contiguous run of tokens so both loads and score stores
// are coalesced.  Score stores are nontemporal: stores mixed into the key
// stream cost far more than their bytes, less so when they bypass the caches.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "topk_core.hpp"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kScoreTile = 1024;  // tokens per workgroup of the exact score
constexpr int kIndexerHistTile = 4096;  // tokens per workgroup, indexer scores counting a histogram

// ------------------------------------------------------------ exact score

struct ExactArgs {
  const void* q;
  sa_dtype q_dtype;
  const uint8_t* k;
  int64_t sb, sh, st;
  int32_t Hq, Hkv, G;
  int32_t kv_div;  // row r reads KV head r / kv_div (1, or G for per-query-head rows)
  int64_t N;
  float scale;
  float* scores;
};

template <typename KT, int D, int U>
__global__ __launch_bounds__(kThreads) void score_exact_kernel(ExactArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int RPW = 64 / LPR;  // rows per wave load
  static_assert(U <= LPR, "one storing lane per unrolled token");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lg = (tid & 63) / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.y;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;

  // sum of the group's queries (G <= 8)
  float qs[E];
  group_query_sum<E, D>(a.q, a.q_dtype, (int64_t)b * a.Hq + (int64_t)r * a.G, a.G, sl * E, a.scale,
                        qs);

  const uint8_t* kbase = a.k + ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh) * EB + sl * 16;
  const int64_t row_bytes = a.st * EB;
  float* srow = a.scores + (int64_t)row * a.N;

  constexpr int per_wave_iter = RPW * U;
  constexpr int per_iter = 4 * per_wave_iter;
  constexpr int kIters = kScoreTile / per_iter;
  static_assert(kScoreTile % per_iter == 0, "whole iterations per tile");
  const int64_t t_tile = (int64_t)blockIdx.x * kScoreTile;
  const int64_t t_end = min(t_tile + (int64_t)kScoreTile, a.N);
  // Each wave covers per_wave_iter consecutive tokens per iteration.
  auto load = [&](int64_t base, uint4 (&kw)[U], bool clamp) {
    const int64_t wbase = base + wave * per_wave_iter + lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t t = wbase + u * RPW;
      if (clamp) t = std::min<int64_t>(t, t_end - 1);
      kw[u] = ld16_nt(kbase + t * row_bytes);
    }
  };
  auto reduce = [&](int64_t base, const uint4 (&kw)[U], bool check) {
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float acc = row_dot<KT, LPR, E>(kw[u], qs);
      if (sl == u) mine = acc;
    }
    const int64_t t = base + wave * per_wave_iter + sl * RPW + lg;
    if (sl < U && (!check || t < t_end)) __builtin_nontemporal_store(mine, srow + t);
  };
  if (t_end - t_tile == kScoreTile) {
    // whole tile: a fixed number of iterations, fully unrolled, so every
    // load is unconditional; the next iteration's keys are requested before
    // this one's are reduced (sched_barrier keeps that order) and the
    // in-order load counter waits only for the buffer being reduced
    uint4 kb[2][U];
    load(t_tile, kb[0], false);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      if (i + 1 < kIters) load(t_tile + (i + 1) * per_iter, kb[(i + 1) & 1], false);
      __builtin_amdgcn_sched_barrier(0);
      reduce(t_tile + i * per_iter, kb[i & 1], false);
    }
  } else {
    // the row's ragged last tile: loads clamped to its last token
    for (int64_t base = t_tile; base < t_end; base += per_iter) {
      uint4 kw[U];
      load(base, kw, true);
      reduce(base, kw, true);
    }
  }
}

// Per-query-head scores of HM view rows that read the same KV row (the
// per-query-head view: G = 1, rows r0 .. r0 + HM - 1 read KV head r0 /
// kv_div): each loaded piece of a key row is dotted with the HM queries, so
// the key cache is read once instead of HM times.  Row h's query values are
// (0 + q_h) * scale and its dot products row_dot's, the arithmetic of
// score_exact_kernel on one view row (group_query_sum of one head), so the
// scores are the same fp32 values bit for bit.
template <typename KT, int D, int U, int HM>
__global__ __launch_bounds__(kThreads) void score_exact_heads_kernel(ExactArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int RPW = 64 / LPR;  // rows per wave load
  static_assert(U <= LPR, "one storing lane per unrolled token");

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lg = (tid & 63) / LPR;
  const int sl = tid % LPR;
  const int row0 = blockIdx.y * HM;  // first view row of the group
  const int b = row0 / a.Hkv;
  const int r0 = row0 % a.Hkv;

  float qs[HM][E];
#pragma unroll
  for (int h = 0; h < HM; ++h) {
    float qv[E];
    const int64_t at = ((int64_t)b * a.Hq + r0 + h) * D + sl * E;
    if (a.q_dtype == SA_BF16)
      load_q_vec<E, true>(a.q, at, qv);
    else
      load_q_vec<E, false>(a.q, at, qv);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = 0.0f;
      acc += qv[e];
      qs[h][e] = acc * a.scale;
    }
  }

  const uint8_t* kbase = a.k + ((int64_t)b * a.sb + (int64_t)(r0 / a.kv_div) * a.sh) * EB + sl * 16;
  const int64_t row_bytes = a.st * EB;
  float* srow = a.scores + (int64_t)row0 * a.N;

  constexpr int per_wave_iter = RPW * U;
  constexpr int per_iter = 4 * per_wave_iter;
  constexpr int kIters = kScoreTile / per_iter;
  static_assert(kScoreTile % per_iter == 0, "whole iterations per tile");
  const int64_t t_tile = (int64_t)blockIdx.x * kScoreTile;
  const int64_t t_end = min(t_tile + (int64_t)kScoreTile, a.N);
  auto load = [&](int64_t base, uint4 (&kw)[U], bool clamp) {
    const int64_t wbase = base + wave * per_wave_iter + lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t t = wbase + u * RPW;
      if (clamp) t = std::min<int64_t>(t, t_end - 1);
      kw[u] = ld16_nt(kbase + t * row_bytes);
    }
  };
  auto reduce = [&](int64_t base, const uint4 (&kw)[U], bool check) {
    float mine[HM];
#pragma unroll
    for (int h = 0; h < HM; ++h) mine[h] = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < HM; ++h) {
        const float acc = row_dot<KT, LPR, E>(kw[u], qs[h]);
        if (sl == u) mine[h] = acc;
      }
    const int64_t t = base + wave * per_wave_iter + sl * RPW + lg;
    if (sl < U && (!check || t < t_end)) {
#pragma unroll
      for (int h = 0; h < HM; ++h) __builtin_nontemporal_store(mine[h], srow + (int64_t)h * a.N + t);
    }
  };
  if (t_end - t_tile == kScoreTile) {
    uint4 kb[2][U];
    load(t_tile, kb[0], false);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      if (i + 1 < kIters) load(t_tile + (i + 1) * per_iter, kb[(i + 1) & 1], false);
      __builtin_amdgcn_sched_barrier(0);
      reduce(t_tile + i * per_iter, kb[i & 1], false);
    }
  } else {
    for (int64_t base = t_tile; base < t_end; base += per_iter) {
      uint4 kw[U];
      load(base, kw, true);
      reduce(base, kw, true);
    }
  }
}

// -------------------------------------------------------- block summaries

struct SumArgs {
  const uint8_t* k;
  int64_t sb, sh, st;
  int32_t Hkv;
  int64_t N;
  int32_t bs;
  int32_t nb;
  uint8_t* kmin;
  uint8_t* kmax;
};

template <typename KT>
__device__ __forceinline__ void store_elem(uint8_t* base, int64_t i, float f);
template <>
__device__ __forceinline__ void store_elem<bf16_t>(uint8_t* base, int64_t i, float f) {
  // f is a widened bf16 value: its low 16 bits are zero, so this is exact.
  reinterpret_cast<uint16_t*>(base)[i] = (uint16_t)(__float_as_uint(f) >> 16);
}
template <>
__device__ __forceinline__ void store_elem<float>(uint8_t* base, int64_t i, float f) {
  reinterpret_cast<float*>(base)[i] = f;
}

template <typename KT, int D>
__global__ __launch_bounds__(kThreads) void block_summarize_kernel(SumArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int NG = kThreads / LPR;
  __shared__ float s_mn[NG][D];
  __shared__ float s_mx[NG][D];

  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.y;
  const int j = blockIdx.x;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const uint8_t* kbase = a.k + ((int64_t)b * a.sb + (int64_t)r * a.sh) * EB + sl * 16;
  const int64_t row_bytes = a.st * EB;
  const int64_t t0 = (int64_t)j * a.bs;
  const int64_t t1 = min(t0 + (int64_t)a.bs, a.N);

  float mn[E], mx[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mn[e] = INFINITY;
    mx[e] = -INFINITY;
  }
  for (int64_t t = t0 + grp; t < t1; t += NG) {
    float kf[E];
    unpack16<KT>(ld16_nt(kbase + t * row_bytes), kf);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      mn[e] = fminf(mn[e], kf[e]);
      mx[e] = fmaxf(mx[e], kf[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s_mn[grp][sl * E + e] = mn[e];
    s_mx[grp][sl * E + e] = mx[e];
  }
  __syncthreads();
  const int64_t out = ((int64_t)row * a.nb + j) * D;
  for (int x = tid; x < 2 * D; x += kThreads) {
    const int dim = x % D;
    if (x < D) {
      float v = INFINITY;
#pragma unroll
      for (int q = 0; q < NG; ++q) v = fminf(v, s_mn[q][dim]);
      store_elem<KT>(a.kmin, out + dim, v);
    } else {
      float v = -INFINITY;
#pragma unroll
      for (int q = 0; q < NG; ++q) v = fmaxf(v, s_mx[q][dim]);
      store_elem<KT>(a.kmax, out + dim, v);
    }
  }
}

// ------------------------------------------------------------ block score

struct BlockArgs {
  const void* q;
  sa_dtype q_dtype;
  const uint8_t* kmin;
  const uint8_t* kmax;
  int32_t Hq, Hkv, G;
  int32_t nb;
  float* scores;
};

template <typename KT, int D>
__global__ __launch_bounds__(kThreads) void score_block_kernel(BlockArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int NG = kThreads / LPR;
  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.y;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const int stride = gridDim.x * NG;
  auto off_of = [&](int j) { return (((int64_t)row * a.nb + j) * D) * EB + sl * 16; };

  // the first block's summaries are requested before the queries, so the
  // two loads' latencies overlap; each later block's load is issued one
  // iteration ahead
  int j = blockIdx.x * NG + grp;
  uint4 lmn = make_uint4(0u, 0u, 0u, 0u), lmx = make_uint4(0u, 0u, 0u, 0u);
  if (j < a.nb) {
    lmn = ld16(a.kmin + off_of(j));
    lmx = ld16(a.kmax + off_of(j));
  }
  float qp[E], qn[E];
  float qv[8][E];
  load_q_group<E, D>(a.q, a.q_dtype, (int64_t)b * a.Hq + (int64_t)r * a.G, a.G, sl * E, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float p = 0.0f, n = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float v = g < a.G ? qv[g][e] : 0.0f;
      p += fmaxf(v, 0.0f);
      n += fminf(v, 0.0f);
    }
    qp[e] = p;
    qn[e] = n;
  }
  for (; j < a.nb; j += stride) {
    float mn[E], mx[E];
    unpack16<KT>(lmn, mn);
    unpack16<KT>(lmx, mx);
    if (j + stride < a.nb) {
      lmn = ld16(a.kmin + off_of(j + stride));
      lmx = ld16(a.kmax + off_of(j + stride));
    }
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(qp[e], mx[e], fmaf(qn[e], mn[e], acc));
    acc = group_sum<LPR>(acc);
    if (sl == 0) a.scores[(int64_t)row * a.nb + j] = acc;
  }
}

// ------------------------------------------------ block score + top-k
// Block selection of a whole row in one workgroup: the row's block scores
// (the same arithmetic as score_block_kernel, so the same fp32 values) from
// its per-block key summaries, kSelBlkU passes of blocks with every summary
// load of a pass group in flight, kept in LDS; then the register-resident
// top-k of the row (reg_row_topk) writes the k best block ids, ascending --
// one launch instead of a score launch and a top-k launch.
constexpr int kSelBlkThreads = 1024;
constexpr int kSelBlkMax = 4 * kSelBlkThreads;  // blocks per row at most
constexpr int kSelBlkU = 4;

template <typename KT, int D>
__global__ __launch_bounds__(kSelBlkThreads) void select_block_kernel(BlockArgs a, int32_t k,
                                                                     int32_t* __restrict__ idx) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int NG = kSelBlkThreads / LPR;  // blocks per pass
  __shared__ float s_sc[kSelBlkMax];
  __shared__ SharedT<kSelBlkThreads> sh;
  __shared__ __align__(16) uint2 cand[kRankMax + 8];
  __shared__ uint32_t s_wave[kSelBlkThreads / 64];
  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  auto off_of = [&](int j) { return (((int64_t)row * a.nb + j) * D) * EB + sl * 16; };

  uint4 lmn[kSelBlkU], lmx[kSelBlkU];
#pragma unroll
  for (int u = 0; u < kSelBlkU; ++u) {
    const int j = u * NG + grp;
    lmn[u] = j < a.nb ? ld16(a.kmin + off_of(j)) : make_uint4(0u, 0u, 0u, 0u);
    lmx[u] = j < a.nb ? ld16(a.kmax + off_of(j)) : make_uint4(0u, 0u, 0u, 0u);
  }
  float qp[E], qn[E];
  float qv[8][E];
  load_q_group<E, D>(a.q, a.q_dtype, (int64_t)b * a.Hq + (int64_t)r * a.G, a.G, sl * E, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float p = 0.0f, n = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const float v = g < a.G ? qv[g][e] : 0.0f;
      p += fmaxf(v, 0.0f);
      n += fminf(v, 0.0f);
    }
    qp[e] = p;
    qn[e] = n;
  }
  for (int j0 = 0; j0 < a.nb; j0 += kSelBlkU * NG) {
#pragma unroll
    for (int u = 0; u < kSelBlkU; ++u) {
      const int j = j0 + u * NG + grp;
      float mn[E], mx[E];
      unpack16<KT>(lmn[u], mn);
      unpack16<KT>(lmx[u], mx);
      const int jn = j + kSelBlkU * NG;  // the next group's block, loaded now
      if (jn < a.nb) {
        lmn[u] = ld16(a.kmin + off_of(jn));
        lmx[u] = ld16(a.kmax + off_of(jn));
      }
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(qp[e], mx[e], fmaf(qn[e], mn[e], acc));
      acc = group_sum<LPR>(acc);
      if (sl == 0 && j < a.nb) s_sc[j] = acc;
    }
  }
  __syncthreads();
  int32_t* __restrict__ out = idx + (int64_t)row * k;
  auto load = [&](int p0, float (&v)[1][4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[0][e] = p0 + e < a.nb ? s_sc[p0 + e] : 0.0f;
  };
  auto emit = [&](uint32_t slot, int32_t p) { out[slot] = p; };
  reg_row_topk<kSelBlkThreads, 1, false>(load, a.nb, k, emit, sh, cand, s_wave);
}

// --------------------------------------------------------------- indexer

struct IndexerArgs {
  const uint8_t* q_idx;  // [B, H, DI] bf16
  const uint8_t* k_idx;  // [B, N, DI] bf16
  const float* w;        // [B, H]
  int32_t H;
  int64_t N;
  float* scores;         // [B, N]
  uint32_t* hist;        // optional: row b's 12-bit key histogram at hist + b * hist_stride
  int64_t hist_stride;
};

constexpr int kKeyBins = 4096;  // histogram of the top 12 bits of score_key

// One lane group of LPR = DI/8 lanes holds a token's indexer key (16 bytes
// per lane); indexer_token (v_dot2_f32_bf16 on the packed bf16 values, DPP
// head sums) gives its score.  (The unpack-and-fma form needed 2.5x the VALU
// instructions per byte; matrix-core tiles need a 16-token by 16-byte load
// pattern that streams worse.)
// With HIST the workgroup also counts the top 12 bits of its scores' keys in
// LDS and adds the non-empty bins to the row's histogram (global atomics)
// for the top-k that follows; its tile is then TILE tokens, larger than the
// plain kernel's, so that fewer workgroups add into the same bins.
template <int DI, int HP, int U, bool HIST, int TILE>
__global__ __launch_bounds__(kThreads) void score_indexer_kernel(IndexerArgs a) {
  constexpr int LPR = DI * 2 / 16;
  constexpr int RPW = 64 / LPR;
  static_assert(U <= LPR, "one storing lane per unrolled token");
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lg = (tid & 63) / LPR;
  const int sl = tid % LPR;
  const int b = blockIdx.y;

  uint4 qv[HP];  // this lane's 8 dims of every indexer query, packed bf16
  float wv[HP];
  load_indexer_queries<DI, HP>(a.q_idx, a.w, b, a.H, sl, qv, wv);

  __shared__ uint32_t s_hist[HIST ? kKeyBins : 1];
  if constexpr (HIST) {
    for (int i = tid; i < kKeyBins; i += kThreads) s_hist[i] = 0u;
    __syncthreads();
  }

  const uint8_t* kbase = a.k_idx + (int64_t)b * a.N * DI * 2 + sl * 16;
  float* srow = a.scores + (int64_t)b * a.N;
  constexpr int per_wave_iter = RPW * U;
  constexpr int per_iter = 4 * per_wave_iter;
  constexpr int kIters = TILE / per_iter;
  static_assert(TILE % per_iter == 0, "whole iterations per tile");
  const int64_t t_tile = (int64_t)blockIdx.x * TILE;
  const int64_t t_end = min(t_tile + (int64_t)TILE, a.N);
  // same load structure as the exact score: clamped, branch-free loads and a
  // ping-pong over two buffers on whole tiles
  auto load = [&](int64_t base, uint4 (&kw)[U], bool clamp) {
    const int64_t wbase = base + wave * per_wave_iter + lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t t = wbase + u * RPW;
      if (clamp) t = std::min<int64_t>(t, t_end - 1);
      kw[u] = ld16_nt(kbase + t * (DI * 2));
    }
  };
  auto reduce = [&](int64_t base, const uint4 (&kw)[U], bool check) {
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = indexer_token<LPR, HP>(kw[u], qv, wv);
      if (sl == u) mine = sc;
    }
    const int64_t t = base + wave * per_wave_iter + sl * RPW + lg;
    if (sl < U && (!check || t < t_end)) {
      __builtin_nontemporal_store(mine, srow + t);
      if constexpr (HIST) atomicAdd(&s_hist[score_key(mine) >> 20], 1u);
    }
  };
  if (t_end - t_tile == TILE) {
    uint4 kb[2][U];
    load(t_tile, kb[0], false);
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      if (i + 1 < kIters) load(t_tile + (i + 1) * per_iter, kb[(i + 1) & 1], false);
      __builtin_amdgcn_sched_barrier(0);
      reduce(t_tile + i * per_iter, kb[i & 1], false);
    }
  } else {
    for (int64_t base = t_tile; base < t_end; base += per_iter) {
      uint4 kw[U];
      load(base, kw, true);
      reduce(base, kw, true);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    uint32_t* g = a.hist + (int64_t)b * a.hist_stride;
    for (int i = tid; i < kKeyBins; i += kThreads)
      if (s_hist[i]) atomicAdd(&g[i], s_hist[i]);
  }
}

template <int DI, int HP>
hipError_t launch_indexer_hp(const IndexerArgs& a, dim3 grid, hipStream_t s) {
  constexpr int LPR = DI * 2 / 16;
  // tokens per lane group in flight: 8 (4 with 16 heads, whose queries fill
  // the registers)
  constexpr int U = HP >= 16 ? (LPR < 4 ? LPR : 4) : (LPR < 8 ? LPR : 8);
  if (a.hist) {
    const dim3 g((unsigned)((a.N + kIndexerHistTile - 1) / kIndexerHistTile), grid.y);
    hipLaunchKernelGGL((score_indexer_kernel<DI, HP, U, true, kIndexerHistTile>), g, dim3(kThreads),
                       0, s, a);
  } else {
    hipLaunchKernelGGL((score_indexer_kernel<DI, HP, U, false, kScoreTile>), grid, dim3(kThreads),
                       0, s, a);
  }
  return hipGetLastError();
}

template <int DI>
hipError_t launch_indexer_di(const IndexerArgs& a, dim3 grid, hipStream_t s) {
  if (a.H <= 4) return launch_indexer_hp<DI, 4>(a, grid, s);
  if (a.H <= 8) return launch_indexer_hp<DI, 8>(a, grid, s);
  return launch_indexer_hp<DI, 16>(a, grid, s);
}

// HM view rows per workgroup row, each wave U token rows per load.
template <int HM>
hipError_t launch_score_heads(const Cache& c, const ExactArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((c.N + kScoreTile - 1) / kScoreTile), (unsigned)(c.B * c.Hkv / HM));
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((score_exact_heads_kernel<bf16_t, 64, 4, HM>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_exact_heads_kernel<bf16_t, 128, 8, HM>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((score_exact_heads_kernel<float, 64, 8, HM>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_exact_heads_kernel<float, 128, 8, HM>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_exact(const Cache& c, const void* q, const void* k, float* scores,
                              hipStream_t s) {
  ExactArgs a{};
  a.q = q;
  a.q_dtype = c.q_dtype;
  a.k = static_cast<const uint8_t*>(k);
  a.sb = c.sb;
  a.sh = c.sh;
  a.st = c.st;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.G = c.G;
  a.kv_div = c.kv_div;
  a.N = c.N;
  a.scale = c.scale;
  a.scores = scores;
  if (per_q_head_shared_rows(c) > 1) {
    if (per_q_head_shared_rows(c) == 2) return launch_score_heads<2>(c, a, s);
    return launch_score_heads<4>(c, a, s);
  }
  const dim3 grid((unsigned)((c.N + kScoreTile - 1) / kScoreTile), (unsigned)(c.B * c.Hkv));
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((score_exact_kernel<bf16_t, 64, 8>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_exact_kernel<bf16_t, 128, 16>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((score_exact_kernel<float, 64, 16>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_exact_kernel<float, 128, 16>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_block_summarize(const Cache& c, int32_t bs, const void* k, void* kmin, void* kmax,
                                  hipStream_t s) {
  SumArgs a{};
  a.k = static_cast<const uint8_t*>(k);
  a.sb = c.sb;
  a.sh = c.sh;
  a.st = c.st;
  a.Hkv = c.Hkv;
  a.N = c.N;
  a.bs = bs;
  a.nb = (int32_t)((c.N + bs - 1) / bs);
  a.kmin = static_cast<uint8_t*>(kmin);
  a.kmax = static_cast<uint8_t*>(kmax);
  const dim3 grid((unsigned)a.nb, (unsigned)(c.B * c.Hkv));
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((block_summarize_kernel<bf16_t, 64>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((block_summarize_kernel<bf16_t, 128>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((block_summarize_kernel<float, 64>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((block_summarize_kernel<float, 128>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_score_block(const Cache& c, int32_t bs, const void* q, const void* kmin,
                              const void* kmax, float* scores, hipStream_t s) {
  BlockArgs a{};
  a.q = q;
  a.q_dtype = c.q_dtype;
  a.kmin = static_cast<const uint8_t*>(kmin);
  a.kmax = static_cast<const uint8_t*>(kmax);
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.G = c.G;
  a.nb = (int32_t)((c.N + bs - 1) / bs);
  a.scores = scores;
  const int lpr = c.D * (c.kv_dtype == SA_BF16 ? 2 : 4) / 16;
  const int ng = kThreads / lpr;
  const unsigned gx = (unsigned)std::min<int64_t>((a.nb + ng - 1) / ng, 65535);
  const dim3 grid(gx, (unsigned)(c.B * c.Hkv));
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((score_block_kernel<bf16_t, 64>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_block_kernel<bf16_t, 128>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((score_block_kernel<float, 64>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((score_block_kernel<float, 128>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

bool select_block_fits(const Cache& c, int32_t bs) {
  return (c.N + bs - 1) / bs <= kSelBlkMax && c.G <= 8;
}

hipError_t launch_select_block(const Cache& c, int32_t bs, const void* q, const void* kmin,
                               const void* kmax, int32_t k, int32_t* idx, hipStream_t s) {
  BlockArgs a{};
  a.q = q;
  a.q_dtype = c.q_dtype;
  a.kmin = static_cast<const uint8_t*>(kmin);
  a.kmax = static_cast<const uint8_t*>(kmax);
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.G = c.G;
  a.nb = (int32_t)((c.N + bs - 1) / bs);
  a.scores = nullptr;
  const dim3 grid((unsigned)(c.B * c.Hkv)), block(kSelBlkThreads);
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((select_block_kernel<bf16_t, 64>), grid, block, 0, s, a, k, idx);
    else
      hipLaunchKernelGGL((select_block_kernel<bf16_t, 128>), grid, block, 0, s, a, k, idx);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((select_block_kernel<float, 64>), grid, block, 0, s, a, k, idx);
    else
      hipLaunchKernelGGL((select_block_kernel<float, 128>), grid, block, 0, s, a, k, idx);
  }
  return hipGetLastError();
}

hipError_t launch_score_indexer(int32_t B, int64_t N, int32_t H, int32_t Di, const void* q_idx,
                                const void* k_idx, const float* w, float* scores, hipStream_t s,
                                uint32_t* hist, int64_t hist_stride) {
  IndexerArgs a{};
  a.hist = hist;
  a.hist_stride = hist_stride;
  a.q_idx = static_cast<const uint8_t*>(q_idx);
  a.k_idx = static_cast<const uint8_t*>(k_idx);
  a.w = w;
  a.H = H;
  a.N = N;
  a.scores = scores;
  const dim3 grid((unsigned)((N + kScoreTile - 1) / kScoreTile), (unsigned)B);
  if (Di == 32) return launch_indexer_di<32>(a, grid, s);
  if (Di == 64) return launch_indexer_di<64>(a, grid, s);
  return launch_indexer_di<128>(a, grid, s);
}

}  // namespace sa
