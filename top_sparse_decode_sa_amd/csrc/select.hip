// Exact top-k selection without the score array.
//
// What is computed: the same index list as exact scoring followed by top-k
// ("Inference-time context sparsity: illusion or opportunity?", section 2:
// oracle top-k over the exact scores q . k_t, the group's query heads summed;
// "Flash Attention vs Sparse Attention", DSA Stage 1: the top-K index list)
// -- the k positions with the largest scores, equal scores taken from the
// lower position, in ascending position order.
//
// Why fused: streaming the key cache is the whole cost of exact selection,
// and writing the fp32 score of every token back to HBM in the middle of that
// stream costs far more than its bytes (the writes interleave with the reads).
// Here the scores never leave the chip:
//
//  1. select_part_kernel: a row is cut into parts of L <= 8192 tokens; one
//     workgroup (256 or 512 threads) streams its part's keys (the score
//     kernel's arithmetic, bit for bit: group_query_sum, row_dot), keeps
//     the part's scores in LDS, then runs the register-resident radix select
//     (reg_row_topk) on them and writes the part's top-min(k, part length)
//     as (score, position) candidates, in position order.
//  2. Merge: the row's candidates, concatenated in part order (so in
//     position order), go through the same top-k with the candidate index
//     mapped back to its position.  Every element of the row's top-k is in
//     its part's top-k (fewer than k elements of its part precede it), so the
//     merge returns exactly the row's top-k.
//  A row of one part writes its index list from step 1 directly.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "topk_core.hpp"

namespace sa {
namespace {

constexpr int kIndexerNT = 512;  // threads of an indexer-score part
constexpr int kChipCUs = 256;    // MI355X compute units
constexpr int kPartMax = 8192;         // longest part: what the register select holds (32 keys
                                       // per thread at 256 threads, 16 at 512)
constexpr int kPartAlign = 256;        // a multiple of every layout's tokens per iteration
constexpr int kSelCand = kRankMax + 8; // threshold-bin candidates ranked in LDS
constexpr int kMinGroups = 512;        // parts shrink (to 256 tokens) until the grid has this many
constexpr int64_t kMergeMax = 32768;   // candidates per row the merge holds in registers

struct SelArgs {
  const void* q;
  sa_dtype q_dtype;
  const uint8_t* k;
  int64_t sb, sh, st;
  int32_t Hq, Hkv, G;
  int32_t kv_div;  // row r reads KV head r / kv_div
  int64_t N;
  float scale;
  int32_t L;        // tokens per part
  int32_t k_sel;    // k
  int32_t kcap;     // candidate slots per part
  int64_t cstride;  // candidate row stride
  float* cand_val;  // [rows, cstride]: candidate scores
  int32_t* cand_pos;
  int32_t* idx;  // one part per row: the final list [rows, k], else null
  // indexer scoring: queries [rows, H, DI] bf16, keys [rows, N, DI] bf16,
  // weights [rows, H]
  const uint8_t* q_idx;
  const uint8_t* k_idx;
  const float* w_idx;
  int32_t H_idx;
};

// Streams a part's n tokens in iterations of PER tokens: whole iterations
// through a 2-deep ping-pong (the next iteration's loads requested before
// this one's are reduced; an odd count peels one first so the pipelined run
// is even), then the ragged end with loads clamped to the last token.
template <int PER, int U, typename Load, typename Reduce>
__device__ __forceinline__ void stream_part(int n, Load load, Reduce reduce) {
  const int nf = n / PER;  // whole iterations
  int i0 = 0;
  if (nf & 1) {
    uint4 kw[U];
    load(0, kw, false);
    reduce(0, kw, false);
    i0 = 1;
  }
  if (i0 < nf) {
    uint4 ka[U], kb[U];
    load(i0 * PER, ka, false);
    int i = i0;
    for (; i + 2 < nf; i += 2) {
      load((i + 1) * PER, kb, false);
      __builtin_amdgcn_sched_barrier(0);
      reduce(i * PER, ka, false);
      load((i + 2) * PER, ka, false);
      __builtin_amdgcn_sched_barrier(0);
      reduce((i + 1) * PER, kb, false);
    }
    load((i + 1) * PER, kb, false);
    __builtin_amdgcn_sched_barrier(0);
    reduce(i * PER, ka, false);
    reduce((i + 1) * PER, kb, false);
  }
  if (nf * PER < n) {
    uint4 kw[U];
    load(nf * PER, kw, true);
    reduce(nf * PER, kw, true);
  }
}

template <int NT>
struct PartLds {
  SharedT<NT> sh;
  uint2 cand[kSelCand];
  uint32_t s_wave[NT / 64];
};

// The part's top-min(k, n) from its LDS scores (histogram already counted):
// the index list itself for a one-part row, else (score, position)
// candidates in position order.
template <int G, int NT>
__device__ __forceinline__ void part_select(const SelArgs& a, const float* s_sc, int n, int row,
                                            int part, int64_t t0, PartLds<NT>& l) {
  auto lds_load = [&](int p0, float (&v)[G][4]) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float4 f = *reinterpret_cast<const float4*>(&s_sc[p0 + 256 * j]);
      v[j][0] = f.x;
      v[j][1] = f.y;
      v[j][2] = f.z;
      v[j][3] = f.w;
    }
  };
  const int32_t kk = std::min(a.k_sel, n);
  if (a.idx) {
    int32_t* out = a.idx + (int64_t)row * a.k_sel;
    reg_row_topk<NT, G, true>(
        lds_load, n, kk, [&](uint32_t slot, int32_t p) { out[slot] = p; }, l.sh, l.cand,
        l.s_wave);
  } else {
    const int64_t c0 = (int64_t)row * a.cstride + (int64_t)part * a.kcap;
    float* cv = a.cand_val + c0;
    int32_t* cp = a.cand_pos + c0;
    reg_row_topk<NT, G, true>(
        lds_load, n, kk,
        [&](uint32_t slot, int32_t p) {
          cv[slot] = s_sc[p];
          cp[slot] = (int32_t)t0 + p;
        },
        l.sh, l.cand, l.s_wave);
  }
}

// Parts of at most 4 * G * NT tokens (the register select holds 4 G keys
// per thread) for workgroups of NT threads.
template <typename KT, int D, int U, int G, int NT>
__global__ __launch_bounds__(NT) void select_part_kernel(SelArgs a) {
  constexpr int EB = Elt<KT>::kBytes;
  constexpr int E = Elt<KT>::kPer16B;
  constexpr int LPR = D * EB / 16;
  constexpr int RPW = 64 / LPR;  // rows per wave load
  constexpr int per_wave_iter = RPW * U;
  constexpr int per_iter = (NT / 64) * per_wave_iter;
  static_assert(U <= LPR, "one storing lane per unrolled token");
  static_assert(kPartAlign % per_iter == 0, "whole iterations per part");

  __shared__ __align__(16) float s_sc[4 * G * NT];
  __shared__ PartLds<NT> l;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lg = (tid & 63) / LPR;
  const int sl = tid % LPR;
  const int part = blockIdx.x;
  const int row = blockIdx.y;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;
  const int64_t t0 = (int64_t)part * a.L;
  const int n = (int)std::min<int64_t>(a.L, a.N - t0);  // tokens of this part

  float qs[E];
  group_query_sum<E, D>(a.q, a.q_dtype, (int64_t)b * a.Hq + (int64_t)r * a.G, a.G, sl * E, a.scale,
                        qs);
  const uint8_t* kbase =
      a.k + ((int64_t)b * a.sb + (int64_t)(r / a.kv_div) * a.sh + t0 * a.st) * EB + sl * 16;
  // the selection's 12-bit histogram is counted as the scores are produced
  zero_hist(l.sh, kBins);
  __syncthreads();
  const int64_t row_bytes = a.st * EB;

  // ---- 1. scores of the part into LDS.  Each wave covers per_wave_iter
  // consecutive tokens per iteration.
  const uint8_t* kwave = kbase + (int64_t)(wave * per_wave_iter + lg) * row_bytes;
  auto load = [&](int base, uint4 (&kw)[U], bool clamp) {
    if (clamp) {
      const int wbase = base + wave * per_wave_iter + lg;
#pragma unroll
      for (int u = 0; u < U; ++u)
        kw[u] = ld16_nt(kbase + (int64_t)std::min(wbase + u * RPW, n - 1) * row_bytes);
    } else {
      const uint8_t* p = kwave + (int64_t)base * row_bytes;
#pragma unroll
      for (int u = 0; u < U; ++u) kw[u] = ld16_nt(p + (int64_t)(u * RPW) * row_bytes);
    }
  };
  auto reduce = [&](int base, const uint4 (&kw)[U], bool check) {
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float acc = row_dot<KT, LPR, E>(kw[u], qs);
      if (sl == u) mine = acc;
    }
    const int t = base + wave * per_wave_iter + sl * RPW + lg;
    if (sl < U && (!check || t < n)) {
      s_sc[t] = mine;
      atomicAdd(&l.sh.hist[score_key(mine) >> 20], 1u);
    }
  };
  stream_part<per_iter, U>(n, load, reduce);
  __syncthreads();

  // ---- 2. top-min(k, n) of the part
  part_select<G, NT>(a, s_sc, n, row, part, t0, l);
}

// The same part selection on indexer scores ("Flash Attention vs Sparse
// Attention", DSA Stage 1): row `row` of the indexer tensors, its keys read
// by lane groups of DI/8 lanes, each token scored by indexer_token (the same
// arithmetic as the indexer scoring kernel).
template <int DI, int HP, int U, int G, int NT>
__global__ __launch_bounds__(NT) void select_indexer_kernel(SelArgs a) {
  constexpr int LPR = DI * 2 / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int per_wave_iter = RPW * U;
  constexpr int per_iter = (NT / 64) * per_wave_iter;
  static_assert(U <= LPR, "one storing lane per unrolled token");
  static_assert(kPartAlign % per_iter == 0, "whole iterations per part");

  __shared__ __align__(16) float s_sc[4 * G * NT];
  __shared__ PartLds<NT> l;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lg = (tid & 63) / LPR;
  const int sl = tid % LPR;
  const int part = blockIdx.x;
  const int row = blockIdx.y;
  const int64_t t0 = (int64_t)part * a.L;
  const int n = (int)std::min<int64_t>(a.L, a.N - t0);

  uint4 qv[HP];
  float wv[HP];
  load_indexer_queries<DI, HP>(a.q_idx, a.w_idx, row, a.H_idx, sl, qv, wv);
  const uint8_t* kbase = a.k_idx + ((int64_t)row * a.N + t0) * DI * 2 + sl * 16;
  zero_hist(l.sh, kBins);
  __syncthreads();

  auto load = [&](int base, uint4 (&kw)[U], bool clamp) {
    const int wbase = base + wave * per_wave_iter + lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int t = wbase + u * RPW;
      if (clamp) t = std::min(t, n - 1);
      kw[u] = ld16_nt(kbase + (int64_t)t * (DI * 2));
    }
  };
  auto reduce = [&](int base, const uint4 (&kw)[U], bool check) {
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float sc = indexer_token<LPR, HP>(kw[u], qv, wv);
      if (sl == u) mine = sc;
    }
    const int t = base + wave * per_wave_iter + sl * RPW + lg;
    if (sl < U && (!check || t < n)) {
      s_sc[t] = mine;
      atomicAdd(&l.sh.hist[score_key(mine) >> 20], 1u);
    }
  };
  stream_part<per_iter, U>(n, load, reduce);
  __syncthreads();
  part_select<G, NT>(a, s_sc, n, row, part, t0, l);
}

}  // namespace

SelectPlan plan_select(const Cache& c, int32_t k) {
  SelectPlan p;
  const int64_t rows = (int64_t)c.B * c.Hkv;
  // candidates per row for parts of L tokens
  auto cands = [&](int64_t L) {
    const int64_t P = (c.N + L - 1) / L;
    return (P - 1) * std::min<int64_t>(k, L) + std::min<int64_t>(k, c.N - (P - 1) * L);
  };
  // the longest parts, shortened while the grid is small and the candidates
  // stay within a quarter of the row
  int64_t L = kPartMax;
  while (L > kPartAlign && rows * ((c.N + L - 1) / L) < kMinGroups && 4 * cands(L / 2) <= c.N)
    L /= 2;
  p.L = (int32_t)L;
  p.P = (int32_t)((c.N + L - 1) / L);
  p.kcap = (int32_t)std::min<int64_t>(k, L);
  p.C = cands(L);
  p.cstride = (p.C + 3) / 4 * 4;
  // fused when the candidates are at most a quarter of the row and fit the
  // merge (measured: at 4 parts of 8192 tokens the fused path is faster
  // from 20x sparsity on, slower at 10x, where each part keeps 40% of its
  // tokens); one part needs no merge.  Per-query-head rows (several view
  // rows on one KV row) split into parts take the unfused path: their
  // scoring reads each key row once for all of the KV head's query heads,
  // where the part kernel would read it once per query head.
  p.fused = p.P == 1 || (p.C <= kMergeMax && 4 * p.C <= c.N && per_q_head_shared_rows(c) == 1);
  if (!p.fused) {
    p.ws_bytes = align_up((size_t)rows * c.N * sizeof(float), 256) +
                 align_up(topk_workspace_bytes(rows, c.N, k), 256);
  } else if (p.P > 1) {
    p.ws_bytes = 2 * align_up((size_t)rows * p.cstride * sizeof(float), 256);
  }
  return p;
}

namespace {

// Indexer-score parts: workgroups of kIndexerNT threads; U as for 256
// threads, halved per doubling of the waves (one workgroup iteration stays
// within kPartAlign tokens), at least 1.
template <int G, int DI, int HP>
void launch_indexer_part(const SelArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NT = kIndexerNT;
  constexpr int LPR = DI * 2 / 16;
  constexpr int U256 = HP >= 16 ? (LPR < 4 ? LPR : 4) : (LPR < 8 ? LPR : 8);
  constexpr int U = U256 * 256 / NT > 0 ? U256 * 256 / NT : 1;
  hipLaunchKernelGGL((select_indexer_kernel<DI, HP, U, G, NT>), grid, dim3(NT), 0, s, a);
}

template <int G, int DI>
void launch_indexer_part_h(const SelArgs& a, dim3 grid, hipStream_t s) {
  if (a.H_idx <= 4) launch_indexer_part<G, DI, 4>(a, grid, s);
  else if (a.H_idx <= 8) launch_indexer_part<G, DI, 8>(a, grid, s);
  else launch_indexer_part<G, DI, 16>(a, grid, s);
}

// Exact-score parts: workgroups of NT threads, each wave U token rows per
// load (U scaled so that one iteration of the workgroup is kPartAlign tokens
// or a divisor of it).
template <int G, int NT>
void launch_exact_part_g(const Cache& c, const SelArgs& a, dim3 grid, hipStream_t s) {
  static_assert(NT == 256 || NT == 512, "four or eight waves");
  const dim3 block(NT);
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64)
      hipLaunchKernelGGL((select_part_kernel<bf16_t, 64, (NT == 256 ? 8 : 4), G, NT>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((select_part_kernel<bf16_t, 128, (NT == 256 ? 16 : 8), G, NT>), grid, block, 0, s, a);
  } else {
    if (c.D == 64)
      hipLaunchKernelGGL((select_part_kernel<float, 64, (NT == 256 ? 16 : 8), G, NT>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((select_part_kernel<float, 128, 16, G, NT>), grid, block, 0, s, a);
  }
}

// Groups of four keys per thread that hold a part of L tokens: eight (at
// 256 threads) for the longest parts, else the form that holds 4096 tokens.
template <int NT>
void launch_exact_part_nt(const Cache& c, const SelArgs& a, dim3 grid, hipStream_t s) {
  if (a.L > 4096)
    launch_exact_part_g<8 * 256 / NT, NT>(c, a, grid, s);
  else
    launch_exact_part_g<4 * 256 / NT, NT>(c, a, grid, s);
}

// Parts that all run at once (two 512-thread workgroups per CU) take eight
// waves each, so the key stream has twice the waves and each part's top-k
// half the keys per thread (llama32k, 512 parts: 176 against 181 us for
// sa_select); grids of several rounds keep 256-thread workgroups, three per
// CU, whose part top-k overlaps the other workgroups' streams (batch128k,
// 16384 parts: 5.51 against 5.65 ms at 100x).
void launch_exact_part(const Cache& c, const SelArgs& a, dim3 grid, hipStream_t s) {
  if ((int64_t)grid.x * grid.y <= 2 * kChipCUs)
    launch_exact_part_nt<512>(c, a, grid, s);
  else
    launch_exact_part_nt<256>(c, a, grid, s);
}

template <int G>
void launch_part(const Cache& c, const SelectIndexer* ix, const SelArgs& a, dim3 grid,
                 hipStream_t s) {
  if (!ix) {
    launch_exact_part(c, a, grid, s);
  } else if (ix->Di == 32) {
    launch_indexer_part_h<G, 32>(a, grid, s);
  } else if (ix->Di == 64) {
    launch_indexer_part_h<G, 64>(a, grid, s);
  } else {
    launch_indexer_part_h<G, 128>(a, grid, s);
  }
}

}  // namespace

hipError_t launch_select(const Cache& c, const SelectPlan& p, const void* q, const void* k,
                         const SelectIndexer* ix, int32_t kk, int32_t* idx, void* ws,
                         hipStream_t s, const MergeAttend* ma, bool* attended) {
  const int64_t rows = (int64_t)c.B * c.Hkv;
  if (attended) *attended = false;
  if (!p.fused) {
    float* scores = static_cast<float*>(ws);
    void* topk_ws = static_cast<uint8_t*>(ws) + align_up((size_t)rows * c.N * sizeof(float), 256);
    if (ix && topk_counted(rows, c.N, kk)) {
      // the indexer launch counts the top-k's histogram as it writes the scores
      int64_t hs = 0;
      uint32_t* hist = topk_counted_hist(topk_ws, &hs);
      hipError_t e = launch_topk_counted_zero(topk_ws, rows, s);
      if (e == hipSuccess)
        e = launch_score_indexer((int32_t)rows, c.N, ix->H, ix->Di, ix->q_idx, ix->k_idx, ix->w,
                                 scores, s, hist, hs);
      if (e != hipSuccess) return e;
      return launch_topk_counted(scores, rows, c.N, c.N, kk, idx, topk_ws, s);
    }
    hipError_t e = ix ? launch_score_indexer((int32_t)rows, c.N, ix->H, ix->Di, ix->q_idx,
                                             ix->k_idx, ix->w, scores, s)
                      : launch_score_exact(c, q, k, scores, s);
    if (e != hipSuccess) return e;
    return launch_topk(scores, rows, c.N, c.N, kk, idx, topk_ws, s);
  }
  SelArgs a{};
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
  a.L = p.L;
  a.k_sel = kk;
  a.kcap = p.kcap;
  a.cstride = p.cstride;
  if (ix) {
    a.q_idx = static_cast<const uint8_t*>(ix->q_idx);
    a.k_idx = static_cast<const uint8_t*>(ix->k_idx);
    a.w_idx = ix->w;
    a.H_idx = ix->H;
  }
  if (p.P == 1) {
    a.idx = idx;
  } else {
    a.cand_val = static_cast<float*>(ws);
    a.cand_pos = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                            align_up((size_t)rows * p.cstride * sizeof(float), 256));
  }
  const dim3 grid((unsigned)p.P, (unsigned)rows);
  if (p.L > 4096)
    launch_part<8 * 256 / kIndexerNT>(c, ix, a, grid, s);
  else
    launch_part<4 * 256 / kIndexerNT>(c, ix, a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.P == 1) return e;
  if (ma && attended && (int64_t)ma->c.B * ma->c.Hkv == rows &&
      merge_attend_ok(ma->c, ma->p, p.C, kk)) {
    *attended = true;
    return launch_merge_attend(ma->c, ma->p, ma->q, ma->k, ma->v, ma->out, a.cand_val, a.cand_pos,
                               p.C, p.cstride, kk, idx, s);
  }
  return launch_topk_merge(a.cand_val, a.cand_pos, rows, p.C, p.cstride, kk, idx, s);
}

}  // namespace sa
