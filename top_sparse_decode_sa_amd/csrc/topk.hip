// Exact top-k selection of fp32 score rows.
//
// What is computed ("Inference-time context sparsity", section 2: oracle
// top-k; "Flash Attention vs Sparse Attention", DSA Stage 1: a top-K index
// list): the k positions of a row with the largest scores, equal scores taken
// from the lower position, returned in ascending position order.
//
// Method: radix select on order-preserving uint32 keys (score_key).
//
// Row paths, one 1024-thread workgroup per row:
//   1. A histogram of the top 12 key bits (4096 bins).  A prefix sum over the
//      bins gives d1, the bin of the k-th largest key, and kleft, how many
//      result elements lie inside that bin.
//   2. The keys of bin d1 (the candidates) are collected with their positions
//      into LDS; the keys of higher bins are all in the result.
//   3. The candidates are resolved into T, the key of the last result element
//      in selection order, and `need`, how many keys equal to T belong to the
//      result: up to kRankCap candidates by pairwise ranking (rank = number of
//      candidates with a larger key or an equal key at a lower position; rank
//      < kleft is kept), more by 8- and 4-bit digit passes over the list.  If
//      the list overflows, digit passes run over the whole row instead.
//   4. Ordered write: every kept element's output slot is the number of kept
//      elements at lower positions = (keys above T before it) + min(keys
//      equal to T before it, need).
// Rows of at most kResident keys (topk_reg_kernel) keep every key in the
// registers of the thread that loaded it, 32 per thread, and work on per-
// thread bit masks after the histogram; longer rows (topk_long_kernel) are
// read from global memory once per phase, the ordered write through LDS
// tiles.
//
// Multi-workgroup path, for few rows longer than kResident (a single 1M-token
// sequence): (a) zero a per-row histogram; (b) workgroups of kMwChunk keys add
// their 12-bit histograms with global atomics (or the scoring launch counts
// the histogram as it writes the scores: launch_topk_counted); (c) the same
// workgroups each recompute d1 from the finished histogram and append, in
// position order within their chunk, the positions of keys above bin d1 and
// the (key, position) candidates of bin d1 to per-row lists; (d) one
// workgroup per row gathers both lists in chunk order, resolves the
// candidates as in step 3 and writes each kept position to its slot (kept
// positions of earlier chunks, then of its own chunk below it).  If the
// candidates overflow their list, (d) runs the row path on the row.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"
#include "topk_core.hpp"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kResident = 32768;  // keys kept in LDS (128 KB)
constexpr int kTile = 16384;      // keys per LDS tile of the ordered write, other rows
constexpr int kCandRes = 1024;    // candidate (key, position) pairs, resident rows
constexpr int kCandGlob = 8192;   // candidate pairs, other rows

constexpr int kMwChunk = 8192;       // keys per workgroup, multi-workgroup path
constexpr int kMwCand = 8192;        // candidate capacity per row
constexpr int kMwMaxRows = 64;       // rows at most, multi-workgroup path
constexpr int kMwMaxChunks = 1024;   // chunks per row at most (n <= 8M)

using Shared = SharedT<kThreads>;

// LDS key layout for a tile in which thread t owns the E keys at positions
// [E*t, E*t + E): groups of four keys stay together and group g of thread t
// sits at group g ^ (t & SW), so the 16-byte reads of eight neighbouring
// threads fall in different banks.
template <int E>
__device__ __forceinline__ uint32_t swz(uint32_t p) {
  constexpr uint32_t G = E / 4;
  constexpr uint32_t SW = G >= 8 ? 7 : G - 1;
  const uint32_t t = p / E;
  const uint32_t g = (p % E) >> 2;
  return E * t + 4 * (g ^ (t & SW)) + (p & 3);
}

// Keys of s[0, n) into LDS tile `keys` (swizzled for E keys per thread); with
// `hist`, the 12-bit histogram is counted too.
template <int E>
__device__ __forceinline__ void load_tile(const float* __restrict__ s, int n, bool vec4,
                                          uint32_t* keys, Shared* hist) {
  const int tid = threadIdx.x;
  int done = 0;
  if (vec4) {
    constexpr int U = (E >= 8 ? E / 4 : 1);  // float4 per thread in flight
    const int n4 = n / 4;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    for (int base = 0; base < n4; base += kThreads * U) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * kThreads + tid;
        v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * kThreads + tid;
        if (i < n4) {
          const uint4 kk = make_uint4(score_key(v[u].x), score_key(v[u].y), score_key(v[u].z),
                                      score_key(v[u].w));
          if (keys) *reinterpret_cast<uint4*>(&keys[swz<E>(4 * i)]) = kk;
          if (hist) {
            atomicAdd(&hist->hist[kk.x >> 20], 1u);
            atomicAdd(&hist->hist[kk.y >> 20], 1u);
            atomicAdd(&hist->hist[kk.z >> 20], 1u);
            atomicAdd(&hist->hist[kk.w >> 20], 1u);
          }
        }
      }
    }
    done = 4 * n4;
  }
  for (int p = done + tid; p < n; p += kThreads) {
    const uint32_t kk = score_key(s[p]);
    if (keys) keys[swz<E>(p)] = kk;
    if (hist) atomicAdd(&hist->hist[kk >> 20], 1u);
  }
}

// 12-bit histogram of s[0, n) from global memory (rows not kept in LDS).
__device__ __forceinline__ void hist_global(const float* __restrict__ s, int64_t n, bool vec4,
                                            Shared& sh) {
  const int tid = threadIdx.x;
  constexpr int U = 8;  // 8 x 16 bytes per thread in flight
  int64_t done = 0;
  if (vec4) {
    const int64_t n4 = n / 4;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    for (int64_t base = 0; base < n4; base += (int64_t)kThreads * U) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        if (i < n4) {
          atomicAdd(&sh.hist[score_key(v[u].x) >> 20], 1u);
          atomicAdd(&sh.hist[score_key(v[u].y) >> 20], 1u);
          atomicAdd(&sh.hist[score_key(v[u].z) >> 20], 1u);
          atomicAdd(&sh.hist[score_key(v[u].w) >> 20], 1u);
        }
      }
    }
    done = 4 * n4;
  }
  for (int64_t i = done + tid; i < n; i += kThreads) atomicAdd(&sh.hist[score_key(s[i]) >> 20], 1u);
}

// Digit passes over a whole row when the candidates overflow: T and need.
template <typename KeyAt>
__device__ void resolve_row(KeyAt key_at, int64_t n, uint32_t kleft, uint32_t prefix, uint32_t mask,
                            Shared& sh, uint32_t& T, uint32_t& need) {
  constexpr int kShift[3] = {12, 4, 0};
  constexpr int kWidth[3] = {8, 8, 4};
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    zero_hist(sh, 1 << kWidth[d]);
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix)
        atomicAdd(&sh.hist[(key >> kShift[d]) & ((1u << kWidth[d]) - 1u)], 1u);
    }
    __syncthreads();
    select_digit(sh, kShift[d], kWidth[d], prefix, mask, kleft);
  }
  T = prefix;
  need = kleft;
}

// Ordered write of one LDS tile (positions tile0 + [0, n_valid), E per
// thread): every key above T, and keys equal to T while fewer than `need`
// came before, go to out at slot = kept keys at lower positions (slots at or
// beyond k are never written).  run_gt / run_eq carry the counts of earlier
// tiles.  Contains barriers.
template <int E>
__device__ __forceinline__ void write_tile(const uint32_t* keys, int64_t tile0, int n_valid,
                                           uint32_t T, uint32_t need, uint32_t& run_gt,
                                           uint32_t& run_eq, int32_t* __restrict__ out,
                                           uint32_t k, Shared& sh) {
  static_assert(E % 4 == 0 && E <= 32, "E keys per thread in groups of four");
  constexpr int G = E / 4;
  constexpr int SW = G >= 8 ? 7 : G - 1;
  const int t = threadIdx.x;
  uint32_t key[E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 v = *reinterpret_cast<const uint4*>(&keys[E * t + 4 * (g ^ (t & SW))]);
    key[4 * g + 0] = v.x;
    key[4 * g + 1] = v.y;
    key[4 * g + 2] = v.z;
    key[4 * g + 3] = v.w;
  }
  uint32_t cg = 0, ce = 0, mg = 0, me = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool valid = E * t + j < n_valid;
    const bool gt = valid && key[j] > T;
    const bool eq = valid && key[j] == T;
    cg += gt ? 1u : 0u;
    ce += eq ? 1u : 0u;
    mg |= (gt ? 1u : 0u) << j;
    me |= (eq ? 1u : 0u) << j;
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan((cg << 16) | ce, sh, total);
  uint32_t gb = run_gt + (excl >> 16);
  uint32_t eb = run_eq + (excl & 0xffffu);
  uint32_t m = mg | me;
  while (m) {
    const int j = __builtin_ctz(m);
    m &= m - 1u;
    const int32_t pos = (int32_t)(tile0 + E * t + j);
    if ((mg >> j) & 1u) {
      const uint32_t slot = gb + std::min(eb, need);
      if (slot < k) out[slot] = pos;
      ++gb;
    } else {
      if (eb < need && gb + eb < k) out[gb + eb] = pos;
      ++eb;
    }
  }
  run_gt += total >> 16;
  run_eq += total & 0xffffu;
}

// Short-list finish of a long row (16-byte aligned rows, n % 4 == 0): one
// ordered pass over the row collects every key of bin d1 or above, with its
// position, into list (in position order; a workgroup prefix sum per chunk of
// 16384 keys, the next chunk's loads in flight meanwhile) and the keys of bin
// d1 into cand; the candidates are resolved, and the ordered write walks the
// list.  buf holds kListCap list pairs and kListCand candidate pairs.
constexpr int kListCap = 12288;
constexpr int kListCand = 4096;

__device__ void long_row_short_list(const float* __restrict__ s, int64_t n, int32_t k, uint32_t d1,
                                    uint32_t c1, uint32_t kleft, uint32_t prefix, uint32_t mask,
                                    int32_t* __restrict__ out, Shared& sh, uint32_t* buf) {
  uint2* list = reinterpret_cast<uint2*>(buf);
  uint2* cand = list + kListCap;
  const int tid = threadIdx.x;
  constexpr int KPT = 16;                  // keys per thread per chunk
  constexpr int CHUNK = KPT * kThreads;    // 16384
  const float4* s4 = reinterpret_cast<const float4*>(s);
  const int64_t n4 = n / 4;
  float4 v[KPT / 4];
  auto fetch = [&](int64_t c0) {
#pragma unroll
    for (int u = 0; u < KPT / 4; ++u) {
      const int64_t i = c0 / 4 + (int64_t)(KPT / 4) * tid + u;  // thread t: positions c0 + 16t ..
      v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  uint32_t list_base = 0, cand_base = 0;
  fetch(0);
  for (int64_t c0 = 0; c0 < n; c0 += CHUNK) {
    uint32_t key[KPT];
#pragma unroll
    for (int u = 0; u < KPT / 4; ++u) {
      key[4 * u + 0] = score_key(v[u].x);
      key[4 * u + 1] = score_key(v[u].y);
      key[4 * u + 2] = score_key(v[u].z);
      key[4 * u + 3] = score_key(v[u].w);
    }
    const int64_t p0 = c0 + (int64_t)KPT * tid;
    uint32_t n_ge = 0, n_c = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool ok = p0 + j < n;
      n_ge += (ok && (key[j] >> 20) >= d1) ? 1u : 0u;
      n_c += (ok && (key[j] >> 20) == d1) ? 1u : 0u;
    }
    if (c0 + CHUNK < n) fetch(c0 + CHUNK);  // in flight during the scan and the stores
    uint32_t total;
    const uint32_t excl = block_exclusive_scan((n_ge << 16) | n_c, sh, total);
    uint32_t at_l = list_base + (excl >> 16), at_c = cand_base + (excl & 0xffffu);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (p0 + j < n && (key[j] >> 20) >= d1) {
        const uint2 e = make_uint2(key[j], (uint32_t)(p0 + j));
        if (at_l < (uint32_t)kListCap) list[at_l] = e;
        ++at_l;
        if ((key[j] >> 20) == d1) {
          if (at_c < (uint32_t)kListCand) cand[at_c] = e;
          ++at_c;
        }
      }
    }
    list_base += total >> 16;
    cand_base += total & 0xffffu;
  }
  __syncthreads();
  uint32_t T, need;
  resolve(cand, c1, kleft, prefix, mask, sh, T, need);
  // ordered write over the list: thread t takes entries [E t, E t + E)
  const uint32_t L = min(list_base, (uint32_t)kListCap);
  const uint32_t E = (L + kThreads - 1) / kThreads;
  const uint32_t e0 = min(E * tid, L), e1 = min(e0 + E, L);
  uint32_t cg = 0, ce = 0;
  for (uint32_t i = e0; i < e1; ++i) {
    cg += list[i].x > T ? 1u : 0u;
    ce += list[i].x == T ? 1u : 0u;
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan((cg << 16) | ce, sh, total);
  uint32_t gb = excl >> 16, eb = excl & 0xffffu;
  for (uint32_t i = e0; i < e1; ++i) {
    const uint2 e = list[i];
    if (e.x > T) {
      const uint32_t slot = gb + std::min(eb, need);
      if (slot < (uint32_t)k) out[slot] = (int32_t)e.y;
      ++gb;
    } else if (e.x == T) {
      if (eb < need && gb + eb < (uint32_t)k) out[gb + eb] = (int32_t)e.y;
      ++eb;
    }
  }
}

// The row path for a row longer than kResident, by the whole workgroup: the
// row is read from global memory for the histogram, again for the candidates
// and, tile by tile through LDS, for the ordered write.
// buf: kTile keys + kCandGlob (key, position) pairs.
__device__ void topk_row_long(const float* __restrict__ s, int64_t n, int32_t k,
                              int32_t* __restrict__ out, bool vec4, Shared& sh, uint32_t* buf) {
  constexpr int E = kTile / kThreads;
  uint32_t* keys = buf;
  uint2* cand = reinterpret_cast<uint2*>(buf + kTile);
  constexpr uint32_t cap = kCandGlob;
  const int tid = threadIdx.x;
  auto key_at = [&](int64_t i) -> uint32_t { return score_key(s[i]); };

  // ---- 1. histogram of the top 12 bits
  zero_hist(sh, kBins);
  __syncthreads();
  hist_global(s, n, vec4, sh);
  __syncthreads();
  uint32_t prefix = 0, mask = 0, kleft = (uint32_t)k;
  const uint32_t c1 = select_digit(sh, 20, 12, prefix, mask, kleft);
  const uint32_t d1 = prefix >> 20;

  // ---- short-list path: every key in bin d1 or above (k - kleft + c1 of
  // them) is collected in position order in one pass, and the ordered write
  // walks that list instead of the row
  if (vec4 && n % 4 == 0 && (uint64_t)(k - kleft) + c1 <= (uint64_t)kListCap &&
      c1 <= (uint32_t)kListCand) {
    long_row_short_list(s, n, k, d1, c1, kleft, prefix, mask, out, sh, buf);
    return;
  }

  // ---- 2-3. candidates of bin d1, resolved to T and need
  uint32_t T, need;
  if (c1 <= cap) {
    if (tid == 0) sh.count = 0;
    __syncthreads();
    if (vec4 && n % 4 == 0) {
      // 16-byte loads, 32 keys per thread in flight; one LDS atomic per wave
      // places the wave's candidates
      constexpr int U = 8;
      const float4* s4 = reinterpret_cast<const float4*>(s);
      const int64_t n4 = n / 4;
      for (int64_t base = 0; base < n4; base += (int64_t)kThreads * U) {
        uint32_t kk[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = base + (int64_t)u * kThreads + tid;
          const float4 v = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
          kk[u][0] = score_key(v.x);
          kk[u][1] = score_key(v.y);
          kk[u][2] = score_key(v.z);
          kk[u][3] = score_key(v.w);
        }
        uint32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cnt += (base + (int64_t)u * kThreads + tid < n4 && (kk[u][e] >> 20) == d1) ? 1u : 0u;
        const uint32_t incl = wave_inclusive_scan(cnt);
        uint32_t at = 0;
        if ((tid & 63) == 63 && incl) at = atomicAdd(&sh.count, incl);
        at = __builtin_amdgcn_readlane(at, 63) + incl - cnt;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = base + (int64_t)u * kThreads + tid;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i < n4 && (kk[u][e] >> 20) == d1) {
              if (at < cap) cand[at] = make_uint2(kk[u][e], (uint32_t)(4 * i + e));
              ++at;
            }
        }
      }
    } else {
      constexpr int U = 8;
      for (int64_t base = 0; base < n; base += (int64_t)kThreads * U) {
        uint32_t kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = base + (int64_t)u * kThreads + tid;
          kk[u] = i < n ? key_at(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = base + (int64_t)u * kThreads + tid;
          if (i < n && (kk[u] >> 20) == d1) {
            const uint32_t at = atomicAdd(&sh.count, 1u);
            if (at < cap) cand[at] = make_uint2(kk[u], (uint32_t)i);
          }
        }
      }
    }
    __syncthreads();
    resolve(cand, c1, kleft, prefix, mask, sh, T, need);
  } else {
    resolve_row(key_at, n, kleft, prefix, mask, sh, T, need);
  }

  // ---- 4. ordered write, one LDS tile at a time
  uint32_t run_gt = 0, run_eq = 0;
  if (vec4 && n % 4 == 0) {
    // two LDS tiles (the candidate list is no longer needed): the next
    // tile's 16-byte loads are in flight while the current tile is written
    constexpr int U4 = E / 4;  // float4 per thread per tile
    const float4* s4 = reinterpret_cast<const float4*>(s);
    const int64_t n4 = n / 4;
    uint32_t* tiles[2] = {keys, buf + kTile};
    float4 v[U4];
    auto fetch = [&](int64_t tile0) {
#pragma unroll
      for (int u = 0; u < U4; ++u) {
        const int64_t i = tile0 / 4 + u * kThreads + tid;
        v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    __syncthreads();  // the candidate list is consumed
    fetch(0);
    int cur = 0;
    for (int64_t tile0 = 0; tile0 < n; tile0 += kTile) {
      const int nv = (int)std::min<int64_t>(kTile, n - tile0);
#pragma unroll
      for (int u = 0; u < U4; ++u) {
        const int i = u * kThreads + tid;  // float4 index inside the tile
        if (4 * i < nv)
          *reinterpret_cast<uint4*>(&tiles[cur][swz<E>(4 * i)]) =
              make_uint4(score_key(v[u].x), score_key(v[u].y), score_key(v[u].z), score_key(v[u].w));
      }
      __syncthreads();
      if (tile0 + kTile < n) fetch(tile0 + kTile);
      write_tile<E>(tiles[cur], tile0, nv, T, need, run_gt, run_eq, out, (uint32_t)k, sh);
      cur ^= 1;
    }
  } else {
    for (int64_t tile0 = 0; tile0 < n; tile0 += kTile) {
      const int nv = (int)std::min<int64_t>(kTile, n - tile0);
      __syncthreads();  // the previous tile is consumed
      load_tile<E>(s + tile0, nv, vec4, keys, nullptr);
      __syncthreads();
      write_tile<E>(keys, tile0, nv, T, need, run_gt, run_eq, out, (uint32_t)k, sh);
    }
  }
}

// ------------------------------------------------- register-resident rows
// Rows of at most 4 * G * NT keys: the register-resident row path of
// reg_row_topk, one workgroup per row.  With MAP the row is a candidate list
// and position p is reported as pos_map[p] (the merge of the fused
// score-and-select path); the map is staged in LDS next to the keys, so the
// ordered write does not wait on a global load per kept element.
template <int NT, int G, bool MAP>
__global__ __launch_bounds__(NT) void topk_reg_kernel(const float* __restrict__ scores, int64_t n64,
                                                      int64_t row_stride, int32_t k,
                                                      int32_t* __restrict__ idx_out, bool vec4,
                                                      const int32_t* __restrict__ pos_map) {
  __shared__ SharedT<NT> sh;
  __shared__ __align__(16) uint2 cand[kRankMax + 8];
  __shared__ uint32_t s_wave[NT / 64];
  __shared__ __align__(16) int32_t s_map[MAP ? 4 * G * NT : 4];
  const int n = (int)n64;  // <= 4 * G * NT
  const float* __restrict__ s = scores + (int64_t)blockIdx.x * row_stride;
  int32_t* __restrict__ out = idx_out + (int64_t)blockIdx.x * k;
  const int32_t* __restrict__ map = MAP ? pos_map + (int64_t)blockIdx.x * row_stride : nullptr;
  auto load = [&](int p0, float (&v)[G][4]) {
    if (vec4 && n % 4 == 0) {
      // a group lies wholly inside or wholly outside the row
      const float4* s4 = reinterpret_cast<const float4*>(s + p0);
      int4 m[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const bool in = p0 + 256 * j < n;
        const float4 f = in ? s4[64 * j] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (MAP) m[j] = in ? reinterpret_cast<const int4*>(map + p0)[64 * j] : make_int4(0, 0, 0, 0);
        v[j][0] = f.x;
        v[j][1] = f.y;
        v[j][2] = f.z;
        v[j][3] = f.w;
      }
      if (MAP) {
#pragma unroll
        for (int j = 0; j < G; ++j)
          *reinterpret_cast<int4*>(&s_map[p0 + 256 * j]) = m[j];
      }
    } else {
      const float* s1 = s + p0;
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool in = p0 + 256 * j + e < n;
          v[j][e] = in ? s1[256 * j + e] : 0.0f;
          if (MAP && in) s_map[p0 + 256 * j + e] = map[p0 + 256 * j + e];
        }
    }
  };
  // s_map is complete before the ordered write: reg_row_topk passes several
  // barriers between the load and the write
  auto emit = [&](uint32_t slot, int32_t p) { out[slot] = MAP ? s_map[p] : p; };
  reg_row_topk<NT, G, false>(load, n, k, emit, sh, cand, s_wave);
}

__global__ __launch_bounds__(kThreads) void topk_long_kernel(const float* __restrict__ scores,
                                                             int64_t n, int64_t row_stride,
                                                             int32_t k, int32_t* __restrict__ idx_out,
                                                             bool vec4) {
  __shared__ Shared sh;
  __shared__ __align__(16) uint32_t buf[kTile + 2 * kCandGlob];
  topk_row_long(scores + (int64_t)blockIdx.x * row_stride, n, k,
                idx_out + (int64_t)blockIdx.x * k, vec4, sh, buf);
}

// ------------------------------------------------- multi-workgroup path

// Per-row workspace.  The two lists hold runs by chunk: a chunk's entries in
// position order, the runs in whatever order the chunks arrived.
struct MwRow {
  uint32_t hist[kBins];             // 12-bit histogram of the row's keys
  uint32_t hist2[kBins];            // key bits 19..8 of the keys of bin d1
  uint32_t n_above_all, n_cand_all;  // list fill counters
  uint32_t sel_prefix, sel_kleft, sel_c1;  // bin d1 (as a key prefix), kleft, its count
  uint32_t pad_[59];
  uint32_t n_above[kMwMaxChunks];   // per chunk: keys above bin d1
  uint32_t above_at[kMwMaxChunks];  // per chunk: start of its run in `above`
  uint32_t n_cand[kMwMaxChunks];    // per chunk: keys of bin d1
  uint32_t cand_at[kMwMaxChunks];   // per chunk: start of its run in `cand`
  uint32_t above[kMwCand];          // positions of the keys above bin d1
  uint2 cand[kMwCand];              // (key, position) of the keys of bin d1
};

constexpr int kMwPer = kMwChunk / kThreads;  // consecutive positions per thread
static_assert(kMwChunk % (4 * kThreads) == 0, "whole float4 groups per thread");
static_assert(kMwMaxChunks <= kThreads, "one chunk per thread in the final scan");

__global__ __launch_bounds__(256) void topk_mw_zero(MwRow* rows) {
  MwRow& w = rows[blockIdx.x];
  for (int i = threadIdx.x; i < kBins; i += 256) {
    w.hist[i] = 0u;
    w.hist2[i] = 0u;
  }
  if (threadIdx.x == 0) {
    w.n_above_all = 0u;
    w.n_cand_all = 0u;
  }
}

__global__ __launch_bounds__(kThreads) void topk_mw_hist(const float* __restrict__ scores, int64_t n,
                                                         int64_t row_stride, bool vec4, MwRow* rows) {
  __shared__ Shared sh;
  const int64_t c0 = (int64_t)blockIdx.x * kMwChunk;
  zero_hist(sh, kBins);
  __syncthreads();
  load_tile<kMwChunk / kThreads>(scores + (int64_t)blockIdx.y * row_stride + c0,
                                 (int)std::min<int64_t>(kMwChunk, n - c0), vec4, nullptr, &sh);
  __syncthreads();
  uint32_t* g = rows[blockIdx.y].hist;
  for (int b = threadIdx.x; b < kBins; b += kThreads)
    if (sh.hist[b]) atomicAdd(&g[b], sh.hist[b]);
}

// d1's prefix and mask, kleft and the count of bin d1 from the finished
// per-row histogram.
__device__ __forceinline__ uint32_t mw_select(const MwRow& w, int32_t k, Shared& sh,
                                              uint32_t& prefix, uint32_t& mask, uint32_t& kleft) {
  for (int b = threadIdx.x; b < kBins; b += kThreads) sh.hist[b] = w.hist[b];
  __syncthreads();
  prefix = 0;
  mask = 0;
  kleft = (uint32_t)k;
  return select_digit(sh, 20, 12, prefix, mask, kleft);
}

// Every workgroup takes one chunk of kMwChunk positions, thread t the kMwPer
// consecutive ones from kMwPer * t, so that a block scan of per-thread counts
// lays the chunk's entries out in position order: the positions above bin d1
// go to `above`, the (key, position) pairs of bin d1 to `cand` (unless they
// overflow it: then the final launch runs the row path).
__global__ __launch_bounds__(kThreads) void topk_mw_collect(const float* __restrict__ scores,
                                                            int64_t n, int64_t row_stride,
                                                            int32_t k, bool vec4, MwRow* rows) {
  __shared__ Shared sh;
  MwRow& w = rows[blockIdx.y];
  const int ch = blockIdx.x;
  const int64_t p0 = (int64_t)ch * kMwChunk + (int64_t)kMwPer * threadIdx.x;
  const float* __restrict__ s = scores + (int64_t)blockIdx.y * row_stride;
  // the chunk's scores are loaded first: they arrive while the histogram is
  // read and scanned
  float v[kMwPer];
  if (vec4 && p0 + kMwPer <= n) {
#pragma unroll
    for (int e = 0; e < kMwPer; e += 4) {
      const float4 f = *reinterpret_cast<const float4*>(s + p0 + e);
      v[e] = f.x;
      v[e + 1] = f.y;
      v[e + 2] = f.z;
      v[e + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kMwPer; ++e) v[e] = p0 + e < n ? s[p0 + e] : 0.0f;
  }
  uint32_t prefix, mask, kleft;
  const uint32_t c1 = mw_select(w, k, sh, prefix, mask, kleft);
  const uint32_t d1 = prefix >> 20;
  const bool keep = c1 <= (uint32_t)kMwCand;
  if (ch == 0 && threadIdx.x == 0) {
    w.sel_prefix = prefix;
    w.sel_kleft = kleft;
    w.sel_c1 = c1;
  }
  uint32_t key[kMwPer];
#pragma unroll
  for (int e = 0; e < kMwPer; ++e) key[e] = score_key(v[e]);
  uint32_t na = 0, nc = 0;
#pragma unroll
  for (int e = 0; e < kMwPer; ++e) {
    const bool valid = p0 + e < n;
    na += (valid && (key[e] >> 20) > d1) ? 1u : 0u;
    nc += (valid && (key[e] >> 20) == d1) ? 1u : 0u;
  }
  uint32_t total;  // both halves stay below 2^16 (at most kMwChunk each)
  const uint32_t excl = block_exclusive_scan((na << 16) | nc, sh, total);
  if (threadIdx.x == 0) {
    const uint32_t ta = total >> 16, tc = keep ? (total & 0xffffu) : 0u;
    const uint32_t at_a = ta ? atomicAdd(&w.n_above_all, ta) : 0u;
    const uint32_t at_c = tc ? atomicAdd(&w.n_cand_all, tc) : 0u;
    w.n_above[ch] = ta;
    w.above_at[ch] = at_a;
    w.n_cand[ch] = tc;
    w.cand_at[ch] = at_c;
    sh.base = at_a;
    sh.cgt = at_c;
  }
  __syncthreads();
  uint32_t pa = sh.base + (excl >> 16), pc = sh.cgt + (excl & 0xffffu);
#pragma unroll
  for (int e = 0; e < kMwPer; ++e) {
    if (p0 + e >= n) continue;
    const uint32_t d = key[e] >> 20;
    if (d > d1) {
      w.above[pa++] = (uint32_t)(p0 + e);
    } else if (keep && d == d1) {
      w.cand[pc++] = make_uint2(key[e], (uint32_t)(p0 + e));
      atomicAdd(&w.hist2[(key[e] >> 8) & (kBins - 1)], 1u);
    }
  }
}

// First index in [lo, hi) whose value is >= x (a[] ascending).
__device__ __forceinline__ uint32_t lower_bound_u32(const uint32_t* a, uint32_t lo, uint32_t hi,
                                                    uint32_t x) {
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// LDS of the final launch: the row path's buffers, or the lists in chunk order.
constexpr int kMwArena = kTile + 2 * kCandGlob;
static_assert(4 * (kMwMaxChunks + 1) + kMwCand + 2 * (kMwCand + 32) + 2 * (kRankCap + 32) <= kMwArena,
              "the chunk tables, both lists and the sub-bin list fit the row path's LDS");

// One workgroup per row: the lists are gathered into LDS in chunk order (so
// both are in position order), the candidates resolved into T and `need`,
// each candidate marked kept or not, and every kept position written to its
// output slot = (kept positions of earlier chunks) + (earlier ones of its own
// list in its chunk) + (those of the other list in its chunk below it, by
// binary search).
__global__ __launch_bounds__(kThreads) void topk_mw_finish(const float* __restrict__ scores,
                                                           int64_t n, int64_t row_stride, int32_t k,
                                                           bool vec4, MwRow* rows,
                                                           int32_t* __restrict__ idx_out) {
  __shared__ Shared sh;
  __shared__ __align__(16) uint32_t arena[kMwArena];
  MwRow& w = rows[blockIdx.x];
  int32_t* __restrict__ out = idx_out + (int64_t)blockIdx.x * k;
  const int tid = threadIdx.x;
  const int nch = (int)((n + kMwChunk - 1) / kMwChunk);
  // the chunk table is loaded first: it arrives while the histogram is read
  // and scanned
  // the selection scalars, the chunk table and the second-level histogram
  // are all loaded at once
  uint32_t na = 0, nc = 0, at_a = 0, at_c = 0;
  if (tid < nch) {
    na = w.n_above[tid];
    nc = w.n_cand[tid];
    at_a = w.above_at[tid];
    at_c = w.cand_at[tid];
  }
  const uint32_t prefix = w.sel_prefix, kleft = w.sel_kleft, c1 = w.sel_c1;
  for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = w.hist2[b];
  if (c1 > (uint32_t)kMwCand) {
    topk_row_long(scores + (int64_t)blockIdx.x * row_stride, n, k, out, vec4, sh, arena);
    return;
  }
  uint32_t* a_off = arena;                              // [nch + 1]
  uint32_t* c_off = arena + (kMwMaxChunks + 1);         // [nch + 1]
  uint32_t* a_at = arena + 2 * (kMwMaxChunks + 1);      // [nch]
  uint32_t* c_at = arena + 3 * (kMwMaxChunks + 1);      // [nch]
  uint32_t* above = arena + 4 * (kMwMaxChunks + 1);     // [k - kleft]
  uint2* cand = reinterpret_cast<uint2*>(above + kMwCand);  // [c1, padded]
  const uint32_t v = (na << 16) | nc;
  if (tid < nch) {
    a_at[tid] = at_a;
    c_at[tid] = at_c;
  }
  uint32_t total;
  const uint32_t excl = block_exclusive_scan(v, sh, total);
  if (tid < nch) {
    a_off[tid] = excl >> 16;
    c_off[tid] = excl & 0xffffu;
  }
  if (tid == 0) {
    a_off[nch] = total >> 16;
    c_off[nch] = total & 0xffffu;
  }
  __syncthreads();
  const uint32_t n_above = a_off[nch];  // = k - kleft
  // gather both lists in chunk order: thread t takes entries [kG t, kG t +
  // kG) of each, finds the chunk of its first entry by binary search and
  // walks forward; every load is in flight before any is stored
  constexpr int kG = kMwCand / kThreads;
  uint32_t src_a[kG], src_c[kG];
  {
    const uint32_t i0 = (uint32_t)tid * kG;
    uint32_t ca = i0 < n_above ? lower_bound_u32(a_off, 0, (uint32_t)nch + 1, i0 + 1) - 1 : 0u;
    uint32_t cc = i0 < c1 ? lower_bound_u32(c_off, 0, (uint32_t)nch + 1, i0 + 1) - 1 : 0u;
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const uint32_t i = i0 + u;
      src_a[u] = src_c[u] = 0u;
      if (i < n_above) {
        while (a_off[ca + 1] <= i) ++ca;
        src_a[u] = a_at[ca] + (i - a_off[ca]);
      }
      if (i < c1) {
        while (c_off[cc + 1] <= i) ++cc;
        src_c[u] = c_at[cc] + (i - c_off[cc]);
      }
    }
  }
  uint32_t ga[kG];
  uint2 gc[kG];
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    ga[u] = w.above[src_a[u]];
    gc[u] = w.cand[src_c[u]];
  }
#pragma unroll
  for (int u = 0; u < kG; ++u) {
    const uint32_t i = (uint32_t)tid * kG + u;
    if (i < n_above) above[i] = ga[u];
    if (i < c1) cand[i] = gc[u];
  }
  // the second digit (key bits 19..8) from the collected histogram of bin
  // d1; its keys (the sub-bin) are copied to `sub` and resolved there
  // (wave 0 finds it and hands it to the other waves, as the register top-k
  // does; after the barrier resolve may reuse sh.hist)
  if ((tid >> 6) == 0) {
    uint32_t a, c;
    const uint32_t d = wave_select_bin<kBins>(sh.hist, kleft, &a, &c);
    if (tid == 0) {
      sh.bc[0] = d;
      sh.bc[1] = a;
      sh.bc[2] = c;
    }
  }
  __syncthreads();
  const uint32_t d2 = sh.bc[0], above2 = sh.bc[1], c2 = sh.bc[2];
  const uint32_t kleft2 = kleft - above2;
  const uint32_t prefix2 = prefix | (d2 << 8), mask2 = 0xffffff00u;
  uint2* sub = cand + (kMwCand + 32);  // [c2 <= kRankCap, padded]
  const bool small = c2 <= (uint32_t)kRankCap;
  uint32_t T, need;
  if (small) {
    if (tid == 0) sh.count = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const uint32_t i = (uint32_t)tid * kG + u;
      if (i < c1 && (gc[u].x & mask2) == prefix2) sub[atomicAdd(&sh.count, 1u)] = gc[u];
    }
    __syncthreads();
    resolve(sub, c2, kleft2, prefix2, mask2, sh, T, need);
  } else {
    // many keys share the second digit: resolve bin d1 as a whole
    resolve(cand, c1, kleft, prefix, 0xfff00000u, sh, T, need);
  }
  // keep: key above T, or equal to T among the first `need` such in
  // position order; cand[j].x becomes (kept candidates before j) << 1 | kept
  constexpr uint32_t kPerC = (kMwCand + kThreads - 1) / kThreads;
  const uint32_t j0 = tid * kPerC, j1 = std::min<uint32_t>(j0 + kPerC, c1);
  uint32_t flags = 0, nk = 0;
  if (small) {
    // few keys share T's top 24 bits: a tied key's rank among them by a scan of `sub`
    for (uint32_t j = j0; j < j1; ++j) {
      const uint2 e = cand[j];
      bool kept = e.x > T;
      if (e.x == T) {
        uint32_t r = 0;
        for (uint32_t m = 0; m < c2; ++m) r += (sub[m].x == T && sub[m].y < e.y) ? 1u : 0u;
        kept = r < need;
      }
      flags |= (kept ? 1u : 0u) << (j - j0);
      nk += kept ? 1u : 0u;
    }
  } else {
    uint32_t ne = 0;
    for (uint32_t j = j0; j < j1; ++j) ne += cand[j].x == T ? 1u : 0u;
    uint32_t eq_before = block_exclusive_scan(ne, sh, total);
    for (uint32_t j = j0; j < j1; ++j) {
      const uint32_t key = cand[j].x;
      const bool kept = key > T || (key == T && eq_before++ < need);
      flags |= (kept ? 1u : 0u) << (j - j0);
      nk += kept ? 1u : 0u;
    }
  }
  uint32_t kept_before = block_exclusive_scan(nk, sh, total);
  for (uint32_t j = j0; j < j1; ++j) {
    const uint32_t kept = (flags >> (j - j0)) & 1u;
    cand[j].x = (kept_before << 1) | kept;
    kept_before += kept;
  }
  __syncthreads();
  auto kept_upto = [&](uint32_t j) { return j < c1 ? cand[j].x >> 1 : kleft; };
  auto cand_pos_lb = [&](uint32_t lo, uint32_t hi, uint32_t x) {
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (cand[mid].y < x) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  for (uint32_t i = tid; i < n_above; i += kThreads) {
    const uint32_t p = above[i];
    const uint32_t c = p / (uint32_t)kMwChunk;
    const uint32_t before = a_off[c] + kept_upto(c_off[c]);
    const uint32_t below = kept_upto(cand_pos_lb(c_off[c], c_off[c + 1], p)) - kept_upto(c_off[c]);
    const uint32_t slot = before + (i - a_off[c]) + below;
    if (slot < (uint32_t)k) out[slot] = (int32_t)p;
  }
  for (uint32_t j = tid; j < c1; j += kThreads) {
    const uint2 e = cand[j];
    if (!(e.x & 1u)) continue;
    const uint32_t c = e.y / (uint32_t)kMwChunk;
    const uint32_t before = a_off[c] + kept_upto(c_off[c]);
    const uint32_t below = lower_bound_u32(above, a_off[c], a_off[c + 1], e.y) - a_off[c];
    const uint32_t slot = before + ((e.x >> 1) - kept_upto(c_off[c])) + below;
    if (slot < (uint32_t)k) out[slot] = (int32_t)e.y;
  }
}

bool use_mw(int64_t n_rows, int64_t n, int32_t k) {
  return n > kResident && n_rows <= kMwMaxRows && n <= (int64_t)kMwChunk * kMwMaxChunks &&
         k <= kMwCand;
}

}  // namespace

// ---------------------------------------------------------------------------
// Overlap of two ascending index sets per row: each thread takes entries of
// row b and binary-searches them in row a (staged in LDS when it fits).
constexpr int kOverlapThreads = 256;
constexpr int kOverlapLds = 8192;

__device__ __forceinline__ bool sorted_contains(const int32_t* a, int32_t k, int32_t x) {
  int32_t lo = 0, hi = k;  // search [lo, hi)
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    const int32_t v = a[mid];
    if (v == x) return true;
    if (v < x) lo = mid + 1;
    else hi = mid;
  }
  return false;
}

__global__ __launch_bounds__(kOverlapThreads) void index_overlap_kernel(const int32_t* __restrict__ ia,
                                                                        const int32_t* __restrict__ ib,
                                                                        int32_t k,
                                                                        int32_t* __restrict__ counts) {
  __shared__ int32_t s_a[kOverlapLds];
  __shared__ int32_t s_cnt[kOverlapThreads / 64];
  const int64_t row = blockIdx.x;
  const int32_t* a = ia + row * k;
  const int32_t* b = ib + row * k;
  const bool in_lds = k <= kOverlapLds;
  if (in_lds) {
    for (int32_t i = threadIdx.x; i < k; i += kOverlapThreads) s_a[i] = a[i];
    __syncthreads();
  }
  int32_t c = 0;
  for (int32_t i = threadIdx.x; i < k; i += kOverlapThreads) {
    const int32_t x = b[i];
    c += (in_lds ? sorted_contains(s_a, k, x) : sorted_contains(a, k, x)) ? 1 : 0;
  }
  // wave sum, then the workgroup's waves
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t t = 0;
    for (int w = 0; w < kOverlapThreads / 64; ++w) t += s_cnt[w];
    counts[row] = t;
  }
}

hipError_t launch_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int32_t k,
                                int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(index_overlap_kernel, dim3((unsigned)n_rows), dim3(kOverlapThreads), 0, s,
                     idx_a, idx_b, k, counts);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int64_t n_rows, int64_t n, int32_t k) {
  return use_mw(n_rows, n, k) ? (size_t)n_rows * sizeof(MwRow) : 0;
}

bool topk_counted(int64_t n_rows, int64_t n, int32_t k) { return use_mw(n_rows, n, k); }

uint32_t* topk_counted_hist(void* ws, int64_t* stride_words) {
  *stride_words = (int64_t)(sizeof(MwRow) / sizeof(uint32_t));
  return static_cast<MwRow*>(ws)->hist;
}

hipError_t launch_topk_counted_zero(void* ws, int64_t n_rows, hipStream_t s) {
  hipLaunchKernelGGL(topk_mw_zero, dim3((unsigned)n_rows), dim3(256), 0, s, static_cast<MwRow*>(ws));
  return hipGetLastError();
}

hipError_t launch_topk_counted(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride,
                               int32_t k, int32_t* idx, void* ws, hipStream_t s) {
  const bool vec4 = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (row_stride % 4 == 0);
  MwRow* rows = static_cast<MwRow*>(ws);
  const dim3 grid((unsigned)((n + kMwChunk - 1) / kMwChunk), (unsigned)n_rows);
  hipLaunchKernelGGL(topk_mw_collect, grid, dim3(kThreads), 0, s, scores, n, row_stride, k, vec4,
                     rows);
  hipLaunchKernelGGL(topk_mw_finish, dim3((unsigned)n_rows), dim3(kThreads), 0, s, scores, n,
                     row_stride, k, vec4, rows, idx);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const float* cand_val, const int32_t* cand_pos, int64_t n_rows,
                             int64_t n, int64_t cstride, int32_t k, int32_t* idx, hipStream_t s) {
  const bool vec4 = (reinterpret_cast<uintptr_t>(cand_val) % 16 == 0) && (cstride % 4 == 0);
  // the fewest keys per thread that hold the row
  if (n <= 4 * 2 * 512)
    hipLaunchKernelGGL((topk_reg_kernel<512, 2, true>), dim3((unsigned)n_rows), dim3(512), 0, s,
                       cand_val, n, cstride, k, idx, vec4, cand_pos);
  else if (n <= 4 * 4 * 512)
    hipLaunchKernelGGL((topk_reg_kernel<512, 4, true>), dim3((unsigned)n_rows), dim3(512), 0, s,
                       cand_val, n, cstride, k, idx, vec4, cand_pos);
  else
    hipLaunchKernelGGL((topk_reg_kernel<kThreads, 8, true>), dim3((unsigned)n_rows), dim3(kThreads),
                       0, s, cand_val, n, cstride, k, idx, vec4, cand_pos);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride, int32_t k,
                       int32_t* idx, void* ws, hipStream_t s) {
  // 16-byte loads when every row starts 16-byte aligned
  const bool vec4 = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (row_stride % 4 == 0);
  if (n <= kResident) {
    // the fewest keys per thread that hold the row: short rows (block scores,
    // merges) do not pay for 32 keys per thread on 16 waves
    if (n <= 4 * 1 * 256)
      hipLaunchKernelGGL((topk_reg_kernel<256, 1, false>), dim3((unsigned)n_rows), dim3(256), 0, s,
                         scores, n, row_stride, k, idx, vec4, nullptr);
    else if (n <= 4 * 2 * 512)
      hipLaunchKernelGGL((topk_reg_kernel<512, 2, false>), dim3((unsigned)n_rows), dim3(512), 0, s,
                         scores, n, row_stride, k, idx, vec4, nullptr);
    else if (n <= 4 * 4 * 512)
      hipLaunchKernelGGL((topk_reg_kernel<512, 4, false>), dim3((unsigned)n_rows), dim3(512), 0, s,
                         scores, n, row_stride, k, idx, vec4, nullptr);
    else
      hipLaunchKernelGGL((topk_reg_kernel<kThreads, 8, false>), dim3((unsigned)n_rows),
                         dim3(kThreads), 0, s, scores, n, row_stride, k, idx, vec4, nullptr);
  } else if (use_mw(n_rows, n, k)) {
    MwRow* rows = static_cast<MwRow*>(ws);
    const dim3 grid((unsigned)((n + kMwChunk - 1) / kMwChunk), (unsigned)n_rows);
    hipLaunchKernelGGL(topk_mw_zero, dim3((unsigned)n_rows), dim3(256), 0, s, rows);
    hipLaunchKernelGGL(topk_mw_hist, grid, dim3(kThreads), 0, s, scores, n, row_stride, vec4, rows);
    return launch_topk_counted(scores, n_rows, n, row_stride, k, idx, ws, s);
  } else {
    hipLaunchKernelGGL(topk_long_kernel, dim3((unsigned)n_rows), dim3(kThreads), 0, s, scores, n,
                       row_stride, k, idx, vec4);
  }
  return hipGetLastError();
}

}  // namespace sa
