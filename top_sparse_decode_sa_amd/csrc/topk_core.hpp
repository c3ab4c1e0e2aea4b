// Radix-select building blocks shared by the top-k kernels (topk.hip) and the
// fused score-and-select kernel (select.hip), for workgroups of NT threads.
//
// The selection is the exact top-k of "Inference-time context sparsity:
// illusion or opportunity?" (section 2, oracle top-k) and "Flash Attention vs
// Sparse Attention" (DSA Stage 1, a top-K index list): the k positions with
// the largest scores, equal scores taken from the lower position, returned in
// ascending position order.  Keys are the order-preserving uint32 images of
// the scores (score_key).
#pragma once

#include <algorithm>

#include "common.hpp"

namespace sa {
namespace {

constexpr int kBins = 4096;    // first digit: 12 bits
constexpr int kRankCap = 256;  // candidates resolved by pairwise ranking

constexpr int kRankMax = 64;   // candidates ranked pairwise by one wave (register rows)

template <int NT>
struct SharedT {
  uint32_t hist[kBins];
  uint32_t hist2[3][256];  // digit passes of a register row, one histogram per pass
  uint32_t tot[NT / 64];
  uint32_t digit, above, count, T, cgt, base;
  uint32_t bc[4];  // a leader wave's selection, broadcast to the workgroup
};

// Workgroup-wide exclusive prefix sum; also returns the total.  Uses sh.tot
// as scratch; contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, SharedT<NT>& sh,
                                                         uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) sh.tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t t = sh.tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ void zero_hist(SharedT<NT>& sh, int bins) {
  for (int i = threadIdx.x; i < bins; i += NT) sh.hist[i] = 0u;
}

// Pick the digit (of `width` bits at `shift`) of the kleft-th largest key among
// those counted in sh.hist; updates prefix/mask/kleft and returns the count of
// keys with that digit.  Called by every thread; contains barriers.
template <int NT>
__device__ __forceinline__ uint32_t select_digit(SharedT<NT>& sh, int shift, int width,
                                                 uint32_t& prefix, uint32_t& mask,
                                                 uint32_t& kleft) {
  const int tid = threadIdx.x;
  const int bins = 1 << width;
  const int per = (bins + NT - 1) / NT;  // bins per thread, descending
  uint32_t c[16];
  uint32_t csum = 0;
#pragma unroll
  for (int j = 0; j < kBins / NT; ++j) {
    const int d = bins - 1 - (tid * per + j);
    c[j] = (j < per && d >= 0) ? sh.hist[d] : 0u;
    csum += c[j];
  }
  uint32_t total;
  uint32_t excl = block_exclusive_scan(csum, sh, total);
#pragma unroll
  for (int j = 0; j < kBins / NT; ++j) {
    const int d = bins - 1 - (tid * per + j);
    if (j < per && d >= 0 && excl < kleft && kleft <= excl + c[j]) {
      sh.digit = (uint32_t)d;
      sh.above = excl;
      sh.count = c[j];
    }
    excl += c[j];
  }
  __syncthreads();
  prefix |= sh.digit << shift;
  mask |= (uint32_t)(bins - 1) << shift;
  kleft -= sh.above;
  const uint32_t cnt = sh.count;
  __syncthreads();
  return cnt;
}

// Resolve the candidates cand[0, c1) (key, position) of the bin fixed by
// (prefix, mask), of which kleft1 belong to the result: T, the key of the
// last kept candidate in selection order, and `need`, the kept candidates
// equal to T.  Up to RANK candidates are ranked pairwise, NT / RANK threads
// each; more go through 8/8/4-bit digit passes.  cand must have room for c1
// rounded up to 32.
template <int NT, int RANK = kRankCap>
__device__ void resolve(uint2* cand, uint32_t c1, uint32_t kleft1, uint32_t prefix, uint32_t mask,
                        SharedT<NT>& sh, uint32_t& T, uint32_t& need) {
  static_assert(RANK <= NT && NT % RANK == 0, "whole threads per ranked candidate");
  constexpr int TPC = NT / RANK;  // threads per ranked candidate
  constexpr uint32_t kCap = RANK;
  const int tid = threadIdx.x;
  if (c1 <= kCap) {
    // rank = candidates with a larger key or an equal key at a lower
    // position; TPC threads per candidate, each over a share of the list
    const uint32_t c1p = (c1 + 31u) & ~31u;
    for (uint32_t c = c1 + tid; c < c1p; c += NT) cand[c] = make_uint2(0u, 0xffffffffu);
    __syncthreads();
    const uint32_t ci = tid / TPC, part = tid % TPC;
    const uint2 me = cand[ci < c1 ? ci : 0];
    uint32_t rank = 0;
    if (ci < c1) {
      const uint32_t q = c1p / TPC;
      for (uint32_t j0 = part * q; j0 < (part + 1) * q; j0 += 8) {
        uint2 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = cand[j0 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          rank += (o[u].x > me.x || (o[u].x == me.x && o[u].y < me.y)) ? 1u : 0u;
      }
    }
#pragma unroll
    for (int m = 1; m < TPC; m <<= 1) rank += __shfl_xor(rank, m, 64);
    if (ci < c1 && part == 0 && rank == kleft1 - 1) sh.T = me.x;
    __syncthreads();
    T = sh.T;
  } else {
    constexpr int kShift[3] = {12, 4, 0};
    constexpr int kWidth[3] = {8, 8, 4};
    uint32_t kleft = kleft1;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      zero_hist(sh, 1 << kWidth[d]);
      __syncthreads();
      for (uint32_t c = tid; c < c1; c += NT) {
        const uint32_t key = cand[c].x;
        if ((key & mask) == prefix)
          atomicAdd(&sh.hist[(key >> kShift[d]) & ((1u << kWidth[d]) - 1u)], 1u);
      }
      __syncthreads();
      select_digit(sh, kShift[d], kWidth[d], prefix, mask, kleft);
    }
    T = prefix;
  }
  if (tid == 0) sh.cgt = 0;
  __syncthreads();
  uint32_t g = 0;
  for (uint32_t c = tid; c < c1; c += NT) g += cand[c].x > T ? 1u : 0u;
  if (g) atomicAdd(&sh.cgt, g);
  __syncthreads();
  need = kleft1 - sh.cgt;  // kept candidates: those above T and `need` equal to T
}

// Digit select by one wave, on its own (every wave of a workgroup can run it
// on the same histogram and reach the same answer without a barrier): the
// bin d of histogram h (B bins, higher bin = larger keys) that holds the
// kleft-th largest key, with *above = keys in bins above d and *cnt = keys in
// bin d.  Needs 1 <= kleft <= the histogram's total.  For B >= 64 lane l sums
// the B/64 bins B-1-(l*B/64 + i) -- read in a rotated order so the 64 lanes
// of one read hit 64 different banks --, a wave prefix sum finds the lane
// whose bins hold the kleft-th key, and a second prefix sum over that lane's
// bins (one per lane) finds the bin.
template <int B>
__device__ __forceinline__ uint32_t wave_select_bin(const uint32_t* h, uint32_t kleft,
                                                    uint32_t* above, uint32_t* cnt) {
  constexpr int PER = B >= 64 ? B / 64 : 1;  // bins per lane
  constexpr int LANES = B >= 64 ? 64 : B;    // lanes holding bins
  const int lane = threadIdx.x & 63;
  constexpr int BATCH = PER < 16 ? PER : 16;  // reads in flight per lane
  uint32_t s = 0;
  if (lane < LANES) {
#pragma unroll 1
    for (int i0 = 0; i0 < PER; i0 += BATCH) {
#pragma unroll
      for (int i = i0; i < i0 + BATCH; ++i) s += h[B - 1 - (lane * PER + ((i + lane) & (PER - 1)))];
    }
  }
  const uint32_t incl = wave_inclusive_scan(s);
  const uint64_t hit = __ballot(incl - s < kleft && kleft <= incl);
  const int L = __builtin_ctzll(hit);
  const uint32_t base = __shfl(incl - s, L, 64);
  uint32_t d, a, c;
  if constexpr (PER == 1) {
    d = (uint32_t)(B - 1 - L);
    a = base;
    c = __shfl(s, L, 64);
  } else {
    const uint32_t v = lane < PER ? h[B - 1 - (L * PER + lane)] : 0u;
    const uint32_t vi = wave_inclusive_scan(v);
    const uint64_t hit2 = __ballot(lane < PER && base + vi - v < kleft && kleft <= base + vi);
    const int j = __builtin_ctzll(hit2);
    d = (uint32_t)(B - 1 - (L * PER + j));
    a = base + __shfl(vi - v, j, 64);
    c = __shfl(v, j, 64);
  }
  *above = a;
  *cnt = c;
  return d;
}

// Top-k of a row of n <= 4 * G * NT keys held in registers, 4 G per thread:
// every key stays in the thread that loaded it, so no phase after the load
// touches the row in memory.  Wave w holds positions [256 G w, 256 G (w+1));
// in group j (0..G-1) lane l holds the four positions 256 G w + 256 j + 4 l +
// e, so positions run in (j, lane, e) order inside a wave.
//
//   load(p0, v): fills v[j][e] (float[G][4]) with the score at position p0 + 256 j + e
//     (any value where that position is >= n);
//   emit(slot, p): the kept position p goes to output slot `slot` < k;
//   HIST: sh.hist already holds the 12-bit histogram of the row's keys (the
//     caller counted them as they were produced), so the load adds nothing.
//
// Phases; wave 0 finds each digit (wave_select_bin) and ranks the last
// candidates, and hands the result to the other waves through LDS (one wave's
// scans instead of every wave's: with several waves per SIMD the repeated
// scans cost more issue cycles than the barriers that broadcast the result):
//   1. histogram of the top 12 key bits; the bin d1 of the k-th largest key;
//   2. within bin d1, 8-, 8- and 4-bit digit passes over the keys still
//      matching (one histogram each) until at most kRankMax keys remain or all
//      bits are fixed; the rest are ranked pairwise by (key, position).  This
//      gives T, the key of the last kept element in selection order, and
//      `need`, the kept keys equal to T;
//   3. the ordered write, where a key's slot is (kept keys of earlier waves)
//      + (of earlier groups of its wave) + (of lower lanes in its group, a
//      DPP prefix sum) + (of lower e in its lane).
// Needs 1 <= k <= n; cand has room for kRankMax + 4 entries.
template <int NT, int G, bool HIST = false, typename Load, typename Emit>
__device__ __forceinline__ void reg_row_topk(Load load, int n, int32_t k, Emit emit,
                                             SharedT<NT>& sh, uint2* cand, uint32_t* s_wave) {
  constexpr int kW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p0 = wave * (G * 256) + 4 * lane;  // position of (j = 0, e = 0)
  auto pos = [&](int j, int e) { return p0 + 256 * j + e; };

  // ---- 1. load (every load issued first) and the 12-bit histogram, each
  // group counted as soon as its load arrives
  for (int i = tid; i < 3 * 256; i += NT) sh.hist2[i >> 8][i & 255] = 0u;
  if (tid == 0) sh.count = 0u;
  if (!HIST) {
    zero_hist(sh, kBins);
    __syncthreads();
  }
  uint32_t key[G][4];
  {
    float v[G][4];
    load(p0, v);
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        key[j][e] = score_key(v[j][e]);
        if (!HIST && pos(j, e) < n) atomicAdd(&sh.hist[key[j][e] >> 20], 1u);
      }
  }
  __syncthreads();
  // wave 0 finds the digit and hands it to the others (one wave's scan of
  // the histogram instead of every wave's)
  if (wave == 0) {
    uint32_t a0, c0;
    const uint32_t d0 = wave_select_bin<kBins>(sh.hist, (uint32_t)k, &a0, &c0);
    if (lane == 0) {
      sh.bc[0] = d0;
      sh.bc[1] = a0;
      sh.bc[2] = c0;
    }
  }
  __syncthreads();
  const uint32_t d1 = sh.bc[0];
  const uint32_t above = sh.bc[1];
  uint32_t cnt = sh.bc[2];
  uint32_t kleft = (uint32_t)k - above;
  uint32_t prefix = d1 << 20, mask = 0xfff00000u;

  // per-thread bit masks over its keys (bit 4j + e): m_above = keys in bins
  // above d1 (all kept), m_cand = keys of bin d1
  uint32_t m_above = 0, m_cand = 0;
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = pos(j, e) < n;
      const uint32_t d = key[j][e] >> 20;
      m_above |= (ok && d > d1) ? 1u << (4 * j + e) : 0u;
      m_cand |= (ok && d == d1) ? 1u << (4 * j + e) : 0u;
    }

  // ---- 2. T and need inside bin d1: digits of 8, 8 and 4 bits below the
  // first 12 (shift 12, 4, 0)
  uint32_t T = 0, need = 0;
  bool resolved = false;
#pragma unroll 1
  for (int level = 0; level < 3; ++level) {
    if (cnt <= (uint32_t)kRankMax) break;
    const int shift = level == 0 ? 12 : (level == 1 ? 4 : 0);
    const uint32_t dmask = level == 2 ? 0xfu : 0xffu;
    uint32_t* h2 = sh.hist2[level];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (((m_cand >> (4 * j + e)) & 1u) && (key[j][e] & mask) == prefix)
          atomicAdd(&h2[(key[j][e] >> shift) & dmask], 1u);
    __syncthreads();
    if (wave == 0) {
      uint32_t a, c, d;
      if (level < 2)
        d = wave_select_bin<256>(h2, kleft, &a, &c);
      else
        d = wave_select_bin<16>(h2, kleft, &a, &c);
      if (lane == 0) {
        sh.bc[0] = d;
        sh.bc[1] = a;
        sh.bc[2] = c;
      }
    }
    __syncthreads();
    // (bc is written again only after the next level's or the ranking's
    // barrier, which every wave reaches after this read)
    const uint32_t d2 = sh.bc[0], a2 = sh.bc[1], c2 = sh.bc[2];
    prefix |= d2 << shift;
    mask |= dmask << shift;
    kleft -= a2;
    cnt = c2;
    if (level == 2) {
      // every bit fixed: the keys left all equal prefix
      T = prefix;
      need = kleft;
      resolved = true;
    }
  }
  if (!resolved) {
    // at most kRankMax keys match (prefix, mask): into LDS, then every wave
    // ranks them, lane i the i-th (rank = keys larger, or equal at a lower
    // position); the lane of rank kleft - 1 holds T
    uint32_t m_match = 0;
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m_match |= (((m_cand >> (4 * j + e)) & 1u) && (key[j][e] & mask) == prefix)
                       ? 1u << (4 * j + e) : 0u;
    const uint32_t mine_n = __builtin_popcount(m_match);
    const uint32_t incl = wave_inclusive_scan(mine_n);
    uint32_t base = 0;
    if (lane == 63 && incl) base = atomicAdd(&sh.count, incl);
    base = __builtin_amdgcn_readlane(base, 63) + incl - mine_n;
    while (m_match) {
      const int bit = __builtin_ctz(m_match);
      m_match &= m_match - 1u;
      uint32_t kv = key[0][0];
#pragma unroll
      for (int t = 1; t < 4 * G; ++t) kv = bit == t ? key[t >> 2][t & 3] : kv;
      cand[base++] = make_uint2(kv, (uint32_t)pos(bit >> 2, bit & 3));
    }
    // the list padded to a multiple of 4 with entries that never rank above
    // a key (key 0, last position)
    if (tid < 4 && cnt + tid < ((cnt + 3u) & ~3u)) cand[cnt + tid] = make_uint2(0u, 0xffffffffu);
    __syncthreads();
    // wave 0 ranks them and hands T and need to the others
    if (wave == 0) {
      const uint2 me = cand[lane < (int)cnt ? lane : 0];
      uint32_t rank = 0;
      for (uint32_t i = 0; i < cnt; i += 4) {
        uint2 o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = cand[i + u];
#pragma unroll
        for (int u = 0; u < 4; ++u) rank += (o[u].x > me.x || (o[u].x == me.x && o[u].y < me.y)) ? 1u : 0u;
      }
      const uint64_t at = __ballot(lane < (int)cnt && rank == kleft - 1);
      const uint32_t t = __shfl(me.x, __builtin_ctzll(at), 64);
      const uint64_t gt = __ballot(lane < (int)cnt && me.x > t);
      if (lane == 0) {
        sh.bc[0] = t;
        sh.bc[1] = kleft - (uint32_t)__builtin_popcountll(gt);
      }
    }
    __syncthreads();
    T = sh.bc[0];
    need = sh.bc[1];
  }
  uint32_t m_gt = m_above, m_eq = 0;  // kept above T, equal to T
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((m_cand >> (4 * j + e)) & 1u) {
        m_gt |= key[j][e] > T ? 1u << (4 * j + e) : 0u;
        m_eq |= key[j][e] == T ? 1u << (4 * j + e) : 0u;
      }

  // ---- 3. ordered write.  Group j's counts, packed (above T) << 16 |
  // (equal to T), are prefix-summed over the wave's lanes; the groups of a
  // wave follow each other, the waves follow each other.
  uint32_t gbase[G];  // kept keys before this lane's group j (packed)
  uint32_t run = 0;
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint32_t c = (__builtin_popcount((m_gt >> (4 * j)) & 0xfu) << 16) |
                       __builtin_popcount((m_eq >> (4 * j)) & 0xfu);
    const uint32_t incl = wave_inclusive_scan(c);
    gbase[j] = run + incl - c;
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) s_wave[wave] = run;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) before += w < wave ? s_wave[w] : 0u;
  uint32_t m_keep = m_gt | m_eq;
  while (m_keep) {
    const int bit = __builtin_ctz(m_keep);
    m_keep &= m_keep - 1u;
    const int j = bit >> 2;
    uint32_t gb = gbase[0];
#pragma unroll
    for (int t = 1; t < G; ++t) gb = j == t ? gbase[t] : gb;
    const uint32_t lower = ((1u << bit) - 1u) & (0xfu << (4 * j));  // same group, lower e
    gb += before;
    const uint32_t g = (gb >> 16) + __builtin_popcount(m_gt & lower);
    const uint32_t q = (gb & 0xffffu) + __builtin_popcount(m_eq & lower);
    const int32_t p = pos(j, bit & 3);
    if ((m_gt >> bit) & 1u) {
      const uint32_t slot = g + std::min(q, need);
      if (slot < (uint32_t)k) emit(slot, p);
    } else if (q < need && g + q < (uint32_t)k) {
      emit(g + q, p);
    }
  }
}

}  // namespace
}  // namespace sa
