// Exact top-k selection of fp32 score rows.
//
// What is computed ("Inference-time context sparsity", section 2: oracle
// top-k; "Flash Attention vs Sparse Attention", DSA Stage 1: a top-K index
// list): the k positions of a row with the largest scores, equal scores taken
// from the lower position, returned in ascending position order.
//
// Method: radix select on order-preserving uint32 keys (score_key), then an
// ordered compaction.  One 1024-thread workgroup per row.
//   1. One pass over the row (global memory, 16-byte loads, many in flight)
//      builds a histogram of the top 12 key bits (4096 bins: fp32 scores of
//      one magnitude spread over 16 bins, so LDS atomics rarely collide);
//      rows of up to kResident keys are kept in LDS at the same time.  The
//      histogram fixes the top 12 bits of T, the key of the k-th largest
//      element.
//   2. The positions whose top 12 bits equal T's are collected into an LDS
//      candidate list; digit passes over the candidates only (bits 19..12,
//      11..4, 3..0) give T exactly, and `need`, the count of elements equal
//      to T that belong to the result.  If the candidates do not fit the
//      list, those passes run over the whole row instead.
//   3. One pass in position order keeps every key > T and the first `need`
//      keys == T; a workgroup prefix sum over (count above, count equal) gives
//      each kept element its output slot, so the output is ascending.
// Resident rows read global memory once; larger rows read it three times.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kResident = 32768;  // keys kept in LDS (128 KB)
constexpr int kCandRes = 2048;    // candidate positions, resident rows
constexpr int kCandGlob = 8192;   // candidate (key, position) pairs, other rows
constexpr int kBins = 4096;       // first digit: 12 bits

// Workgroup-wide exclusive prefix sum; also returns the total.  Uses s_tot
// (kWaves entries) as scratch; contains two barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_tot,
                                                         uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) s_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = s_tot[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

struct Shared {
  uint32_t hist[kBins];
  uint32_t tot[kWaves];
  uint32_t digit, above, count;
};

__device__ __forceinline__ void zero_hist(Shared& sh, int bins) {
  for (int i = threadIdx.x; i < bins; i += kThreads) sh.hist[i] = 0u;
}

// Pick the digit (of `width` bits at `shift`) of the kleft-th largest key among
// those counted in sh.hist; updates prefix/mask/kleft and returns the count of
// keys with that digit.  Called by every thread; contains barriers.
__device__ __forceinline__ uint32_t select_digit(Shared& sh, int shift, int width, uint32_t& prefix,
                                                 uint32_t& mask, uint32_t& kleft) {
  const int tid = threadIdx.x;
  const int bins = 1 << width;
  const int per = (bins + kThreads - 1) / kThreads;  // bins per thread, descending
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  uint32_t csum = 0;
  for (int j = 0; j < per; ++j) {
    const int d = bins - 1 - (tid * per + j);
    c[j] = d >= 0 ? sh.hist[d] : 0u;
    csum += c[j];
  }
  uint32_t total;
  uint32_t excl = block_exclusive_scan(csum, sh.tot, total);
  for (int j = 0; j < per; ++j) {
    const int d = bins - 1 - (tid * per + j);
    if (d >= 0 && excl < kleft && kleft <= excl + c[j]) {
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

template <bool RES>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int64_t n,
                                                        int64_t row_stride, int32_t k,
                                                        int32_t* __restrict__ idx_out, bool vec4) {
  __shared__ Shared sh;
  // RES: keys[kResident] then candidate positions; else (key, position) pairs
  __shared__ uint32_t buf[RES ? kResident + kCandRes : 2 * kCandGlob];
  uint32_t* keys = buf;                                  // RES only
  uint32_t* cand = RES ? buf + kResident : buf;          // positions
  uint32_t* ckey = RES ? nullptr : buf + kCandGlob;      // keys of candidates (!RES)
  const int cap = RES ? kCandRes : kCandGlob;

  const int tid = threadIdx.x;
  const float* s = scores + (int64_t)blockIdx.x * row_stride;
  int32_t* out = idx_out + (int64_t)blockIdx.x * k;

  auto key_at = [&](int64_t i) -> uint32_t {
    if constexpr (RES) return keys[i];
    else return score_key(s[i]);
  };

  // ---- pass 1: 12-bit histogram (and the LDS copy of resident rows)
  zero_hist(sh, kBins);
  __syncthreads();
  auto count_key = [&](int64_t i, float v) {
    const uint32_t key = score_key(v);
    if constexpr (RES) keys[i] = key;
    atomicAdd(&sh.hist[key >> 20], 1u);
  };
  if (vec4) {
    constexpr int U = 8;  // 8 x 16 bytes per thread in flight
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
          count_key(4 * i + 0, v[u].x);
          count_key(4 * i + 1, v[u].y);
          count_key(4 * i + 2, v[u].z);
          count_key(4 * i + 3, v[u].w);
        }
      }
    }
    for (int64_t i = 4 * n4 + tid; i < n; i += kThreads) count_key(i, s[i]);
  } else {
    constexpr int U = 8;
    for (int64_t base = 0; base < n; base += (int64_t)kThreads * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        v[u] = i < n ? s[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kThreads + tid;
        if (i < n) count_key(i, v[u]);
      }
    }
  }
  __syncthreads();
  uint32_t prefix = 0, mask = 0, kleft = (uint32_t)k;
  const uint32_t c1 = select_digit(sh, 20, 12, prefix, mask, kleft);

  // ---- pass 2: candidates sharing the top 12 bits, then the remaining digits
  constexpr int kShift[3] = {12, 4, 0};
  constexpr int kWidth[3] = {8, 8, 4};
  if (c1 <= (uint32_t)cap) {
    if (tid == 0) sh.count = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) {
        const uint32_t pos = atomicAdd(&sh.count, 1u);
        cand[pos] = (uint32_t)i;
        if constexpr (!RES) ckey[pos] = key;
      }
    }
    __syncthreads();
    for (int d = 0; d < 3; ++d) {
      zero_hist(sh, 1 << kWidth[d]);
      __syncthreads();
      for (uint32_t c = tid; c < c1; c += kThreads) {
        const uint32_t key = RES ? keys[cand[c]] : ckey[c];
        if ((key & mask) == prefix)
          atomicAdd(&sh.hist[(key >> kShift[d]) & ((1u << kWidth[d]) - 1u)], 1u);
      }
      __syncthreads();
      select_digit(sh, kShift[d], kWidth[d], prefix, mask, kleft);
    }
  } else {
    for (int d = 0; d < 3; ++d) {
      zero_hist(sh, 1 << kWidth[d]);
      __syncthreads();
      for (int64_t i = tid; i < n; i += kThreads) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix)
          atomicAdd(&sh.hist[(key >> kShift[d]) & ((1u << kWidth[d]) - 1u)], 1u);
      }
      __syncthreads();
      select_digit(sh, kShift[d], kWidth[d], prefix, mask, kleft);
    }
  }
  const uint32_t T = prefix;
  const uint32_t need = kleft;  // keys == T to keep, lowest positions first

  // ---- pass 3: ordered compaction
  uint32_t gt_run = 0, eq_run = 0;
  constexpr int PER = 4;
  for (int64_t base = 0; base < n; base += (int64_t)kThreads * PER) {
    const int64_t i0 = base + (int64_t)tid * PER;
    uint32_t key[PER];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool valid = i0 + e < n;
      key[e] = valid ? key_at(i0 + e) : 0u;
      cg += (valid && key[e] > T) ? 1u : 0u;
      ce += (valid && key[e] == T) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan((cg << 16) | ce, sh.tot, total);
    uint32_t gt_b = gt_run + (excl >> 16);
    uint32_t eq_b = eq_run + (excl & 0xffffu);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (i0 + e >= n) break;
      if (key[e] > T) {
        out[gt_b + min(eq_b, need)] = (int32_t)(i0 + e);
        ++gt_b;
      } else if (key[e] == T) {
        if (eq_b < need) out[gt_b + eq_b] = (int32_t)(i0 + e);
        ++eq_b;
      }
    }
    gt_run += total >> 16;
    eq_run += total & 0xffffu;
  }
}

}  // namespace

size_t topk_workspace_bytes(int64_t, int64_t, int32_t) { return 0; }

hipError_t launch_topk(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride, int32_t k,
                       int32_t* idx, void*, hipStream_t s) {
  // 16-byte loads when every row starts 16-byte aligned
  const bool vec4 = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (row_stride % 4 == 0);
  if (n <= kResident)
    hipLaunchKernelGGL(topk_kernel<true>, dim3((unsigned)n_rows), dim3(kThreads), 0, s, scores, n,
                       row_stride, k, idx, vec4);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3((unsigned)n_rows), dim3(kThreads), 0, s, scores, n,
                       row_stride, k, idx, vec4);
  return hipGetLastError();
}

}  // namespace sa
