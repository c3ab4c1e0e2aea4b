// Exact top-k selection of fp32 score rows.
//
// What is computed ("Inference-time context sparsity", section 2: oracle
// top-k; "Flash Attention vs Sparse Attention", DSA Stage 1: a top-K index
// list): the k positions of a row with the largest scores, equal scores taken
// from the lower position, returned in ascending position order.
//
// Method: radix select on order-preserving uint32 keys (score_key), then an
// ordered compaction.
//   1. Four 8-bit digit passes from the most significant digit find the exact
//      key T of the k-th largest element and `need`, the number of elements
//      equal to T that belong to the result (k minus the count above T).
//      Each pass histograms the keys that match the digits fixed so far into
//      per-wave LDS histograms (16 x 256 counters), then one scan over the 256
//      digits (largest first) picks the next digit.
//   2. One pass in position order keeps every key > T and the first `need`
//      keys == T; a workgroup-wide prefix sum over (count above, count equal)
//      gives each kept element its output slot, so the output is ascending.
// One 1024-thread workgroup per row; rows are read from global memory (L2)
// on every pass.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace sa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

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

__global__ __launch_bounds__(kThreads) void topk_row_kernel(const float* __restrict__ scores,
                                                            int64_t n, int64_t row_stride, int32_t k,
                                                            int32_t* __restrict__ idx_out) {
  __shared__ uint32_t hist[kWaves][256];
  __shared__ uint32_t s_tot[kWaves];
  __shared__ uint32_t s_digit, s_above;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const float* s = scores + (int64_t)blockIdx.x * row_stride;
  int32_t* out = idx_out + (int64_t)blockIdx.x * k;

  uint32_t prefix = 0, mask = 0;
  uint32_t kleft = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kThreads) {
      const uint32_t key = score_key(s[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // digits in descending order: thread t < 256 holds digit 255 - t
    uint32_t c = 0;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) c += hist[w][255 - tid];
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan(tid < 256 ? c : 0u, s_tot, total);
    if (tid < 256 && excl < kleft && kleft <= excl + c) {
      s_digit = 255u - (uint32_t)tid;
      s_above = excl;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    kleft -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t need = kleft;  // keys == T to keep, lowest positions first

  uint32_t gt_run = 0, eq_run = 0;
  constexpr int PER = 4;
  for (int64_t base = 0; base < n; base += (int64_t)kThreads * PER) {
    const int64_t i0 = base + (int64_t)tid * PER;
    uint32_t key[PER];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      key[e] = (i0 + e < n) ? score_key(s[i0 + e]) : 0u;
      const bool valid = i0 + e < n;
      cg += (valid && key[e] > T) ? 1u : 0u;
      ce += (valid && key[e] == T) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t excl = block_exclusive_scan((cg << 16) | ce, s_tot, total);
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
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)n_rows), dim3(kThreads), 0, s, scores, n,
                     row_stride, k, idx);
  return hipGetLastError();
}

}  // namespace sa
