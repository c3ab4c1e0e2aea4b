// Validation of selected index lists (not a step of the method): the
// selected-set attention reads the K/V rows the indices name, and it requires
// ("Inference-time context sparsity", section 3.C: attention over the selected
// tokens) each row's indices to name distinct tokens or blocks of the cache.
// This check counts the rows that break either rule, so a caller can test an
// index list (from its own selector, or kept for a later layer to reuse)
// before handing it over.  Indices are read as data only.
//
// One workgroup per row: every index is tested against the range, then the
// row is sorted in LDS (bitonic, padded to a power of two with INT32_MAX) and
// neighbours are compared.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace sa {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    const int32_t* __restrict__ idx, int32_t n, int32_t n_pow2, int64_t limit,
    int32_t* __restrict__ counts) {
  extern __shared__ int32_t s_v[];
  const int64_t row = blockIdx.x;
  const int32_t* __restrict__ x = idx + row * n;
  __shared__ int s_bad, s_dup;
  if (threadIdx.x == 0) {
    s_bad = 0;
    s_dup = 0;
  }
  __syncthreads();
  bool bad = false;
  for (int i = threadIdx.x; i < n_pow2; i += kCheckThreads) {
    int32_t v = INT32_MAX;
    if (i < n) {
      v = x[i];
      bad |= v < 0 || (int64_t)v >= limit;
    }
    s_v[i] = v;
  }
  if (bad) s_bad = 1;
  __syncthreads();
  // bitonic sort, ascending
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n_pow2 / 2; i += kCheckThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t a = s_v[lo], b = s_v[hi];
        if ((a > b) == up) {
          s_v[lo] = b;
          s_v[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  bool dup = false;
  for (int i = threadIdx.x; i + 1 < n; i += kCheckThreads) dup |= s_v[i] == s_v[i + 1];
  if (dup) s_dup = 1;
  __syncthreads();
  if (threadIdx.x == 0) {
    if (s_bad) atomicAdd(&counts[0], 1);
    if (s_dup) atomicAdd(&counts[1], 1);
  }
}

}  // namespace

size_t check_indices_lds_bytes(int32_t n) {
  int32_t p = 1;
  while (p < n) p <<= 1;
  return (size_t)std::max(p, 2) * sizeof(int32_t);
}

hipError_t launch_check_indices(const int32_t* idx, int64_t rows, int32_t n, int64_t limit,
                                int32_t* counts, hipStream_t s) {
  hipError_t e = launch_zero(counts, 2 * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  int32_t p = 1;
  while (p < n) p <<= 1;
  p = std::max(p, 2);
  hipLaunchKernelGGL(check_indices_kernel, dim3((unsigned)rows), dim3(kCheckThreads),
                     (size_t)p * sizeof(int32_t), s, idx, n, p, limit, counts);
  return hipGetLastError();
}

}  // namespace sa
