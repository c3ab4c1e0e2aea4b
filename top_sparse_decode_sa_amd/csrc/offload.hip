// Index-guided offload ("HyLRA", section 2.4): when the KV cache does not fit
// in device memory it stays in host memory, and each layer fetches only the
// blocks its (reused) index set selects.
//
// gather_blocks_kernel copies the selected blocks of K and V from a cache in
// pinned host memory -- read by the GPU directly over the host link, through
// the device address of the pinned allocation -- into compact device
// buffers [B, Hkv, n_blk * bs, d].  Full decode attention over those buffers
// is then attention restricted to the selected blocks (softmax does not
// depend on the order of its tokens).
//
// A fixed grid of at most kGatherGroups workgroups walks the (row, block)
// items: a block's token rows are read in 16-byte pieces, eight pieces of K
// and eight of V per thread in flight before any is stored, since every read
// crosses the host link and waits on its latency.  64 workgroups keep about
// 8 MB of reads in flight -- far more than the link's bandwidth-latency
// product -- while leaving most compute units free for the attention that
// runs beside a prefetch.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace sa {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;
constexpr int kGatherGroups = 64;

struct GatherArgs {
  const uint8_t* k;  // device address of the pinned host cache
  const uint8_t* v;
  int64_t sb, sh, st;  // element strides of the host cache
  int32_t Hkv;
  int32_t elt;         // bytes per element
  int32_t row_bytes;   // D * elt, a multiple of 16
  const int32_t* idx;  // [rows, n_blk] block ids
  int32_t n_blk, bs;
  int64_t nb;          // blocks in the cache; ids are clamped into [0, nb)
  uint8_t* k_out;  // [rows, n_blk * bs, D]
  uint8_t* v_out;
};

__global__ __launch_bounds__(kGatherThreads) void gather_blocks_kernel(GatherArgs a, int64_t items) {
  const int pieces = a.row_bytes / 16;  // per token row
  const int total = a.bs * pieces;      // per block
  const int64_t st_bytes = a.st * a.elt;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int64_t row = item / a.n_blk;
    const int j = (int)(item % a.n_blk);
    const int64_t b = row / a.Hkv;
    const int64_t r = row % a.Hkv;
    // an out-of-range id is clamped: the kernel never reads outside the cache
    const int64_t blk = min(max((int64_t)a.idx[row * a.n_blk + j], (int64_t)0), a.nb - 1);
    const int64_t src0 = (b * a.sb + r * a.sh + blk * a.bs * a.st) * a.elt;
    const int64_t dst0 = ((row * a.n_blk + j) * (int64_t)a.bs) * a.row_bytes;
    for (int base = 0; base < total; base += kGatherThreads * kGatherUnroll) {
      uint4 kw[kGatherUnroll], vw[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int i = min(base + u * kGatherThreads + (int)threadIdx.x, total - 1);
        const int64_t off = src0 + (int64_t)(i / pieces) * st_bytes + (i % pieces) * 16;
        kw[u] = ld16(a.k + off);
        vw[u] = ld16(a.v + off);
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const int i = base + u * kGatherThreads + (int)threadIdx.x;
        if (i < total) {
          const int64_t off = dst0 + (int64_t)i * 16;
          *reinterpret_cast<uint4*>(a.k_out + off) = kw[u];
          *reinterpret_cast<uint4*>(a.v_out + off) = vw[u];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gather_blocks(const Cache& c, const void* k_dev, const void* v_dev,
                                const int32_t* idx, int32_t n_blk, int32_t bs, void* k_out,
                                void* v_out, hipStream_t s) {
  GatherArgs a{};
  a.k = static_cast<const uint8_t*>(k_dev);
  a.v = static_cast<const uint8_t*>(v_dev);
  a.sb = c.sb;
  a.sh = c.sh;
  a.st = c.st;
  a.Hkv = c.Hkv;
  a.elt = c.kv_dtype == SA_BF16 ? 2 : 4;
  a.row_bytes = c.D * a.elt;
  a.idx = idx;
  a.n_blk = n_blk;
  a.bs = bs;
  a.nb = c.N / bs;
  a.k_out = static_cast<uint8_t*>(k_out);
  a.v_out = static_cast<uint8_t*>(v_out);
  const int64_t items = (int64_t)c.B * c.Hkv * n_blk;
  const unsigned groups = (unsigned)std::min<int64_t>(items, kGatherGroups);
  hipLaunchKernelGGL(gather_blocks_kernel, dim3(groups), dim3(kGatherThreads), 0, s, a, items);
  return hipGetLastError();
}

}  // namespace sa
