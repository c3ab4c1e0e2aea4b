// Split-K online-softmax decode attention over a selected token set (or over
// the whole cache), with the log-sum-exp combine of the splits fused into the
// same launch.
//
// What is computed ("Flash Attention vs Sparse Attention", DSA Stage 2 and
// the tiling + online-softmax section; "Inference-time context sparsity",
// section 3.C): for every query head of a (sequence, KV head) row, softmax
// attention restricted to the row's selected tokens, reading only those K/V
// rows from HBM.
//
// Work split (gfx950, wave64):
//   grid = (nsplit, rows).  A 256-thread workgroup takes `chunk` consecutive
//   slots of its row's selection.  A "lane group" of LPR lanes holds one cache
//   row as LPR 16-byte pieces (bf16, d=128: 16 lanes x 8 values), so one wave
//   load instruction fetches 64/LPR whole rows with 128-bit loads.
//   Every lane group runs its own online softmax (running max m, sum l,
//   unnormalised output o, all fp32, exp in base 2 with log2(e) folded into
//   q), groups merge through LDS, and the workgroup writes one partial
//   (m, l, o) per query head.  The last workgroup of a row to finish (device
//   atomic counter) merges the nsplit partials and writes the output, then
//   resets the counter to zero for the next call.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;        // slots per lane group in flight per iteration
constexpr int kTargetGroups = 4096;

struct AttendArgs {
  const void* q;
  sa_dtype q_dtype;
  const uint8_t* k;
  const uint8_t* v;
  int64_t sb, sh, st;  // element strides
  int32_t Hq, Hkv;
  int64_t N;
  float qscale;  // softmax scale * log2(e)
  const int32_t* idx;
  int32_t n_idx;
  int32_t bs;
  int64_t n_slots;
  int32_t chunk;
  int32_t nsplit;
  float* out;
  float* part;
  uint32_t* counters;
};

template <int MODE>
__device__ __forceinline__ int64_t resolve_slot(const AttendArgs& a, int row, int b, int64_t j,
                                                bool& ok) {
  if constexpr (MODE == kIdxDense) {
    return j;
  } else if constexpr (MODE == kIdxTokenPerHead) {
    return a.idx[(int64_t)row * a.n_idx + j];
  } else if constexpr (MODE == kIdxTokenShared) {
    return a.idx[(int64_t)b * a.n_idx + j];
  } else {
    const int64_t blk = a.idx[(int64_t)row * a.n_idx + j / a.bs];
    const int64_t t = blk * a.bs + j % a.bs;
    ok = ok && (t < a.N);
    return t;
  }
}

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
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int grp = tid / LPR;
  const int sl = tid % LPR;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int b = row / a.Hkv;
  const int r = row % a.Hkv;

  float qv[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e)
      qv[g][e] = load_q(a.q, a.q_dtype, ((int64_t)b * a.Hq + r * G + g) * D + sl * E + e) * a.qscale;

  const int64_t kv_off = ((int64_t)b * a.sb + (int64_t)r * a.sh) * EB + sl * 16;
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

  // ---- merge the lane groups of this workgroup
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

  const int64_t out_base = ((int64_t)b * a.Hq + (int64_t)r * G) * D;
  constexpr int PS = G * (D + 2);  // floats per partial: o[G][D], m[G], l[G]
  float* my_part = a.part + ((int64_t)row * a.nsplit + split) * PS;
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
    if (a.nsplit == 1) {
      a.out[out_base + x] = O / L;
    } else {
      my_part[x] = O;
      if (dim == 0) {
        my_part[G * D + g] = M;
        my_part[G * D + G + g] = L;
      }
    }
  }
  if (a.nsplit == 1) return;

  // ---- fused split combine: the last workgroup of the row merges
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&a.counters[row], 1u);
    s_last = (prev == (uint32_t)(a.nsplit - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pr = a.part + (int64_t)row * a.nsplit * PS;
  for (int x = tid; x < G * D; x += kThreads) {
    const int g = x / D;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pr[(int64_t)s * PS + G * D + g]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float* ps = pr + (int64_t)s * PS;
      const float w = exp2f(ps[G * D + g] - M);
      L = fmaf(ps[G * D + G + g], w, L);
      O = fmaf(ps[x], w, O);
    }
    a.out[out_base + x] = O / L;
  }
  if (tid == 0) a.counters[row] = 0u;
}

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

int lanes_per_row(const Cache& c) { return c.D * (c.kv_dtype == SA_BF16 ? 2 : 4) / 16; }

}  // namespace

AttendPlan plan_attend(const Cache& c, int mode, int32_t n_idx, int32_t bs) {
  AttendPlan p{};
  p.mode = mode;
  if (mode == kIdxDense) {
    p.n_slots = c.N;
  } else if (mode == kIdxBlockPerHead) {
    p.n_slots = (int64_t)n_idx * bs;
  } else {
    p.n_slots = n_idx;
  }
  const int64_t rows = (int64_t)c.B * c.Hkv;
  const int64_t unit = (int64_t)(kThreads / lanes_per_row(c)) * kUnroll;
  int64_t chunk = (rows * p.n_slots + kTargetGroups - 1) / kTargetGroups;
  chunk = (chunk + unit - 1) / unit * unit;
  chunk = std::max<int64_t>(unit, std::min<int64_t>(chunk, 256 * unit));
  // keep the number of splits per row bounded so the combine stays cheap
  while ((p.n_slots + chunk - 1) / chunk > 4096) chunk *= 2;
  p.chunk = (int32_t)chunk;
  p.nsplit = (int32_t)((p.n_slots + chunk - 1) / chunk);
  const size_t counters = align_up((size_t)rows * sizeof(uint32_t), 256);
  const size_t part =
      p.nsplit > 1 ? (size_t)rows * p.nsplit * c.G * (c.D + 2) * sizeof(float) : 0;
  p.ws_bytes = counters + align_up(part, 256);
  return p;
}

hipError_t launch_attend(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                         const void* v, const int32_t* idx, int32_t n_idx, int32_t bs, float* out,
                         void* ws, hipStream_t s) {
  AttendArgs a{};
  a.q = q;
  a.q_dtype = c.q_dtype;
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.sb = c.sb;
  a.sh = c.sh;
  a.st = c.st;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.N = c.N;
  a.qscale = c.scale * kLog2e;
  a.idx = idx;
  a.n_idx = n_idx;
  a.bs = bs;
  a.n_slots = p.n_slots;
  a.chunk = p.chunk;
  a.nsplit = p.nsplit;
  a.out = out;
  const int64_t rows = (int64_t)c.B * c.Hkv;
  a.counters = static_cast<uint32_t*>(ws);
  a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                    align_up((size_t)rows * sizeof(uint32_t), 256));
  const dim3 grid(p.nsplit, (unsigned)rows);
  if (c.kv_dtype == SA_BF16) {
    if (c.D == 64) return dispatch_group<bf16_t, 64>(c.G, p.mode, grid, a, s);
    return dispatch_group<bf16_t, 128>(c.G, p.mode, grid, a, s);
  }
  if (c.D == 64) return dispatch_group<float, 64>(c.G, p.mode, grid, a, s);
  return dispatch_group<float, 128>(c.G, p.mode, grid, a, s);
}

}  // namespace sa
