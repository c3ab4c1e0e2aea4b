// C ABI of libsa: argument validation, workspace planning and dispatch.
// Every entry point checks its arguments on the host and returns an error
// code before anything is enqueued; kernels are launched only on success.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.hpp"
#include "internal.hpp"
#include "sa.h"

namespace sa {
namespace {

thread_local std::string g_last_error;

sa_status fail(sa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sa_status ok() {
  g_last_error.clear();
  return SA_OK;
}

sa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elt_bytes(sa_dtype d) { return d == SA_BF16 ? 2 : 4; }

bool valid_dtype(sa_dtype d) { return d == SA_F32 || d == SA_BF16; }

// Validate a descriptor and produce the internal cache view.
sa_status check_desc(const sa_kv_desc* d, Cache* c) {
  if (!d) return fail(SA_ERR_NULL, "descriptor is null");
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype))
    return fail(SA_ERR_DTYPE, "unknown dtype (q %d, kv %d)", (int)d->q_dtype, (int)d->kv_dtype);
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(SA_ERR_SHAPE, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(SA_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", d->n_q_heads,
                d->n_kv_heads);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (d->ctx_len < 1 || d->ctx_len > INT32_MAX)
    return fail(SA_ERR_SHAPE, "ctx_len %lld outside [1, 2^31)", (long long)d->ctx_len);
  if ((int64_t)d->batch * d->n_kv_heads > 65535)
    return fail(SA_ERR_SHAPE, "batch * n_kv_heads above 65535");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", d->head_dim);
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SA_ERR_UNSUPPORTED, "group size %d (built: 1, 2, 4, 8)", G);
  const int eb = elt_bytes(d->kv_dtype);
  if (d->kv_stride_t < d->head_dim || d->kv_stride_h < 0 || d->kv_stride_b < 0)
    return fail(SA_ERR_SHAPE, "strides must satisfy kv_stride_t >= head_dim, others >= 0");
  if ((d->kv_stride_t * eb) % 16 || (d->kv_stride_h * eb) % 16 || (d->kv_stride_b * eb) % 16)
    return fail(SA_ERR_ALIGN, "cache strides must be multiples of 16 bytes");
  if (!(d->softmax_scale >= 0.0f) || isinf(d->softmax_scale))
    return fail(SA_ERR_SHAPE, "softmax_scale must be finite and >= 0");
  c->B = d->batch;
  c->Hq = d->n_q_heads;
  c->Hkv = d->n_kv_heads;
  c->G = G;
  c->D = d->head_dim;
  c->N = d->ctx_len;
  c->q_dtype = d->q_dtype;
  c->kv_dtype = d->kv_dtype;
  c->sb = d->kv_stride_b;
  c->sh = d->kv_stride_h;
  c->st = d->kv_stride_t;
  c->scale = d->softmax_scale > 0.0f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return SA_OK;
}

sa_status check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(SA_ERR_NULL, "%s is null", name);
  if (!aligned(p, align)) return fail(SA_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return SA_OK;
}

sa_status check_ws(void* ws, size_t have, size_t need, const char* what) {
  if (need == 0) return SA_OK;
  if (!ws) return fail(SA_ERR_WORKSPACE, "%s needs a %zu-byte workspace, got null", what, need);
  if (!aligned(ws, 256)) return fail(SA_ERR_ALIGN, "workspace is not 256-byte aligned");
  if (have < need)
    return fail(SA_ERR_WORKSPACE, "%s needs %zu workspace bytes, got %zu", what, need, have);
  return SA_OK;
}

int mode_of(sa_index_kind ik) {
  switch (ik) {
    case SA_IDX_TOKEN_PER_KV_HEAD: return kIdxTokenPerHead;
    case SA_IDX_TOKEN_SHARED: return kIdxTokenShared;
    case SA_IDX_BLOCK_PER_KV_HEAD: return kIdxBlockPerHead;
    case SA_IDX_TOKEN_PER_Q_HEAD: return kIdxTokenPerHead;  // on the per-query-head view
  }
  return -1;
}

// The cache as the attention kernels see it for an index kind: per-query-head
// sets run on the view with one row per query head.
Cache attend_view(const Cache& c, sa_index_kind ik) {
  return ik == SA_IDX_TOKEN_PER_Q_HEAD ? per_q_head_view(c) : c;
}

// grid rows of the per-query-head view
sa_status check_q_rows(const Cache& c) {
  if ((int64_t)c.B * c.Hq > 65535)
    return fail(SA_ERR_SHAPE, "per-query-head rows: batch * n_q_heads above 65535");
  return SA_OK;
}

sa_status check_indexer_aux(const Cache& c, const sa_score_aux* aux) {
  if (!aux) return fail(SA_ERR_NULL, "indexer scoring needs aux");
  if (aux->n_idx_heads < 1 || aux->n_idx_heads > 16)
    return fail(SA_ERR_SHAPE, "n_idx_heads %d outside [1, 16]", aux->n_idx_heads);
  if (aux->idx_dim != 32 && aux->idx_dim != 64 && aux->idx_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "idx_dim %d (built: 32, 64, 128)", aux->idx_dim);
  sa_status st;
  if ((st = check_ptr(aux->q_idx, "aux.q_idx", 16)) != SA_OK) return st;
  if ((st = check_ptr(aux->k_idx, "aux.k_idx", 16)) != SA_OK) return st;
  if ((st = check_ptr(aux->idx_w, "aux.idx_w", 4)) != SA_OK) return st;
  (void)c;
  return SA_OK;
}

sa_status check_block_aux(const Cache& c, const sa_score_aux* aux) {
  if (!aux) return fail(SA_ERR_NULL, "block scoring needs aux");
  if (aux->block_size < 1 || aux->block_size > 4096)
    return fail(SA_ERR_SHAPE, "block_size %d outside [1, 4096]", aux->block_size);
  sa_status st;
  if ((st = check_ptr(aux->kmin, "aux.kmin", 16)) != SA_OK) return st;
  if ((st = check_ptr(aux->kmax, "aux.kmax", 16)) != SA_OK) return st;
  (void)c;
  return SA_OK;
}

int64_t score_row_len(const Cache& c, sa_score_kind kind, const sa_score_aux* aux) {
  if (kind == SA_SCORE_BLOCK_MINMAX) return (c.N + aux->block_size - 1) / aux->block_size;
  return c.N;
}

int64_t score_rows(const Cache& c, sa_score_kind kind) {
  if (kind == SA_SCORE_INDEXER) return c.B;
  if (kind == SA_SCORE_EXACT_PER_Q_HEAD) return (int64_t)c.B * c.Hq;
  return (int64_t)c.B * c.Hkv;
}

bool known_score_kind(sa_score_kind kind) {
  return kind == SA_SCORE_EXACT || kind == SA_SCORE_BLOCK_MINMAX || kind == SA_SCORE_INDEXER ||
         kind == SA_SCORE_INDEXER_PER_KV_HEAD || kind == SA_SCORE_EXACT_PER_Q_HEAD;
}

bool is_indexer(sa_score_kind kind) {
  return kind == SA_SCORE_INDEXER || kind == SA_SCORE_INDEXER_PER_KV_HEAD;
}

// The index kind a score kind selects into.
sa_index_kind index_kind_of(sa_score_kind kind) {
  switch (kind) {
    case SA_SCORE_BLOCK_MINMAX: return SA_IDX_BLOCK_PER_KV_HEAD;
    case SA_SCORE_INDEXER: return SA_IDX_TOKEN_SHARED;
    case SA_SCORE_EXACT_PER_Q_HEAD: return SA_IDX_TOKEN_PER_Q_HEAD;
    default: return SA_IDX_TOKEN_PER_KV_HEAD;
  }
}

// Score kinds that sa_select takes: the exact ones and the indexers.
bool selectable(sa_score_kind kind) {
  return kind == SA_SCORE_EXACT || kind == SA_SCORE_EXACT_PER_Q_HEAD || is_indexer(kind);
}

// Rows of a selection: one per KV head, per query head, or per sequence
// (shared indexer).
Cache select_view(const Cache& c, sa_score_kind kind) {
  if (kind == SA_SCORE_EXACT_PER_Q_HEAD) return per_q_head_view(c);
  Cache v = c;
  if (kind == SA_SCORE_INDEXER) v.Hkv = 1;
  return v;
}

// The indexer inputs of a selection (null for the exact kinds).
const SelectIndexer* select_indexer(sa_score_kind kind, const sa_score_aux* aux,
                                    SelectIndexer* buf) {
  if (!is_indexer(kind)) return nullptr;
  buf->q_idx = aux->q_idx;
  buf->k_idx = aux->k_idx;
  buf->w = aux->idx_w;
  buf->H = aux->n_idx_heads;
  buf->Di = aux->idx_dim;
  return buf;
}

sa_status do_score(const Cache& c, sa_score_kind kind, const void* q, const void* k,
                   const sa_score_aux* aux, float* scores, hipStream_t s) {
  hipError_t e;
  switch (kind) {
    case SA_SCORE_EXACT: e = launch_score_exact(c, q, k, scores, s); break;
    case SA_SCORE_EXACT_PER_Q_HEAD: e = launch_score_exact(per_q_head_view(c), q, k, scores, s); break;
    case SA_SCORE_BLOCK_MINMAX:
      e = launch_score_block(c, aux->block_size, q, aux->kmin, aux->kmax, scores, s);
      break;
    default:
      // the per-KV-head indexer is the shared one over B * Hkv sequences:
      // its tensors are the shared layout with (batch, KV head) flattened
      e = launch_score_indexer(
          kind == SA_SCORE_INDEXER_PER_KV_HEAD ? c.B * c.Hkv : c.B, c.N, aux->n_idx_heads,
          aux->idx_dim, aux->q_idx, aux->k_idx, aux->idx_w, scores, s);
      break;
  }
  return hip_status(e, "sa_score launch");
}

sa_status check_score_args(const sa_kv_desc* desc, sa_score_kind kind, const void* q,
                           const void* k_cache, const sa_score_aux* aux, const float* scores,
                           Cache* c) {
  sa_status st;
  if ((st = check_desc(desc, c)) != SA_OK) return st;
  if (!known_score_kind(kind)) return fail(SA_ERR_SHAPE, "unknown score kind %d", (int)kind);
  if ((st = check_ptr(scores, "scores", 4)) != SA_OK) return st;
  if (is_indexer(kind)) return check_indexer_aux(*c, aux);
  if ((st = check_ptr(q, "q", 16)) != SA_OK) return st;
  if (kind == SA_SCORE_BLOCK_MINMAX) return check_block_aux(*c, aux);
  if (kind == SA_SCORE_EXACT_PER_Q_HEAD && (st = check_q_rows(*c)) != SA_OK) return st;
  return check_ptr(k_cache, "k_cache", 16);
}

sa_status check_attend_args(const Cache& c, const void* q, const void* k, const void* v,
                            const float* out) {
  sa_status st;
  if ((st = check_ptr(q, "q", 16)) != SA_OK) return st;
  if ((st = check_ptr(k, "k_cache", 16)) != SA_OK) return st;
  if ((st = check_ptr(v, "v_cache", 16)) != SA_OK) return st;
  if ((st = check_ptr(out, "out", 4)) != SA_OK) return st;
  (void)c;
  return SA_OK;
}

sa_status check_sparse_idx(const Cache& c, sa_index_kind ik, const int32_t* idx, int32_t n_idx,
                           int32_t bs) {
  if (mode_of(ik) < 0) return fail(SA_ERR_SHAPE, "unknown index kind %d", (int)ik);
  sa_status st;
  if (ik == SA_IDX_TOKEN_PER_Q_HEAD && (st = check_q_rows(c)) != SA_OK) return st;
  if ((st = check_ptr(idx, "idx", 4)) != SA_OK) return st;
  if (n_idx < 1) return fail(SA_ERR_SHAPE, "n_idx %d must be >= 1", n_idx);
  if (ik == SA_IDX_BLOCK_PER_KV_HEAD) {
    if (bs < 1 || bs > 4096) return fail(SA_ERR_SHAPE, "block_size %d outside [1, 4096]", bs);
    if ((int64_t)n_idx * bs > (int64_t)INT32_MAX)
      return fail(SA_ERR_SHAPE, "n_idx * block_size overflows");
  }
  return SA_OK;
}

// Workspace layout of one SPARSE layer step: [scores | top-k | attention].
struct LayerWs {
  size_t scores, topk, attend, total;
};

LayerWs layer_ws(const Cache& c, const sa_layer_args* a, sa_layer_mode mode) {
  LayerWs w{};
  if (mode == SA_LAYER_DENSE) {
    w.attend = plan_attend(c, kIdxDense, 0, 0).ws_bytes;
  } else if (mode == SA_LAYER_DENSE_SELECT) {
    const int64_t rows = (int64_t)c.B * c.Hkv;
    w.scores = align_up((size_t)rows * c.N * sizeof(float), 256);
    w.topk = align_up(topk_workspace_bytes(rows, c.N, a->k), 256);
    w.attend = plan_attend(c, fused_scores_supported(c) ? kIdxDenseScored : kIdxDense, 0, 0).ws_bytes;
  } else {
    const sa_index_kind ik = index_kind_of(a->score_kind);
    const int32_t bs = a->score_kind == SA_SCORE_BLOCK_MINMAX ? a->aux.block_size : 0;
    w.attend = plan_attend(attend_view(c, ik), mode_of(ik), a->k, bs).ws_bytes;
    if (mode == SA_LAYER_SPARSE && selectable(a->score_kind)) {
      // the fused selection's candidates (or its scores and top-k fallback)
      w.scores = align_up(plan_select(select_view(c, a->score_kind), a->k).ws_bytes, 256);
    } else if (mode == SA_LAYER_SPARSE) {
      const int64_t rows = score_rows(c, a->score_kind);
      const int64_t len = score_row_len(c, a->score_kind, &a->aux);
      w.scores = align_up((size_t)rows * len * sizeof(float), 256);
      w.topk = align_up(topk_workspace_bytes(rows, len, a->k), 256);
    }
  }
  w.total = w.scores + w.topk + align_up(w.attend, 256);
  return w;
}

// Dense decode plus the exact score of every token: one fused launch where
// the gather kernel takes the shape, else the scoring kernel and then the
// dense decode.
sa_status run_dense_scored(const Cache& c, const void* q, const void* k, const void* v, float* out,
                           float* scores, void* ws, hipStream_t s) {
  if (fused_scores_supported(c)) {
    const AttendPlan p = plan_attend(c, kIdxDenseScored, 0, 0);
    return hip_status(launch_attend(c, p, q, k, v, nullptr, 0, 0, out, ws, s, scores),
                      "dense decode (scored) launch");
  }
  sa_status st = hip_status(launch_score_exact(c, q, k, scores, s), "exact scoring launch");
  if (st != SA_OK) return st;
  const AttendPlan p = plan_attend(c, kIdxDense, 0, 0);
  return hip_status(launch_attend(c, p, q, k, v, nullptr, 0, 0, out, ws, s), "dense decode launch");
}

size_t dense_scored_ws(const Cache& c) {
  return plan_attend(c, fused_scores_supported(c) ? kIdxDenseScored : kIdxDense, 0, 0).ws_bytes;
}

__global__ void zero_kernel(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes % 16;
  const unsigned blocks = (unsigned)std::max<size_t>(1, std::min<size_t>((n16 + 255) / 256, 4096));
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint4*>(p), n16,
                     static_cast<uint8_t*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace sa

using namespace sa;

// ---------------------------------------------------------------------------
// The allocation-free entry point's scratch: a file-scope device array that
// every GPU the library runs on holds until the process ends.  Host code uses
// it only through the address hipGetSymbolAddress returns on each device
// (the array's name in host code is a host-side stand-in, not a device
// address).
static __device__ __align__(256) uint8_t scratch[sa::kNoAllocScratchBytes];

namespace sa {
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

// The scratch's device address on the device `stream` belongs to, looked up
// once per device with that device current.
sa_status noalloc_scratch(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return fail(SA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(SA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(SA_ERR_HIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  e != hipSuccess ? hipGetErrorString(e) : "null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}
}  // namespace sa

extern "C" {

const char* sa_version(void) { return "sa 0.1.0 (gfx950)"; }

const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is null";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: a size, count, stride or k is out of range";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: misaligned pointer or stride";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE: unsupported dtype";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE: workspace missing or too small";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: configuration not built";
    case SA_ERR_HIP: return "SA_ERR_HIP: HIP runtime error";
    case SA_ERR_MEMORY: return "SA_ERR_MEMORY: a buffer is not the kind of memory the call needs";
  }
  return "unknown sa_status";
}

const char* sa_last_error(void) { return g_last_error.c_str(); }

sa_status sa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes == 0) return ok();
  if (!ws) return fail(SA_ERR_NULL, "workspace is null");
  return hip_status(launch_zero(ws, ws_bytes, stream), "sa_workspace_init launch");
}

sa_status sa_score(const sa_kv_desc* desc, sa_score_kind kind, const void* q, const void* k_cache,
                   const sa_score_aux* aux, float* scores, hipStream_t stream) {
  Cache c;
  sa_status st = check_score_args(desc, kind, q, k_cache, aux, scores, &c);
  if (st != SA_OK) return st;
  return do_score(c, kind, q, k_cache, aux, scores, stream);
}

sa_status sa_block_summarize(const sa_kv_desc* desc, int32_t block_size, const void* k_cache,
                             void* kmin, void* kmax, hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if (block_size < 1 || block_size > 4096)
    return fail(SA_ERR_SHAPE, "block_size %d outside [1, 4096]", block_size);
  if ((st = check_ptr(k_cache, "k_cache", 16)) != SA_OK) return st;
  if ((st = check_ptr(kmin, "kmin", 16)) != SA_OK) return st;
  if ((st = check_ptr(kmax, "kmax", 16)) != SA_OK) return st;
  return hip_status(launch_block_summarize(c, block_size, k_cache, kmin, kmax, stream),
                    "sa_block_summarize launch");
}

size_t sa_topk_workspace_size(int64_t n_rows, int64_t n, int32_t k) {
  if (n_rows < 1 || n < 1 || k < 1 || k > n) return 0;
  return align_up(topk_workspace_bytes(n_rows, n, k), 256);
}

sa_status sa_topk(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride, int32_t k,
                  int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  sa_status st;
  if ((st = check_ptr(scores, "scores", 4)) != SA_OK) return st;
  if ((st = check_ptr(idx_out, "idx_out", 4)) != SA_OK) return st;
  if (n_rows < 1 || n_rows >= (1 << 22))
    return fail(SA_ERR_SHAPE, "n_rows %lld outside [1, 2^22)", (long long)n_rows);
  if (n < 1 || n > INT32_MAX) return fail(SA_ERR_SHAPE, "n %lld outside [1, 2^31)", (long long)n);
  if (k < 1 || k > n) return fail(SA_ERR_SHAPE, "k %d outside [1, n=%lld]", k, (long long)n);
  if (row_stride < n) return fail(SA_ERR_SHAPE, "row_stride < n");
  if ((st = check_ws(ws, ws_bytes, sa_topk_workspace_size(n_rows, n, k), "sa_topk")) != SA_OK)
    return st;
  return hip_status(launch_topk(scores, n_rows, n, row_stride, k, idx_out, ws, stream),
                    "sa_topk launch");
}

size_t sa_select_workspace_size(const sa_kv_desc* desc, sa_score_kind kind, int32_t k) {
  Cache c;
  if (check_desc(desc, &c) != SA_OK || !selectable(kind) || k < 1 || k > c.N) return 0;
  return align_up(plan_select(select_view(c, kind), k).ws_bytes, 256);
}

sa_status sa_select(const sa_kv_desc* desc, sa_score_kind kind, const void* q, const void* k_cache,
                    const sa_score_aux* aux, int32_t k, int32_t* idx_out, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if (!selectable(kind))
    return fail(SA_ERR_SHAPE, "sa_select takes the exact and indexer score kinds (kind %d)",
                (int)kind);
  if (is_indexer(kind)) {
    if ((st = check_indexer_aux(c, aux)) != SA_OK) return st;
  } else {
    if ((st = check_ptr(q, "q", 16)) != SA_OK) return st;
    if ((st = check_ptr(k_cache, "k_cache", 16)) != SA_OK) return st;
  }
  if ((st = check_ptr(idx_out, "idx_out", 4)) != SA_OK) return st;
  if (kind == SA_SCORE_EXACT_PER_Q_HEAD && (st = check_q_rows(c)) != SA_OK) return st;
  if (k < 1 || k > c.N) return fail(SA_ERR_SHAPE, "k %d outside [1, %lld]", k, (long long)c.N);
  const Cache v = select_view(c, kind);
  const SelectPlan p = plan_select(v, k);
  if ((st = check_ws(ws, ws_bytes, align_up(p.ws_bytes, 256), "sa_select")) != SA_OK) return st;
  SelectIndexer ixb;
  return hip_status(
      launch_select(v, p, q, k_cache, select_indexer(kind, aux, &ixb), k, idx_out, ws, stream),
      "sa_select launch");
}

size_t sa_sparse_workspace_size(const sa_kv_desc* desc, sa_index_kind ik, int32_t n_idx,
                                int32_t block_size) {
  Cache c;
  if (check_desc(desc, &c) != SA_OK || mode_of(ik) < 0 || n_idx < 1) return 0;
  if (ik == SA_IDX_BLOCK_PER_KV_HEAD && (block_size < 1 || block_size > 4096)) return 0;
  return align_up(plan_attend(attend_view(c, ik), mode_of(ik), n_idx, block_size).ws_bytes, 256);
}

sa_status sa_sparse_decode(const sa_kv_desc* desc, const void* q, const void* k_cache,
                           const void* v_cache, sa_index_kind ik, const int32_t* idx, int32_t n_idx,
                           int32_t block_size, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_attend_args(c, q, k_cache, v_cache, out)) != SA_OK) return st;
  if ((st = check_sparse_idx(c, ik, idx, n_idx, block_size)) != SA_OK) return st;
  const Cache v = attend_view(c, ik);
  const AttendPlan p = plan_attend(v, mode_of(ik), n_idx, block_size);
  if ((st = check_ws(ws, ws_bytes, p.ws_bytes, "sa_sparse_decode")) != SA_OK) return st;
  return hip_status(
      launch_attend(v, p, q, k_cache, v_cache, idx, n_idx, block_size, out, ws, stream),
      "sa_sparse_decode launch");
}

sa_status sa_sparse_decode_noalloc(const sa_kv_desc* desc, const void* q, const void* k_cache,
                                   const void* v_cache, sa_index_kind ik, const int32_t* idx,
                                   int32_t n_idx, int32_t block_size, float* out,
                                   hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_attend_args(c, q, k_cache, v_cache, out)) != SA_OK) return st;
  if ((st = check_sparse_idx(c, ik, idx, n_idx, block_size)) != SA_OK) return st;
  const Cache v = attend_view(c, ik);
  const AttendPlan p = plan_attend(v, mode_of(ik), n_idx, block_size);
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    if (p.ws_bytes > sa::kNoAllocScratchBytes)
      return fail(SA_ERR_WORKSPACE,
                  "sa_sparse_decode_noalloc: this call needs %zu bytes of scratch, the static "
                  "scratch holds %zu",
                  p.ws_bytes, sa::kNoAllocScratchBytes);
    if ((st = sa::noalloc_scratch(stream, &ws)) != SA_OK) return st;
  }
  return hip_status(
      launch_attend(v, p, q, k_cache, v_cache, idx, n_idx, block_size, out, ws, stream),
      "sa_sparse_decode_noalloc launch");
}

sa_status sa_gather_read(const sa_kv_desc* desc, const void* k_cache, const void* v_cache,
                         sa_index_kind ik, const int32_t* idx, int32_t n_idx, int32_t block_size,
                         uint32_t* sink, hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_ptr(k_cache, "k_cache", 16)) != SA_OK) return st;
  if ((st = check_ptr(v_cache, "v_cache", 16)) != SA_OK) return st;
  if ((st = check_ptr(sink, "sink", 4)) != SA_OK) return st;
  if ((st = check_sparse_idx(c, ik, idx, n_idx, block_size)) != SA_OK) return st;
  const Cache v = attend_view(c, ik);
  const AttendPlan p = plan_attend(v, mode_of(ik), n_idx, block_size);
  if (p.kernel != kKernPairs)
    return fail(SA_ERR_UNSUPPORTED,
                "sa_gather_read covers the pair-pipelined gather-attend only (bf16, head_dim 128, "
                "at most 4 query heads per KV head, token indices or whole blocks)");
  return hip_status(launch_gather_read(v, p, k_cache, v_cache, idx, n_idx, block_size, sink, stream),
                    "sa_gather_read launch");
}

sa_status sa_check_indices(const sa_kv_desc* desc, sa_index_kind ik, const int32_t* idx,
                           int32_t n_idx, int32_t block_size, int32_t* counts,
                           hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_sparse_idx(c, ik, idx, n_idx, block_size)) != SA_OK) return st;
  if ((st = check_ptr(counts, "counts", 4)) != SA_OK) return st;
  if (n_idx > kCheckMaxIdx)
    return fail(SA_ERR_UNSUPPORTED, "n_idx %d above %d", n_idx, kCheckMaxIdx);
  int64_t rows = (int64_t)c.B * c.Hkv;
  if (ik == SA_IDX_TOKEN_SHARED) rows = c.B;
  if (ik == SA_IDX_TOKEN_PER_Q_HEAD) rows = (int64_t)c.B * c.Hq;
  const int64_t limit =
      ik == SA_IDX_BLOCK_PER_KV_HEAD ? (c.N + block_size - 1) / block_size : c.N;
  return hip_status(launch_check_indices(idx, rows, n_idx, limit, counts, stream),
                    "sa_check_indices launch");
}

size_t sa_dense_workspace_size(const sa_kv_desc* desc) {
  Cache c;
  if (check_desc(desc, &c) != SA_OK) return 0;
  return align_up(plan_attend(c, kIdxDense, 0, 0).ws_bytes, 256);
}

sa_status sa_dense_decode(const sa_kv_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, float* out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_attend_args(c, q, k_cache, v_cache, out)) != SA_OK) return st;
  const AttendPlan p = plan_attend(c, kIdxDense, 0, 0);
  if ((st = check_ws(ws, ws_bytes, p.ws_bytes, "sa_dense_decode")) != SA_OK) return st;
  return hip_status(launch_attend(c, p, q, k_cache, v_cache, nullptr, 0, 0, out, ws, stream),
                    "sa_dense_decode launch");
}

size_t sa_dense_scored_workspace_size(const sa_kv_desc* desc) {
  Cache c;
  if (check_desc(desc, &c) != SA_OK) return 0;
  return align_up(dense_scored_ws(c), 256);
}

sa_status sa_dense_decode_scored(const sa_kv_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, float* out, float* scores, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if ((st = check_attend_args(c, q, k_cache, v_cache, out)) != SA_OK) return st;
  if ((st = check_ptr(scores, "scores", 4)) != SA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, dense_scored_ws(c), "sa_dense_decode_scored")) != SA_OK)
    return st;
  return run_dense_scored(c, q, k_cache, v_cache, out, scores, ws, stream);
}

size_t sa_layer_workspace_size(const sa_layer_args* a, sa_layer_mode mode) {
  Cache c;
  if (!a || check_desc(&a->desc, &c) != SA_OK) return 0;
  if (mode != SA_LAYER_DENSE && a->k < 1) return 0;
  if (mode != SA_LAYER_DENSE && a->score_kind == SA_SCORE_BLOCK_MINMAX &&
      (a->aux.block_size < 1 || a->aux.block_size > 4096))
    return 0;
  return layer_ws(c, a, mode).total;
}

sa_status sa_decode_layer(const sa_layer_args* a, sa_layer_mode mode, int32_t* idx,
                          hipStream_t stream) {
  if (!a) return fail(SA_ERR_NULL, "layer args are null");
  Cache c;
  sa_status st;
  if ((st = check_desc(&a->desc, &c)) != SA_OK) return st;
  if (mode != SA_LAYER_DENSE && mode != SA_LAYER_SPARSE && mode != SA_LAYER_REUSE &&
      mode != SA_LAYER_DENSE_SELECT)
    return fail(SA_ERR_SHAPE, "unknown layer mode %d", (int)mode);
  if ((st = check_attend_args(c, a->q, a->k_cache, a->v_cache, a->out)) != SA_OK) return st;
  if (mode == SA_LAYER_DENSE) {
    const LayerWs w = layer_ws(c, a, mode);
    if ((st = check_ws(a->ws, a->ws_bytes, w.total, "sa_decode_layer(DENSE)")) != SA_OK) return st;
    const AttendPlan p = plan_attend(c, kIdxDense, 0, 0);
    return hip_status(launch_attend(c, p, a->q, a->k_cache, a->v_cache, nullptr, 0, 0, a->out,
                                    a->ws, stream),
                      "sa_decode_layer(DENSE) launch");
  }
  // selection-based modes
  if (!known_score_kind(a->score_kind))
    return fail(SA_ERR_SHAPE, "unknown score kind %d", (int)a->score_kind);
  if (mode == SA_LAYER_DENSE_SELECT) {
    if (a->score_kind != SA_SCORE_EXACT)
      return fail(SA_ERR_UNSUPPORTED, "DENSE_SELECT selects on exact scores only (score kind %d)",
                  (int)a->score_kind);
    if (a->k < 1 || a->k > c.N)
      return fail(SA_ERR_SHAPE, "k %d outside [1, %lld]", a->k, (long long)c.N);
    if ((st = check_sparse_idx(c, SA_IDX_TOKEN_PER_KV_HEAD, idx, a->k, 0)) != SA_OK) return st;
    const LayerWs w = layer_ws(c, a, mode);
    if ((st = check_ws(a->ws, a->ws_bytes, w.total, "sa_decode_layer(DENSE_SELECT)")) != SA_OK)
      return st;
    uint8_t* base = static_cast<uint8_t*>(a->ws);
    float* scores = reinterpret_cast<float*>(base);
    void* topk_ws = base + w.scores;
    void* att_ws = base + w.scores + w.topk;
    if ((st = run_dense_scored(c, a->q, a->k_cache, a->v_cache, a->out, scores, att_ws, stream)) !=
        SA_OK)
      return st;
    const int64_t rows = (int64_t)c.B * c.Hkv;
    return hip_status(launch_topk(scores, rows, c.N, c.N, a->k, idx, topk_ws, stream),
                      "sa_decode_layer(DENSE_SELECT) top-k launch");
  }
  const sa_index_kind ik = index_kind_of(a->score_kind);
  const int32_t bs = a->score_kind == SA_SCORE_BLOCK_MINMAX ? a->aux.block_size : 0;
  if (a->score_kind == SA_SCORE_BLOCK_MINMAX) {
    if ((st = check_block_aux(c, &a->aux)) != SA_OK) return st;
  } else if (is_indexer(a->score_kind) && mode == SA_LAYER_SPARSE) {
    if ((st = check_indexer_aux(c, &a->aux)) != SA_OK) return st;
  }
  const int64_t len = score_row_len(c, a->score_kind, &a->aux);
  if (a->k < 1 || a->k > len)
    return fail(SA_ERR_SHAPE, "k %d outside [1, %lld]", a->k, (long long)len);
  if ((st = check_sparse_idx(c, ik, idx, a->k, bs)) != SA_OK) return st;
  const LayerWs w = layer_ws(c, a, mode);
  if ((st = check_ws(a->ws, a->ws_bytes, w.total, "sa_decode_layer")) != SA_OK) return st;
  uint8_t* base = static_cast<uint8_t*>(a->ws);
  float* scores = reinterpret_cast<float*>(base);
  void* topk_ws = base + w.scores;
  void* att_ws = base + w.scores + w.topk;
  const Cache v = attend_view(c, ik);
  const AttendPlan p = plan_attend(v, mode_of(ik), a->k, bs);
  if (mode == SA_LAYER_SPARSE && selectable(a->score_kind)) {
    // the gather-attend runs in the selection's merge launch when the plans
    // allow it (merge_attend_ok), else after it
    const Cache sv = select_view(c, a->score_kind);
    SelectIndexer ixb;
    const MergeAttend ma{v, p, a->q, a->k_cache, a->v_cache, a->out};
    bool attended = false;
    if ((st = hip_status(launch_select(sv, plan_select(sv, a->k), a->q, a->k_cache,
                                       select_indexer(a->score_kind, &a->aux, &ixb), a->k, idx,
                                       base, stream, &ma, &attended),
                         "sa_decode_layer selection launch")) != SA_OK)
      return st;
    if (attended) return SA_OK;
  } else if (mode == SA_LAYER_SPARSE && a->score_kind == SA_SCORE_BLOCK_MINMAX &&
             select_block_fits(c, bs)) {
    // block scores and their top-k in one launch
    if ((st = hip_status(launch_select_block(c, bs, a->q, a->aux.kmin, a->aux.kmax, a->k, idx,
                                             stream),
                         "sa_decode_layer block selection launch")) != SA_OK)
      return st;
  } else if (mode == SA_LAYER_SPARSE) {
    if ((st = do_score(c, a->score_kind, a->q, a->k_cache, &a->aux, scores, stream)) != SA_OK)
      return st;
    const int64_t rows = score_rows(c, a->score_kind);
    if ((st = hip_status(launch_topk(scores, rows, len, len, a->k, idx, topk_ws, stream),
                         "sa_decode_layer top-k launch")) != SA_OK)
      return st;
  }
  return hip_status(
      launch_attend(v, p, a->q, a->k_cache, a->v_cache, idx, a->k, bs, a->out, att_ws, stream),
      "sa_decode_layer attention launch");
}

sa_status sa_plan_validate(const int32_t* modes, const int32_t* src, int32_t n_layers) {
  if (n_layers < 1) return fail(SA_ERR_SHAPE, "n_layers %d must be >= 1", n_layers);
  if (!modes || !src) return fail(SA_ERR_NULL, "modes or src is null");
  if (n_layers > 4096) return fail(SA_ERR_SHAPE, "n_layers %d above 4096", n_layers);
  bool has_idx[4096];
  for (int32_t l = 0; l < n_layers; ++l) {
    const int32_t m = modes[l];
    if (m != SA_LAYER_DENSE && m != SA_LAYER_SPARSE && m != SA_LAYER_REUSE &&
        m != SA_LAYER_DENSE_SELECT)
      return fail(SA_ERR_SHAPE, "layer %d: unknown mode %d", l, m);
    if (m == SA_LAYER_REUSE) {
      const int32_t s = src[l];
      if (s < 0 || s >= l)
        return fail(SA_ERR_SHAPE, "layer %d: reuse source %d is not an earlier layer", l, s);
      if (!has_idx[s]) return fail(SA_ERR_SHAPE, "layer %d: reuse source %d holds no index set", l, s);
    }
    has_idx[l] = (m != SA_LAYER_DENSE);
  }
  return ok();
}

sa_status sa_gather_blocks(const sa_kv_desc* desc, const void* k_host, const void* v_host,
                           const int32_t* idx, int32_t n_blk, int32_t block_size, void* k_out,
                           void* v_out, hipStream_t stream) {
  Cache c;
  sa_status st;
  if ((st = check_desc(desc, &c)) != SA_OK) return st;
  if (block_size < 1 || block_size > 4096)
    return fail(SA_ERR_SHAPE, "block_size %d outside [1, 4096]", block_size);
  if (c.N % block_size != 0)
    return fail(SA_ERR_SHAPE, "ctx_len %lld is not a multiple of block_size %d", (long long)c.N,
                block_size);
  if (n_blk < 1 || n_blk > c.N / block_size)
    return fail(SA_ERR_SHAPE, "n_blk %d outside [1, %lld]", n_blk, (long long)(c.N / block_size));
  if ((st = check_ptr(k_host, "k_host", 16)) != SA_OK) return st;
  if ((st = check_ptr(v_host, "v_host", 16)) != SA_OK) return st;
  if ((st = check_ptr(idx, "idx", 4)) != SA_OK) return st;
  if ((st = check_ptr(k_out, "k_out", 16)) != SA_OK) return st;
  if ((st = check_ptr(v_out, "v_out", 16)) != SA_OK) return st;
  // the device address of each pinned host allocation; fails for memory the
  // runtime does not know as pinned host memory
  void* kd = nullptr;
  void* vd = nullptr;
  if (hipHostGetDevicePointer(&kd, const_cast<void*>(k_host), 0) != hipSuccess || !kd) {
    (void)hipGetLastError();
    return fail(SA_ERR_MEMORY, "k_host is not pinned host memory the device can read");
  }
  if (hipHostGetDevicePointer(&vd, const_cast<void*>(v_host), 0) != hipSuccess || !vd) {
    (void)hipGetLastError();
    return fail(SA_ERR_MEMORY, "v_host is not pinned host memory the device can read");
  }
  return hip_status(
      launch_gather_blocks(c, kd, vd, idx, n_blk, block_size, k_out, v_out, stream),
      "sa_gather_blocks launch");
}

sa_status sa_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream) {
  sa_status st;
  if ((st = check_ptr(data, "data", 16)) != SA_OK) return st;
  if ((st = check_ptr(sink, "sink", 4)) != SA_OK) return st;
  if (bytes == 0 || bytes % 16)
    return fail(SA_ERR_SHAPE, "bytes %zu must be a positive multiple of 16", bytes);
  return hip_status(launch_stream_read(data, bytes, sink, stream), "sa_stream_read launch");
}

sa_status sa_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int32_t k,
                           int32_t* counts, hipStream_t stream) {
  sa_status st;
  if ((st = check_ptr(idx_a, "idx_a", 4)) != SA_OK) return st;
  if ((st = check_ptr(idx_b, "idx_b", 4)) != SA_OK) return st;
  if ((st = check_ptr(counts, "counts", 4)) != SA_OK) return st;
  if (n_rows < 1 || n_rows > INT32_MAX)
    return fail(SA_ERR_SHAPE, "n_rows %lld outside [1, 2^31)", (long long)n_rows);
  if (k < 1) return fail(SA_ERR_SHAPE, "k %d must be >= 1", k);
  return hip_status(launch_index_overlap(idx_a, idx_b, n_rows, k, counts, stream),
                    "sa_index_overlap launch");
}

sa_status sa_plan_reuse(const int64_t* overlap, int64_t total, int32_t n_layers, double theta,
                        const int32_t* sensitive, int32_t* modes, int32_t* src) {
  constexpr int kMaxLayers = 256;
  if (!overlap || !modes || !src) return fail(SA_ERR_NULL, "overlap, modes or src is null");
  if (n_layers < 1 || n_layers > kMaxLayers)
    return fail(SA_ERR_SHAPE, "n_layers %d outside [1, %d]", n_layers, kMaxLayers);
  if (total < 1) return fail(SA_ERR_SHAPE, "total %lld must be >= 1", (long long)total);
  if (isnan(theta)) return fail(SA_ERR_SHAPE, "theta is NaN");
  const int L = n_layers;
  for (int i = 0; i < L; ++i)
    for (int j = i + 1; j < L; ++j) {
      const int64_t o = overlap[(int64_t)i * L + j];
      if (o < 0 || o > total)
        return fail(SA_ERR_SHAPE, "overlap[%d][%d] = %lld outside [0, total]", i, j, (long long)o);
    }
  // may_reuse(i, j): layer j may reuse the set of layer i (the vertical move
  // into (i, j) is allowed)
  auto may_reuse = [&](int i, int j) {
    if (sensitive && sensitive[j]) return false;
    return (double)overlap[(int64_t)i * L + j] / (double)total > theta;
  };
  // Suffix dynamic programme over reset layers: (fulls[j], sim[j]) = the
  // best (full layers, summed overlap) of layers j..L-1 given that layer j
  // resets; next[j] = the following reset layer (L: none).  The reused run
  // after reset j is
  // j+1..j'-1, so the policy's path is (j, j) -> (j, j+1) -> ... -> (j, j'-1)
  // -> (j', j').
  int32_t fulls[kMaxLayers + 1];
  int64_t sim[kMaxLayers + 1];
  int32_t next[kMaxLayers + 1];
  fulls[L] = 0;
  sim[L] = 0;
  for (int j = L - 1; j >= 0; --j) {
    int32_t bf = INT32_MAX;
    int64_t bs = -1;
    int32_t bn = -1;
    int64_t run = 0;  // summed overlap of layers j+1 .. jn-1 reusing layer j
    for (int jn = j + 1; jn <= L; ++jn) {
      // candidate: layers j+1 .. jn-1 reuse j (checked below on the way),
      // jn resets (jn == L: no further reset); on a tie the later jn wins
      const int32_t f = 1 + fulls[jn];
      const int64_t sv = run + sim[jn];
      if (f < bf || (f == bf && sv >= bs)) {
        bf = f;
        bs = sv;
        bn = jn;
      }
      if (jn == L || !may_reuse(j, jn)) break;  // layer jn cannot join the run
      run += overlap[(int64_t)j * L + jn];
    }
    fulls[j] = bf;
    sim[j] = bs;
    next[j] = bn;
  }
  for (int l = 0; l < L; ++l) src[l] = -1;
  int j = 0;
  while (j < L) {
    const int jn = next[j];
    modes[j] = jn > j + 1 ? SA_LAYER_DENSE_SELECT : SA_LAYER_DENSE;
    for (int t = j + 1; t < jn; ++t) {
      modes[t] = SA_LAYER_REUSE;
      src[t] = j;
    }
    j = jn;
  }
  return ok();
}

sa_status sa_plan_fixed_jump(int32_t n_layers, int32_t step, int32_t* modes, int32_t* src) {
  if (!modes || !src) return fail(SA_ERR_NULL, "modes or src is null");
  if (n_layers < 1 || n_layers > 256)
    return fail(SA_ERR_SHAPE, "n_layers %d outside [1, 256]", n_layers);
  if (step < 1) return fail(SA_ERR_SHAPE, "step %d must be >= 1", step);
  for (int32_t l = 0; l < n_layers; ++l) {
    if (l % step == 0) {
      const bool reused = step > 1 && l + 1 < n_layers;
      modes[l] = reused ? SA_LAYER_DENSE_SELECT : SA_LAYER_DENSE;
      src[l] = -1;
    } else {
      modes[l] = SA_LAYER_REUSE;
      src[l] = l - l % step;
    }
  }
  return ok();
}

}  // extern "C"
