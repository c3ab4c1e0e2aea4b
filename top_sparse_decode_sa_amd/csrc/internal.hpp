// Host-side interfaces between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa.h"

namespace sa {

// Validated view of one layer's KV cache (strides in elements).  A "row" is
// (sequence, r) for r < Hkv; row r reads KV head r / kv_div and query heads
// r*G .. r*G + G - 1.
struct Cache {
  int32_t B, Hq, Hkv, G, D;
  int64_t N;
  sa_dtype q_dtype, kv_dtype;
  int64_t sb, sh, st;
  float scale;  // softmax scale (already defaulted)
  int32_t kv_div = 1;
};

// The same cache seen with one row per (sequence, QUERY head): G = 1 and row
// h reads KV head h / G of the real cache, so every query head scores and
// selects on its own.
inline Cache per_q_head_view(const Cache& c) {
  Cache v = c;
  v.Hkv = c.Hq;
  v.G = 1;
  v.kv_div = c.G * c.kv_div;
  return v;
}

// Rows of the per-query-head view that read one KV row (its query heads:
// kv_div), when 2 or 4: the exact scoring reads each key row once for all
// of them.  1 otherwise (scored row by row; eight queries per key load
// would not fit the registers).
inline int per_q_head_shared_rows(const Cache& c) {
  const bool view = c.G == 1 && c.kv_div > 1 && c.Hkv % c.kv_div == 0;
  return view && (c.kv_div == 2 || c.kv_div == 4) ? c.kv_div : 1;
}

// ------------------------------------------------------------- scoring
hipError_t launch_score_exact(const Cache& c, const void* q, const void* k, float* scores,
                              hipStream_t s);
hipError_t launch_block_summarize(const Cache& c, int32_t bs, const void* k, void* kmin, void* kmax,
                                  hipStream_t s);
hipError_t launch_score_block(const Cache& c, int32_t bs, const void* q, const void* kmin,
                              const void* kmax, float* scores, hipStream_t s);
// Block scores and their top-k in one launch (one workgroup per row), for
// rows of at most 4096 blocks (select_block_fits): idx [rows, k] ascending,
// the same list as launch_score_block followed by launch_topk.
bool select_block_fits(const Cache& c, int32_t bs);
hipError_t launch_select_block(const Cache& c, int32_t bs, const void* q, const void* kmin,
                               const void* kmax, int32_t k, int32_t* idx, hipStream_t s);
// With hist, the launch also adds the 12-bit key histogram of row b's scores
// into hist + b * hist_stride (the counted top-k below).
hipError_t launch_score_indexer(int32_t B, int64_t N, int32_t H, int32_t Di, const void* q_idx,
                                const void* k_idx, const float* w, float* scores, hipStream_t s,
                                uint32_t* hist = nullptr, int64_t hist_stride = 0);

// --------------------------------------------------------------- top-k
size_t topk_workspace_bytes(int64_t n_rows, int64_t n, int32_t k);
hipError_t launch_topk(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride, int32_t k,
                       int32_t* idx, void* ws, hipStream_t s);
// The multi-workgroup top-k of few long rows with the histogram counted by the
// launch that writes the scores: when topk_counted(rows, n, k), run
// launch_topk_counted_zero, then the scoring launch adding into
// topk_counted_hist(ws) (row r at + r * stride words), then
// launch_topk_counted; same result and workspace as launch_topk.
bool topk_counted(int64_t n_rows, int64_t n, int32_t k);
uint32_t* topk_counted_hist(void* ws, int64_t* stride_words);
hipError_t launch_topk_counted_zero(void* ws, int64_t n_rows, hipStream_t s);
hipError_t launch_topk_counted(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride,
                               int32_t k, int32_t* idx, void* ws, hipStream_t s);
// Top-k of candidate rows (n <= 32768 values each, row stride cstride) whose
// element i stands for position pos[i]: idx gets the k selected positions in
// ascending candidate order.
hipError_t launch_topk_merge(const float* cand_val, const int32_t* cand_pos, int64_t n_rows,
                             int64_t n, int64_t cstride, int32_t k, int32_t* idx, hipStream_t s);
// counts[r] = |idx_a[r, :] intersect idx_b[r, :]|, rows of k ascending indices.
hipError_t launch_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int32_t k,
                                int32_t* counts, hipStream_t s);

// ------------------------------------------------------- fused select
// Top-k of every row of c (B * Hkv rows; per_q_head_view for one row per
// query head) by exact or indexer scores, without writing the scores: rows
// are cut into parts of L tokens scored and pre-selected in LDS, then merged.
// Falls back to scoring plus top-k when the part candidates would be more
// than a quarter of the row.
struct SelectPlan {
  int32_t L = 0;        // tokens per part (a multiple of 256, at most 8192)
  int32_t P = 0;        // parts per row
  int32_t kcap = 0;     // candidate slots per part: min(k, L)
  int64_t C = 0;        // candidates per row
  int64_t cstride = 0;  // candidate row stride (C rounded up to 4)
  bool fused = false;
  size_t ws_bytes = 0;  // workspace of the chosen path
};
// Indexer scoring instead of exact scores: rows of c (B * Hkv) are the
// indexer's rows; q_idx [rows, H, Di] bf16, k_idx [rows, N, Di] bf16,
// w [rows, H] fp32.
struct SelectIndexer {
  const void* q_idx;
  const void* k_idx;
  const float* w;
  int32_t H, Di;
};
SelectPlan plan_select(const Cache& c, int32_t k);
struct MergeAttend;
// With `ma`, the gather-attend that follows may run in the merge's launch
// (merge_attend_ok); *attended then says whether it did.
hipError_t launch_select(const Cache& c, const SelectPlan& p, const void* q, const void* k,
                         const SelectIndexer* ix, int32_t kk, int32_t* idx, void* ws,
                         hipStream_t s, const MergeAttend* ma = nullptr, bool* attended = nullptr);

// ----------------------------------------------------------- attention
// kIdxDenseScored: dense decode that also writes each token's exact score
// (scale * sum_g q_g . k_t) from the logits it computes anyway.
enum IndexMode : int {
  kIdxTokenPerHead = 0,
  kIdxTokenShared = 1,
  kIdxBlockPerHead = 2,
  kIdxDense = 3,
  kIdxDenseScored = 4
};

inline bool is_dense_mode(int mode) { return mode == kIdxDense || mode == kIdxDenseScored; }

// Which gather-attend kernel a plan runs: lane groups holding whole rows (any
// dtype and head size), MFMA waves over rounds of tiles (bf16, head_dim 128,
// dense scans and blocks), or MFMA waves pipelined by pairs of tiles (bf16,
// head_dim 128, selected tokens).
enum AttendKernel : int { kKernGeneric = 0, kKernWave = 1, kKernPairs = 2 };

struct AttendPlan {
  int mode;
  int kernel;       // AttendKernel
  int64_t n_slots;  // selected slots per row (tokens, or block slots)
  int32_t chunk;    // slots per workgroup
  int32_t nsplit;   // workgroups per row
  int32_t waves;    // waves per workgroup
  int32_t rounds;   // slot rounds per wave (kKernWave)
  int32_t pairs;    // pairs of 16-slot tiles per wave (kKernPairs)
  int32_t vhalves;  // kKernPairs: 2 = two workgroups per row, one per half of the value dims
  size_t ws_bytes;  // split partials (0 when nsplit == 1)
};

AttendPlan plan_attend(const Cache& c, int mode, int32_t n_idx, int32_t bs);
// scores: kIdxDenseScored only, [B, Hkv, N] fp32.
// The gather-attend's reads alone for a kKernPairs plan (measurement reference).
hipError_t launch_gather_read(const Cache& c, const AttendPlan& p, const void* k, const void* v,
                              const int32_t* idx, int32_t n_idx, int32_t bs, uint32_t* sink,
                              hipStream_t s);
hipError_t launch_attend(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                         const void* v, const int32_t* idx, int32_t n_idx, int32_t bs, float* out,
                         void* ws, hipStream_t s, float* scores = nullptr);
bool fused_scores_supported(const Cache& c);

// The gather-attend over a selection's index list: cache view, plan, q,
// K/V and the output.
struct MergeAttend {
  Cache c;
  AttendPlan p;
  const void* q;
  const void* k;
  const void* v;
  float* out;
};

// Merge-then-attend (the selection's merge and a whole-row gather-attend in
// one launch): whether plan p over n_cand candidates per row allows it, and
// the launch, which writes idx [rows, kk] and out.
bool merge_attend_ok(const Cache& c, const AttendPlan& p, int64_t n_cand, int32_t k);
hipError_t launch_merge_attend(const Cache& c, const AttendPlan& p, const void* q, const void* k,
                               const void* v, float* out, const float* cand_val,
                               const int32_t* cand_pos, int64_t n_cand, int64_t cstride, int32_t kk,
                               int32_t* idx, hipStream_t s);

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// ------------------------------------------------------- index checks
// counts[0] = rows of `rows` x n indices with one outside [0, limit);
// counts[1] = rows with a repeated index.  n <= kCheckMaxIdx.
constexpr int32_t kCheckMaxIdx = 8192;
hipError_t launch_check_indices(const int32_t* idx, int64_t rows, int32_t n, int64_t limit,
                                int32_t* counts, hipStream_t s);

// ------------------------------------------------------------- offload
// k_dev / v_dev: device addresses of a cache in pinned host memory; c.N is a
// multiple of bs.  Out: [B, Hkv, n_blk * bs, D] contiguous.
hipError_t launch_gather_blocks(const Cache& c, const void* k_dev, const void* v_dev,
                                const int32_t* idx, int32_t n_blk, int32_t bs, void* k_out,
                                void* v_out, hipStream_t s);

// --------------------------------------------------------- measurement
// A plain streaming read of `bytes` (a multiple of 16) of device memory.
hipError_t launch_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------ allocation-free calls
// Bytes of the static device scratch of sa_sparse_decode_noalloc (16 MiB).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
// Its device address on the device of `stream` (looked up once per device).
sa_status noalloc_scratch(hipStream_t stream, void** out);

}  // namespace sa
