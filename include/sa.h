/*
 * sa.h -- C ABI of the top-k sparse decode attention library (libsa.so).
 *
 * One decode step of one attention layer, for a batch of sequences whose keys
 * and values sit in a device-resident KV cache:
 *   1. score every cached token against the current query   (sa_score)
 *   2. keep the top-k tokens or token blocks per row          (sa_topk)
 *      -- for exact or indexer scores, steps 1 and 2 in one
 *      pass that keeps the scores on chip                     (sa_select)
 *   3. gather only those K/V rows and run a split-K
 *      online-softmax decode over them                        (sa_sparse_decode)
 * plus full-attention decode for layers routed dense (sa_dense_decode) and a
 * per-layer mode flag that runs one of these paths or reuses the index set of
 * an earlier layer (sa_decode_layer, sa_plan_validate).
 *
 * Sources for what each call computes (pages describing the method):
 *   [P1] "Flux Attention: Context-Aware Hybrid Attention for Efficient LLMs
 *        Inference", paper review: per-layer hard choice of full or sparse
 *        attention (key terms; method).
 *   [P2] "HyLRA: Hybrid Layer Reuse Attention", technical summary: index reuse
 *        across layers (sections 2.2-2.3), 128-token blocks (section 2.4).
 *   [P3] "Inference-time context sparsity: illusion or opportunity?",
 *        technical summary: oracle top-k (section 2), a sparse decode kernel
 *        with irregular token-level sparsity and O(k*d) traffic (section 3.C).
 *   [P5] "Flash Attention vs Sparse Attention": tiling with online softmax;
 *        DSA indexer (Stage 1) and selective attention (Stage 2); IndexCache.
 *
 * Conventions shared by every call
 *   - Every pointer argument named *_cache, q, out, scores, idx*, kmin, kmax,
 *     ws is a DEVICE pointer; descriptors and plan arrays are HOST pointers;
 *     *_host (sa_gather_blocks) point to pinned host memory.
 *   - The caller owns every buffer.  No call allocates or frees device memory
 *     or keeps state between calls.
 *   - Every call validates its arguments on the host first.  On an invalid
 *     argument it returns an error code with NOTHING enqueued; the reason is
 *     available from sa_last_error() on the calling thread.
 *   - On success the work is enqueued on `stream` and the call returns
 *     without synchronising.  A launch failure returns SA_ERR_HIP.
 *   - Calls are thread-safe.  Two calls that run concurrently must not share
 *     a workspace.
 *   - Workspaces: any call taking (ws, ws_bytes) needs at least the bytes the
 *     matching *_workspace_size() function returns (0 means none; ws may then
 *     be null), 256-byte aligned.  The library only uses it as scratch
 *     between the launches of one call: no initialisation is needed and
 *     nothing is kept in it between calls.
 *   - Layouts are row-major.  "Row" means one (sequence, KV head) pair.
 *     Query head h belongs to KV head h / G with G = n_q_heads / n_kv_heads.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

/* The enumerations are 32-bit integers on both sides of the ABI.  C++ gets
 * the fixed underlying type written out, so that a value outside the listed
 * ones (which a C caller may pass, and which the calls reject) is still a
 * valid value of the type. */
#ifdef __cplusplus
#define SA_ENUM enum : int32_t
#else
#define SA_ENUM enum
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility: the functions declared
 * here are its only exports. */
#pragma GCC visibility push(default)

typedef SA_ENUM {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is null */
  SA_ERR_SHAPE = 2,       /* a size, count, stride or k is out of range */
  SA_ERR_ALIGN = 3,       /* a pointer or stride breaks 16-byte (ws: 256-byte) alignment */
  SA_ERR_DTYPE = 4,       /* unknown dtype, or a dtype the call does not take */
  SA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  SA_ERR_UNSUPPORTED = 6, /* valid but not built (e.g. head_dim 96, group size 3) */
  SA_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  SA_ERR_MEMORY = 8       /* a buffer is not the kind of memory the call needs */
} sa_status;

typedef SA_ENUM { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

/* One layer's KV cache and query shape.
 *   K and V: element (b, h, t, i) at base + b*kv_stride_b + h*kv_stride_h
 *            + t*kv_stride_t + i   (strides in ELEMENTS; K and V share them).
 *   q:       [batch, n_q_heads, head_dim], contiguous, q_dtype.
 * Limits: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0 with the group
 * size G in {1, 2, 4, 8}; 1 <= ctx_len < 2^31; kv_stride_t >= head_dim; every
 * stride times the element size a multiple of 16 bytes; cache and q base
 * pointers 16-byte aligned.  softmax_scale 0 means 1/sqrt(head_dim). */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t ctx_len;
  sa_dtype q_dtype;
  sa_dtype kv_dtype;
  int64_t kv_stride_b;
  int64_t kv_stride_h;
  int64_t kv_stride_t;
  float softmax_scale;
} sa_kv_desc;

/* ---------------------------------------------------------------- scoring */

typedef SA_ENUM {
  /* Exact score of every token of every row: [P3] section 2 (oracle top-k).
   *   scores[b, r, t] = scale * sum_{g < G} q[b, r*G + g, :] . K[b, r, t, :]
   * Output [batch, n_kv_heads, ctx_len] fp32. */
  SA_SCORE_EXACT = 0,
  /* Block upper bound from per-block key summaries: [P2] section 2.4.
   *   scores[b, r, j] = sum_{g<G} sum_i max(q_gi * kmin[b,r,j,i], q_gi * kmax[b,r,j,i])
   * (no scale).  Output [batch, n_kv_heads, ceil(ctx_len / block_size)] fp32. */
  SA_SCORE_BLOCK_MINMAX = 1,
  /* Low-dimensional indexer: [P5] DSA Stage 1.
   *   scores[b, t] = sum_{h < n_idx_heads} w[b, h] * max(0, q_idx[b, h, :] . k_idx[b, t, :])
   * Output [batch, ctx_len] fp32 (one row per sequence, shared by its KV heads). */
  SA_SCORE_INDEXER = 2,
  /* The same indexer form with one indexer per KV head, so selection is per
   * (sequence, KV head) as for SA_SCORE_EXACT:
   *   scores[b, r, t] = sum_{h < n_idx_heads} w[b, r, h] *
   *                     max(0, q_idx[b, r, h, :] . k_idx[b, r, t, :])
   * q_idx [batch, n_kv_heads, n_idx_heads, idx_dim] bf16, k_idx [batch,
   * n_kv_heads, ctx_len, idx_dim] bf16, w [batch, n_kv_heads, n_idx_heads]
   * fp32, all contiguous.  Output [batch, n_kv_heads, ctx_len] fp32. */
  SA_SCORE_INDEXER_PER_KV_HEAD = 3,
  /* Exact score per QUERY head, for selection that differs between the query
   * heads of a group ([P3] section 2: the sparse decode kernel takes
   * irregular patterns per token, per query and per head):
   *   scores[b, h, t] = scale * q[b, h, :] . K[b, h / G, t, :]
   * Output [batch, n_q_heads, ctx_len] fp32; batch * n_q_heads <= 65535. */
  SA_SCORE_EXACT_PER_Q_HEAD = 4
} sa_score_kind;

typedef struct {
  /* SA_SCORE_BLOCK_MINMAX: summaries from sa_block_summarize, kv_dtype,
   * [batch, n_kv_heads, ceil(ctx_len / block_size), head_dim], contiguous. */
  const void* kmin;
  const void* kmax;
  int32_t block_size;
  /* SA_SCORE_INDEXER: q_idx [batch, n_idx_heads, idx_dim] bf16,
   * k_idx [batch, ctx_len, idx_dim] bf16, w [batch, n_idx_heads] fp32, all
   * contiguous; 1 <= n_idx_heads <= 16, idx_dim in {32, 64, 128}. */
  const void* q_idx;
  const void* k_idx;
  const float* idx_w;
  int32_t n_idx_heads;
  int32_t idx_dim;
} sa_score_aux;

/* Score every cached token (or block).  `aux` may be null for SA_SCORE_EXACT. */
sa_status sa_score(const sa_kv_desc* desc, sa_score_kind kind, const void* q, const void* k_cache,
                   const sa_score_aux* aux, float* scores, hipStream_t stream);

/* Per-block elementwise min and max of the keys: [P2] section 2.4 (fixed
 * blocks, QUEST-compatible summaries).  kmin/kmax: [batch, n_kv_heads,
 * ceil(ctx_len / block_size), head_dim] in kv_dtype, contiguous.  The last
 * block summarises only the tokens below ctx_len.  1 <= block_size <= 4096. */
sa_status sa_block_summarize(const sa_kv_desc* desc, int32_t block_size, const void* k_cache,
                             void* kmin, void* kmax, hipStream_t stream);

/* ------------------------------------------------------------------ top-k */

/* Top-k of each row of an fp32 score matrix: [P3] section 2 (oracle top-k)
 * and [P5] DSA Stage 1 (a top-K index list).
 *   scores: [n_rows] rows of n values, row r starting at scores + r*row_stride
 *           (row_stride >= n, in elements).
 *   idx_out: [n_rows, k] int32, each row the k positions with the largest
 *           scores in ASCENDING position order; equal scores are taken from
 *           the lower position first; -0.0 equals +0.0; NaN ranks below
 *           -inf.  The result is exact and deterministic.
 * Limits: 1 <= n_rows < 2^22, 1 <= k <= n < 2^31. */
sa_status sa_topk(const float* scores, int64_t n_rows, int64_t n, int64_t row_stride, int32_t k,
                  int32_t* idx_out, void* ws, size_t ws_bytes, hipStream_t stream);
size_t sa_topk_workspace_size(int64_t n_rows, int64_t n, int32_t k);

/* Selection in one pass over the keys: the index list that sa_score(kind)
 * followed by sa_topk(k) writes ([P3] section 2, oracle top-k; [P5] DSA
 * Stage 1, a top-K index list from the indexer), identical position for
 * position, without writing the scores.  kind and idx_out:
 *   SA_SCORE_EXACT                [batch, n_kv_heads, k]
 *   SA_SCORE_EXACT_PER_Q_HEAD     [batch, n_q_heads, k]  (batch * n_q_heads <= 65535)
 *   SA_SCORE_INDEXER              [batch, k]            (aux as for sa_score)
 *   SA_SCORE_INDEXER_PER_KV_HEAD  [batch, n_kv_heads, k] (aux as for sa_score)
 * q and k_cache are read for the exact kinds, aux for the indexers (q and
 * k_cache may then be null).
 * Method: each row is cut into parts of at most 8192 tokens; a workgroup
 * scores its part into on-chip memory and keeps the part's top-k as (score,
 * position) candidates; a merge selects the row's top-k among them (every
 * element of the row's top-k is in its part's top-k).  When the candidates
 * would be more than a quarter of the row it runs sa_score and sa_topk
 * instead (same result); so does SA_SCORE_EXACT_PER_Q_HEAD on rows longer
 * than one part, whose scoring reads each key row once for the 2 or 4
 * query heads of its KV head.  ws: sa_select_workspace_size bytes (may be 0),
 * 256-byte aligned; no state is kept in it between calls.
 * Errors: SA_ERR_NULL / SA_ERR_ALIGN for q, k_cache (16 bytes), idx_out or
 * the indexer tensors; SA_ERR_SHAPE for another kind, bad indexer sizes or k
 * outside [1, ctx_len]; SA_ERR_WORKSPACE when ws_bytes is short. */
sa_status sa_select(const sa_kv_desc* desc, sa_score_kind kind, const void* q, const void* k_cache,
                    const sa_score_aux* aux, int32_t k, int32_t* idx_out, void* ws,
                    size_t ws_bytes, hipStream_t stream);
size_t sa_select_workspace_size(const sa_kv_desc* desc, sa_score_kind kind, int32_t k);

/* ------------------------------------------------------------ attention */

typedef SA_ENUM {
  /* idx [batch, n_kv_heads, n_idx] token positions, one set per row. */
  SA_IDX_TOKEN_PER_KV_HEAD = 0,
  /* idx [batch, n_idx] token positions shared by every KV head of a sequence. */
  SA_IDX_TOKEN_SHARED = 1,
  /* idx [batch, n_idx_rows=n_kv_heads, n_idx] ids of block_size-token blocks;
   * a block covers tokens [j*block_size, min((j+1)*block_size, ctx_len)). */
  SA_IDX_BLOCK_PER_KV_HEAD = 2,
  /* idx [batch, n_q_heads, n_idx] token positions, one set per QUERY head
   * ([P3] section 2); query head h reads its own tokens of KV head h / G.
   * batch * n_q_heads <= 65535. */
  SA_IDX_TOKEN_PER_Q_HEAD = 3
} sa_index_kind;

/* Attention of every query head over the selected set of its row only:
 * [P5] DSA Stage 2 and [P3] section 3.C (a decode kernel for irregular
 * token-level sparsity that reads O(k*d) of the cache).  For query head h of
 * sequence b, with S the selected tokens of row (b, h / G) (of row (b, h)
 * for SA_IDX_TOKEN_PER_Q_HEAD):
 *   out[b, h, :] = sum_{t in S} softmax_S(scale * q[b,h,:] . K[b,h/G,t,:]) * V[b,h/G,t,:]
 * out: [batch, n_q_heads, head_dim] fp32.  Preconditions: every index in
 * range and the indices of one row distinct (not checked here; see
 * sa_check_indices); 1 <= n_idx.  For bf16 caches with head_dim 128 and
 * token indices, an index outside the row reads zeros or another token of the
 * row, never memory outside the row's cache.
 * Computed as a split-K online softmax ([P5] tiling + online softmax): each
 * workgroup attends a run of a row's slots; when a row is split over several
 * workgroups their partial results (o, max, sum) are merged by a log-sum-exp
 * combine in a second launch (the workspace holds them in between). */
sa_status sa_sparse_decode(const sa_kv_desc* desc, const void* q, const void* k_cache,
                           const void* v_cache, sa_index_kind ik, const int32_t* idx, int32_t n_idx,
                           int32_t block_size, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);
size_t sa_sparse_workspace_size(const sa_kv_desc* desc, sa_index_kind ik, int32_t n_idx,
                                int32_t block_size);

/* Check an index list before sa_sparse_decode (or before a REUSE layer reads
 * it): [P3] section 3.C attends over a set of tokens, so each row's indices
 * must name distinct tokens (blocks) inside the cache.  One launch writes
 *   counts[0] = number of rows holding an index outside [0, ctx_len)
 *               (block kind: outside [0, ceil(ctx_len / block_size)))
 *   counts[1] = number of rows in which some index appears more than once
 * (counts: int32[2], device, overwritten).  Rows and layout as for
 * sa_sparse_decode with the same index kind.  Indices are only read as data.
 * Limits: 1 <= n_idx <= 8192 (larger: SA_ERR_UNSUPPORTED). */
sa_status sa_check_indices(const sa_kv_desc* desc, sa_index_kind ik, const int32_t* idx,
                           int32_t n_idx, int32_t block_size, int32_t* counts,
                           hipStream_t stream);

/* sa_sparse_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and results, without (ws,
 * ws_bytes).  The split partials that sa_sparse_decode keeps in the caller's
 * workspace go to a static device array of the library instead, 16 MiB
 * (16777216 bytes), which every GPU the library runs on holds until the
 * process ends; a call whose plan needs more (sa_sparse_workspace_size above
 * 16 MiB) returns SA_ERR_WORKSPACE with nothing enqueued.  The call allocates
 * nothing; the first call on a device looks the array's address up on that
 * device (the device of `stream`).  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (different streams, or different
 * threads) race on it and must be serialised by the caller. */
sa_status sa_sparse_decode_noalloc(const sa_kv_desc* desc, const void* q, const void* k_cache,
                                   const void* v_cache, sa_index_kind ik, const int32_t* idx,
                                   int32_t n_idx, int32_t block_size, float* out,
                                   hipStream_t stream);

/* Full decode attention over all ctx_len tokens (layers routed to full
 * attention, [P1]; the dense baseline of [P3] section 3.C).  Same output as
 * sa_sparse_decode with S = [0, ctx_len). */
sa_status sa_dense_decode(const sa_kv_desc* desc, const void* q, const void* k_cache,
                          const void* v_cache, float* out, void* ws, size_t ws_bytes,
                          hipStream_t stream);
size_t sa_dense_workspace_size(const sa_kv_desc* desc);

/* Full decode attention that also writes the exact score of every token
 * ([P2] section 2.3: a sensitive layer runs full attention and passes the
 * top-k indices it extracts on to the layers that reuse them).  out is what
 * sa_dense_decode writes; scores [batch, n_kv_heads, ctx_len] fp32 is what
 * sa_score(SA_SCORE_EXACT) writes, up to fp32 summation order:
 *   scores[b, r, t] = scale * sum_{g < G} q[b, r*G + g, :] . K[b, r, t, :]
 * For bf16 q and K with head_dim 128 and G <= 4 the scores come out of the
 * attention kernel's own logits (one pass over K); other shapes run the
 * scoring and the attention as two launches. */
sa_status sa_dense_decode_scored(const sa_kv_desc* desc, const void* q, const void* k_cache,
                                 const void* v_cache, float* out, float* scores, void* ws,
                                 size_t ws_bytes, hipStream_t stream);
size_t sa_dense_scored_workspace_size(const sa_kv_desc* desc);

/* ----------------------------------------------------- per-layer mode flag */

typedef SA_ENUM {
  SA_LAYER_DENSE = 0,  /* full attention; idx untouched */
  SA_LAYER_SPARSE = 1, /* score -> top-k -> selected-set attention; WRITES idx.
                        * With exact or per-KV-head indexer scores the
                        * selection is sa_select's; when its candidates are
                        * merged and a row's attention fits one workgroup the
                        * merge and the attention run in one launch (the same
                        * idx and out as the separate calls). */
  SA_LAYER_REUSE = 2,  /* selected-set attention over idx as given; READS idx */
  SA_LAYER_DENSE_SELECT = 3 /* full attention + top-k of its exact scores; WRITES idx */
} sa_layer_mode;

/* Everything one layer's decode step needs.  The score kind fixes the index
 * kind: EXACT and INDEXER_PER_KV_HEAD -> SA_IDX_TOKEN_PER_KV_HEAD,
 * BLOCK_MINMAX -> SA_IDX_BLOCK_PER_KV_HEAD (aux.block_size), INDEXER ->
 * SA_IDX_TOKEN_SHARED, EXACT_PER_Q_HEAD -> SA_IDX_TOKEN_PER_Q_HEAD.
 * k is the number of tokens (blocks for BLOCK_MINMAX) kept per row. */
typedef struct {
  sa_kv_desc desc;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  sa_score_kind score_kind;
  sa_score_aux aux;
  int32_t k;
  float* out;
  void* ws;
  size_t ws_bytes;
} sa_layer_args;

/* One layer of decode under a per-layer mode: [P1] hard routing between full
 * and sparse attention; [P2] sections 2.2-2.3 and [P5] IndexCache: a layer may
 * reuse the top-k index set an earlier layer produced, unchanged.
 *   DENSE:  sa_dense_decode.
 *   SPARSE: sa_score -> sa_topk -> sa_sparse_decode (sa_select for the exact
 *           and indexer score kinds, the same index set), the index set written to
 *           idx ([batch, n_kv_heads, k]; [batch, k] for INDEXER; [batch,
 *           n_q_heads, k] for EXACT_PER_Q_HEAD).
 *   REUSE:  sa_sparse_decode over idx exactly as given (no scoring, no top-k);
 *           idx must hold the set of an earlier SPARSE or DENSE_SELECT layer
 *           with the same score kind and k.
 *   DENSE_SELECT: [P2] sections 2.2-2.3, a "reset" layer: sa_dense_decode_scored
 *           -> sa_topk of those exact scores into idx [batch, n_kv_heads, k].
 *           Needs score_kind SA_SCORE_EXACT (else SA_ERR_UNSUPPORTED).
 * idx may be null for DENSE. */
sa_status sa_decode_layer(const sa_layer_args* a, sa_layer_mode mode, int32_t* idx,
                          hipStream_t stream);
size_t sa_layer_workspace_size(const sa_layer_args* a, sa_layer_mode mode);

/* Check a per-layer plan on the host: modes[l] in sa_layer_mode; a REUSE layer
 * needs 0 <= src[l] < l with layer src[l] owning an index set (SPARSE,
 * DENSE_SELECT, or a REUSE layer, which carries its source's set).  src[l] is
 * ignored for other modes.  Returns SA_OK or SA_ERR_SHAPE (reason in
 * sa_last_error). */
sa_status sa_plan_validate(const int32_t* modes, const int32_t* src, int32_t n_layers);

/* ------------------------------------------- layer-reuse policy ([P2] 2.2) */

/* Top-k overlap of two index sets per row: [P2] section 2.2, the entries of
 * the similarity matrix count how many top-k token indices a source layer and
 * a target layer share.  idx_a, idx_b: [n_rows, k] int32 (device), each row
 * k distinct positions in ASCENDING order (what sa_topk writes; not checked:
 * an unsorted row gives a wrong count, never an out-of-range access).
 *   counts[r] = |{idx_a[r, :]} intersect {idx_b[r, :]}|   (int32, device)
 * Limits: 1 <= n_rows < 2^31, 1 <= k. */
sa_status sa_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t n_rows, int32_t k,
                           int32_t* counts, hipStream_t stream);

/* Offline layer policy by dynamic programming: [P2] section 2.2 (HOST call,
 * host arrays).  Layer j either runs full attention and refreshes the index
 * set (a "reset jump" to state (j, j)) or reuses the set of the last reset
 * layer i (a "vertical move" (i, j-1) -> (i, j)), allowed only when their
 * overlap ratio exceeds theta:
 *   overlap[i * n_layers + j] / total > theta      (compared in double)
 * where overlap[i * n_layers + j] (i < j; other entries unread) is the summed
 * sa_index_overlap count of layers i and j over all rows and total = n_rows * k.
 * Layer 0 and every layer with sensitive[l] != 0 (may be null) run full
 * attention.  Among feasible plans the one with the fewest full layers wins,
 * then the largest summed overlap of the reused layers; remaining ties go to
 * the plan whose list of full layers is lexicographically largest (resets as
 * late as possible).  Output: modes[l] is SA_LAYER_DENSE_SELECT for a full
 * layer whose set a later layer reuses, SA_LAYER_DENSE for any other full
 * layer, SA_LAYER_REUSE with src[l] = its reset layer otherwise (src[l] = -1
 * for full layers).  Limits: 1 <= n_layers <= 256, total >= 1, overlap
 * entries in [0, total]. */
sa_status sa_plan_reuse(const int64_t* overlap, int64_t total, int32_t n_layers, double theta,
                        const int32_t* sensitive, int32_t* modes, int32_t* src);

/* The static baseline of [P2] section 4 ("Jump" with a fixed step): layers
 * 0, step, 2*step, ... run full attention and every other layer reuses the
 * set of the full layer before it.  modes/src as in sa_plan_reuse.  Limits:
 * 1 <= n_layers <= 256, step >= 1. */
sa_status sa_plan_fixed_jump(int32_t n_layers, int32_t step, int32_t* modes, int32_t* src);

/* ------------------------------------------------------------- offload */

/* Index-guided offload: [P2] section 2.4, when the KV cache exceeds device
 * memory the (reused) index set decides which blocks are fetched from host
 * memory.  Copies the selected blocks of one layer's K and V, held in PINNED
 * HOST memory (k_host, v_host: host pointers of one pinned allocation each,
 * laid out as desc says), into device buffers:
 *   k_out[b, r, j*block_size + i, :] = K[b, r, idx[b, r, j]*block_size + i, :]
 * (same for V), k_out/v_out [batch, n_kv_heads, n_blk*block_size, head_dim]
 * contiguous, kv_dtype, 16-byte aligned (device).  idx [batch, n_kv_heads,
 * n_blk] int32 block ids (device); an id outside [0, ctx_len/block_size) is
 * clamped into it (the kernel never reads outside the cache).  The GPU reads
 * the host cache directly over the host link.  Full decode attention over the
 * gathered buffers (sa_dense_decode with ctx_len = n_blk*block_size) is then
 * the selected-block attention of SA_IDX_BLOCK_PER_KV_HEAD.
 * Limits: ctx_len a multiple of block_size (blocks are whole); 1 <=
 * block_size <= 4096; 1 <= n_blk <= ctx_len/block_size.  A host pointer that
 * is not pinned, device-accessible memory gives SA_ERR_MEMORY. */
sa_status sa_gather_blocks(const sa_kv_desc* desc, const void* k_host, const void* v_host,
                           const int32_t* idx, int32_t n_blk, int32_t block_size, void* k_out,
                           void* v_out, hipStream_t stream);

/* ----------------------------------------------------------------- misc */

/* Zero a device region on `stream` with a fill kernel (safe inside stream
 * capture).  Workspaces need no initialisation; this is a utility. */
sa_status sa_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* sa_status_string(sa_status s);

/* Detail of the last failing call on the calling thread ("" if none). */
const char* sa_last_error(void);

/* Library version string. */
const char* sa_version(void);

/* ------------------------------------------------------------ measurement */

/* Not a step of the method: a plain streaming read of `bytes` (a positive
 * multiple of 16) of device memory at `data` (16-byte aligned), 16-byte
 * nontemporal loads from 4096 workgroups reading contiguous chunks, folded
 * so they cannot be removed (`sink`, one uint32, is written only if the fold
 * hits a fixed constant).  Its duration gives the HBM read rate this device
 * reaches, the reference the kernels' rates are compared with.
 * Errors: SA_ERR_NULL / SA_ERR_ALIGN for data, sink; SA_ERR_SHAPE for bytes. */
sa_status sa_stream_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream);

/* The reads of sa_sparse_decode without its arithmetic (a measurement
 * reference, not a step of the method): for the same descriptor, index kind
 * and index list, the same launch plan, index loads and key/value row loads
 * as the pair-pipelined gather-attend, in the same order (every key row of a
 * wave's slots before their value rows), folded with XOR into *sink only if
 * the fold hits a fixed constant.  Its duration is how long reading the
 * selected rows alone takes, the floor for that gather-attend launch.
 * Errors: as sa_sparse_decode for desc, k_cache, v_cache and the index
 * arguments; SA_ERR_NULL / SA_ERR_ALIGN for sink; SA_ERR_UNSUPPORTED when
 * sa_sparse_decode would not take the pair-pipelined kernel (fp32, head_dim
 * 64, more than 4 query heads per KV head, partial last blocks). */
sa_status sa_gather_read(const sa_kv_desc* desc, const void* k_cache, const void* v_cache,
                         sa_index_kind ik, const int32_t* idx, int32_t n_idx, int32_t block_size,
                         uint32_t* sink, hipStream_t stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
