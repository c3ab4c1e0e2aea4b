"""CPU oracle for top-k sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The product path never calls it and shares no code with it.

Plain, slow, obviously correct: numpy in float64, one (sequence, KV head) row
at a time, each function written from the definition it cites.  Library
primitives (a matrix-vector product, ``exp``, a stable sort) serve as single
steps; there is no tiling, fusion or reordering beyond what a definition says.

Sources (the pages this method is described on):
  [P1] "Flux Attention: Context-Aware Hybrid Attention for Efficient LLMs
       Inference", paper review (blog.secrett2633.cloud)
  [P2] "HyLRA: Hybrid Layer Reuse Attention for efficient long-context
       inference", technical summary (gist.science, 2602.00777)
  [P3] "Inference-time context sparsity: illusion or opportunity?",
       technical summary (gist.science, 2605.24168)
  [P5] "Flash Attention vs Sparse Attention" (sotaaz.com)

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):
  * attention and exact scores use the scale 1/sqrt(d);
  * query head h belongs to KV head h // G (contiguous groups of G);
  * a per-(sequence, KV head) selection scores a token by the SUM over the G
    grouped queries of their logits;
  * ties in a top-k go to the lower index, -0.0 equals +0.0, NaN ranks below
    every number; the selected indices are returned in ascending order;
  * block scores carry no 1/sqrt(d) and are summed over the group;
  * the decode query attends to all N cached tokens (no mask inside the cache).

Values come in as numpy arrays of stored bits (``uint16`` bf16 patterns or
``float32``); ``widen`` turns them into float64 exactly.
"""
from __future__ import annotations

import math

import numpy as np

DENSE, SPARSE, REUSE, DENSE_SELECT = 0, 1, 2, 3


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------

def widen(x: np.ndarray, dtype: str | None = None) -> np.ndarray:
    """Stored values -> float64, exactly.

    ``uint16`` arrays hold bf16 bit patterns: the bf16 value is the float32
    whose upper 16 bits are the pattern and whose lower 16 bits are zero.
    """
    x = np.asarray(x)
    if dtype == "bf16" or x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def default_scale(head_dim: int) -> float:
    """Softmax temperature 1/sqrt(d) (reading: the pages state no formula)."""
    return 1.0 / math.sqrt(head_dim)


# ---------------------------------------------------------------------------
# Step 1: score every cached token
# ---------------------------------------------------------------------------

def scores_exact(q_group: np.ndarray, k_row: np.ndarray, scale: float) -> np.ndarray:
    """Exact ("oracle") token scores of one (sequence, KV head) row.

    [P3] section 2, sparsity mechanisms: the oracle top-k picks the k tokens
    with the highest true query-key score.  With G query heads sharing one KV
    head, a token's row score is the sum of its G logits:
        s_t = sum_g  (q_g . K_t) * scale.
    q_group: [G, d] float64; k_row: [N, d] float64 -> [N] float64.
    """
    s = np.zeros(k_row.shape[0], dtype=np.float64)
    for g in range(q_group.shape[0]):
        s += (k_row @ q_group[g]) * scale
    return s


def scores_per_query_head(q_head: np.ndarray, k_row: np.ndarray, scale: float) -> np.ndarray:
    """Exact token scores of ONE query head, for selection that differs
    between the query heads of a group.

    [P3] section 2 (hardware implementation): the sparse decode kernel takes
    irregular sparsity per token, per query and per head.  Query head h scores
    the keys of its KV head on its own:  s_t = (q_h . K_t) * scale.
    q_head: [d]; k_row: [N, d] -> [N] float64.
    """
    return (k_row @ q_head) * scale


def block_summaries(k_row: np.ndarray, block_size: int):
    """Elementwise min and max of the keys of each fixed-size token block.

    [P2] section 2.4: selection runs on fixed blocks of tokens (for example
    128) so that memory access is regular; a block is summarised by the
    per-dimension minimum and maximum of its keys (the QUEST-compatible form).
    The last block covers only the tokens that exist.
    k_row: [N, d] -> (kmin, kmax) each [ceil(N / block_size), d].
    """
    n, d = k_row.shape
    nb = (n + block_size - 1) // block_size
    kmin = np.empty((nb, d), dtype=np.float64)
    kmax = np.empty((nb, d), dtype=np.float64)
    for j in range(nb):
        blk = k_row[j * block_size:min(n, (j + 1) * block_size)]
        kmin[j] = blk.min(axis=0)
        kmax[j] = blk.max(axis=0)
    return kmin, kmax


def scores_block(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> np.ndarray:
    """Upper-bound score of each block, summed over the query group.

    For one query q and block summary (kmin, kmax):
        sb_j = sum_i max(q_i * kmin_ji, q_i * kmax_ji),
    which is >= q . k for every key k inside block j.  Summed over the G
    grouped queries, with no 1/sqrt(d) (rank-invariant).  [P2] section 2.4.
    """
    nb = kmin.shape[0]
    sb = np.zeros(nb, dtype=np.float64)
    for g in range(q_group.shape[0]):
        q = q_group[g]
        sb += np.maximum(kmin * q, kmax * q).sum(axis=1)
    return sb


def scores_indexer(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Lightning-indexer token scores of one sequence.

    [P5] section "DeepSeek Sparse Attention (DSA)", Stage 1: a cheap scan
    scores every token and keeps a top-K index list.  Score form (the pages
    give none; this is the stated workload's form):
        si_t = sum_h w_h * max(0, q_idx_h . k_idx_t).
    q_idx: [H, Di], k_idx: [N, Di], w: [H] -> [N].
    """
    si = np.zeros(k_idx.shape[0], dtype=np.float64)
    for h in range(q_idx.shape[0]):
        si += float(w[h]) * np.maximum(0.0, k_idx @ q_idx[h])
    return si


# ---------------------------------------------------------------------------
# Step 2: select the top-k
# ---------------------------------------------------------------------------

def topk(s: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring positions, ascending.

    [P3] section 2 (oracle top-k) and [P5] DSA Stage 1 (a top-K index list).
    Order positions by (score descending, index ascending) and keep the first
    k; -0.0 is the same score as +0.0; NaN sorts after every number.
    """
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n (k=%d, n=%d)" % (k, n))
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s) + 0.0          # + 0.0 maps -0.0 to +0.0
    order = np.lexsort((np.arange(n), neg, nan))  # last key is primary
    return np.sort(order[:k]).astype(np.int32)


def block_tokens(blocks: np.ndarray, block_size: int, n: int) -> np.ndarray:
    """Token positions covered by a set of block ids (ascending, < n)."""
    toks = [np.arange(j * block_size, min(n, (j + 1) * block_size)) for j in np.sort(blocks)]
    return np.concatenate(toks).astype(np.int64) if toks else np.zeros(0, dtype=np.int64)


# ---------------------------------------------------------------------------
# Steps 3-4: attend over the selected set (and the dense special case)
# ---------------------------------------------------------------------------

def attend_lse(q_group: np.ndarray, k_row: np.ndarray, v_row: np.ndarray, sel, scale: float):
    """Softmax attention of each query head restricted to the selected tokens.

    [P5] DSA Stage 2: full attention computed only over the tokens Stage 1
    selected; [P3] section 3.C: decoding then reads O(k*d) of the cache.
    For each query head g, over t in S (ascending):
        l_t = (q_g . K_t) * scale,  m = max l,  w_t = exp(l_t - m),
        o_g = sum_t w_t V_t / sum_t w_t.
    Returns (o [G, d], lse [G]) with lse = m + log(sum_t w_t).
    """
    sel = np.sort(np.asarray(sel, dtype=np.int64))
    ks = k_row[sel]
    vs = v_row[sel]
    g_heads = q_group.shape[0]
    out = np.empty((g_heads, v_row.shape[1]), dtype=np.float64)
    lse = np.empty(g_heads, dtype=np.float64)
    for g in range(g_heads):
        logits = (ks @ q_group[g]) * scale
        m = logits.max()
        w = np.exp(logits - m)
        den = w.sum()
        out[g] = (w @ vs) / den
        lse[g] = m + math.log(den)
    return out, lse


def attend(q_group, k_row, v_row, sel, scale):
    """Selected-set attention output [G, d] (see ``attend_lse``)."""
    return attend_lse(q_group, k_row, v_row, sel, scale)[0]


def dense(q_group, k_row, v_row, scale):
    """Full decode attention over all N cached tokens.

    [P5] section on the O(n^2) wall: standard attention relates the query to
    every token; at decode time that is one softmax over all N keys.
    """
    return attend(q_group, k_row, v_row, np.arange(k_row.shape[0]), scale)


def attend_bytes(n_selected: int, head_dim: int, elt_bytes: int) -> int:
    """Cache bytes one row's selected-set attention reads: K and V rows of S.

    [P3] section 3.C: traffic O(k*d) instead of O(N*d) -- the count depends on
    |S| and d only, not on the context length.
    """
    return 2 * int(n_selected) * int(head_dim) * int(elt_bytes)


# ---------------------------------------------------------------------------
# Per-layer mode and index reuse
# ---------------------------------------------------------------------------

def plan_check(modes, src):
    """Validate a per-layer plan; returns None if valid, else a reason.

    [P1] key terms: a per-layer hard decision between full and sparse
    attention.  [P2] sections 2.2-2.3 and [P5] "IndexCache": a tolerant layer
    reuses the top-k indices of an earlier layer unchanged.  A REUSE layer
    names a source layer that comes before it and that owns an index set
    (a SPARSE layer, a DENSE_SELECT layer -- full attention that hands its
    top-k on, [P2] section 2.3 -- or a REUSE layer, which carries its
    source's set).
    """
    if len(modes) != len(src):
        return "modes and src differ in length"
    has_idx = []
    for l, m in enumerate(modes):
        if m not in (DENSE, SPARSE, REUSE, DENSE_SELECT):
            return "layer %d: unknown mode %r" % (l, m)
        if m == REUSE:
            s = src[l]
            if not 0 <= s < l:
                return "layer %d: reuse source %d is not an earlier layer" % (l, s)
            if not has_idx[s]:
                return "layer %d: reuse source %d holds no index set" % (l, s)
        has_idx.append(m != DENSE)
    return None


def run_plan(modes, src, k, score_fn, attend_fn, dense_fn):
    """Run a layer plan.

    For layer l: DENSE -> dense_fn(l), no index set; SPARSE -> idx =
    topk(score_fn(l), k), attend_fn(l, idx); DENSE_SELECT -> dense_fn(l) and
    idx = topk(score_fn(l), k); REUSE -> idx = index set of layer src[l] (the
    same array), attend_fn(l, idx).  Returns (outputs, index sets).
    """
    why = plan_check(modes, src)
    if why is not None:
        raise ValueError(why)
    outs, idxs = [], []
    for l, m in enumerate(modes):
        if m == DENSE:
            outs.append(dense_fn(l))
            idxs.append(None)
        elif m == DENSE_SELECT:
            outs.append(dense_fn(l))
            idxs.append(topk(score_fn(l), k))
        elif m == SPARSE:
            idx = topk(score_fn(l), k)
            outs.append(attend_fn(l, idx))
            idxs.append(idx)
        else:
            idx = idxs[src[l]]
            outs.append(attend_fn(l, idx))
            idxs.append(idx)
    return outs, idxs


# ---------------------------------------------------------------------------
# Layer-reuse policy ([P2] section 2.2)
# ---------------------------------------------------------------------------

def index_overlap(a, b) -> int:
    """Number of token indices two top-k sets share ([P2] section 2.2: the
    similarity matrix holds the overlap of a source and a target layer's
    top-k indices)."""
    return int(np.intersect1d(np.asarray(a), np.asarray(b)).shape[0])


def reuse_plan_feasible(full, overlap, total, theta, sensitive):
    """Whether a set of full-attention layers gives a valid policy.

    [P2] section 2.2: a full layer j is the state (j, j) (a "reset jump");
    every other layer t stays on the column of the last full layer i before it
    (a "vertical move" into (i, t)), which is allowed only when the overlap
    ratio of layers i and t exceeds theta.  Layer 0 has no earlier set, so it
    is full; a sensitive layer ([P2] section 2.1) is full too.
    """
    n = len(overlap)
    if 0 not in full:
        return False
    last = None
    for t in range(n):
        if t in full:
            last = t
            continue
        if sensitive is not None and sensitive[t]:
            return False
        if not float(overlap[last][t]) / float(total) > theta:
            return False
    return True


def reuse_plan_bruteforce(overlap, total, theta, sensitive=None):
    """The optimal policy of [P2] section 2.2 by exhaustive search.

    Every set of full layers is tried (2^(L-1) of them).  Objective, in this
    order: fewest full layers (full attention is the cost the policy
    minimises), then the largest summed overlap over the reused layers
    (maximise cumulative similarity), then -- a tie rule of this
    implementation -- the lexicographically largest sorted list of full layers.
    Returns (modes, src): a full layer is DENSE_SELECT when a later layer
    reuses its set and DENSE otherwise; a reused layer is REUSE with src = its
    full layer; src = -1 for full layers.
    """
    n = len(overlap)
    best = None
    for mask in range(1 << (n - 1)):
        full = [0] + [t for t in range(1, n) if mask >> (t - 1) & 1]
        fs = set(full)
        if not reuse_plan_feasible(fs, overlap, total, theta, sensitive):
            continue
        sim, last = 0, 0
        for t in range(n):
            if t in fs:
                last = t
            else:
                sim += int(overlap[last][t])
        key = (len(full), -sim, [-x for x in full])
        if best is None or key < best[0]:
            best = (key, full)
    full = best[1]
    return _plan_from_full(full, n)


def _plan_from_full(full, n):
    fs = set(full)
    modes, src = [], []
    last = -1
    for t in range(n):
        if t in fs:
            last = t
            reused = t + 1 < n and (t + 1) not in fs
            modes.append(DENSE_SELECT if reused else DENSE)
            src.append(-1)
        else:
            modes.append(REUSE)
            src.append(last)
    return modes, src


def fixed_jump_plan(n_layers: int, step: int):
    """The static baseline of [P2] section 4: full attention at layers 0,
    step, 2*step, ...; every other layer reuses the full layer before it."""
    return _plan_from_full(list(range(0, n_layers, step)), n_layers)


# ---------------------------------------------------------------------------
# Acceptance rule for a selected index set
# ---------------------------------------------------------------------------

def index_set_verdict(s: np.ndarray, got, k: int, rel: float = 1e-4):
    """Classify a selected set against the fp64 scores of its row.

    Let s_(1) >= s_(2) >= ... be the sorted scores and tau = rel * max(|s_(k)|,
    |s_(k+1)|, 1e-30).  If s_(k) - s_(k+1) > tau the set must equal the exact
    top-k.  Otherwise (a near tie) it must hold k distinct in-range indices,
    contain every t with s_t > s_(k) + tau and lie inside {t : s_t >=
    s_(k+1) - tau}.  Returns "exact" (equal to the exact top-k), "excused"
    (a different set inside a near-tie band) or "failed: <reason>".
    """
    s = np.asarray(s, dtype=np.float64)
    got = np.asarray(got, dtype=np.int64)
    n = s.shape[0]
    if got.shape != (k,):
        return "failed: expected %d indices, got shape %s" % (k, got.shape)
    if got.min() < 0 or got.max() >= n:
        return "failed: index out of range"
    if np.unique(got).shape[0] != k:
        return "failed: repeated index"
    want = topk(s, k)
    if np.array_equal(np.sort(got), want):
        return "exact"
    if k == n:
        return "failed: k == n but set differs"
    srt = np.sort(s)[::-1]
    sk, sk1 = srt[k - 1], srt[k]
    tau = rel * max(abs(sk), abs(sk1), 1e-30)
    if sk - sk1 > tau:
        return "failed: separated row but set differs in %d positions" % (
            k - np.intersect1d(got, want).shape[0])
    must = np.nonzero(s > sk + tau)[0]
    allowed = s >= sk1 - tau
    if not np.all(np.isin(must, got)):
        return "failed: near-tie row misses a clearly-above index"
    if not np.all(allowed[got]):
        return "failed: near-tie row holds a clearly-below index"
    return "excused"


# ---------------------------------------------------------------------------
# Cost model (arithmetic the pages state; not part of the path)
# ---------------------------------------------------------------------------

def score_matrix_bytes(n_tokens: int, bytes_per_score: int) -> int:
    """Size of one head's n x n attention-score matrix ([P5], the O(n^2) wall)."""
    return int(n_tokens) * int(n_tokens) * int(bytes_per_score)


def dsa_cost(context: int, indexer_ops: int, selected: int):
    """[P5] DSA example: (indexer + selected) operations against a full pass
    over the context, and the fraction saved."""
    total = indexer_ops + selected
    return total, 1.0 - total / context
