"""ctypes binding of ``libsa.so`` (declared in ``include/sa.h``).

Argument marshalling only: every function below validates tensor placement,
builds the C descriptor from torch tensor shapes/strides, passes
``tensor.data_ptr()`` and the current HIP stream, and raises ``RuntimeError``
with the library's message on a non-OK status.  All computation happens in the
HIP kernels of the library; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIBRARY names another build of the same library to load instead (the
# host-sanitized one: build.build_sanitized()).
LIB_PATH = os.environ.get("SA_LIBRARY") or os.path.join(_HERE, "libsa.so")

# sa_status
SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_ALIGN, SA_ERR_DTYPE, SA_ERR_WORKSPACE, \
    SA_ERR_UNSUPPORTED, SA_ERR_HIP, SA_ERR_MEMORY = range(9)
# sa_dtype
SA_F32, SA_BF16 = 0, 1
# sa_score_kind
SA_SCORE_EXACT, SA_SCORE_BLOCK_MINMAX, SA_SCORE_INDEXER, SA_SCORE_INDEXER_PER_KV_HEAD = 0, 1, 2, 3
SA_SCORE_EXACT_PER_Q_HEAD = 4
# sa_index_kind
SA_IDX_TOKEN_PER_KV_HEAD, SA_IDX_TOKEN_SHARED, SA_IDX_BLOCK_PER_KV_HEAD = 0, 1, 2
SA_IDX_TOKEN_PER_Q_HEAD = 3
# sa_layer_mode
SA_LAYER_DENSE, SA_LAYER_SPARSE, SA_LAYER_REUSE, SA_LAYER_DENSE_SELECT = 0, 1, 2, 3

EXPORTED = [
    "sa_score", "sa_block_summarize", "sa_topk", "sa_topk_workspace_size", "sa_select",
    "sa_select_workspace_size", "sa_sparse_decode", "sa_sparse_decode_noalloc",
    "sa_check_indices",
    "sa_sparse_workspace_size", "sa_dense_decode", "sa_dense_workspace_size",
    "sa_dense_decode_scored", "sa_dense_scored_workspace_size", "sa_decode_layer",
    "sa_layer_workspace_size", "sa_plan_validate", "sa_index_overlap", "sa_plan_reuse",
    "sa_plan_fixed_jump", "sa_gather_blocks", "sa_workspace_init", "sa_stream_read", "sa_gather_read",
    "sa_status_string", "sa_last_error", "sa_version",
]


class KVDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ctx_len", ctypes.c_int64), ("q_dtype", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("kv_stride_b", ctypes.c_int64),
                ("kv_stride_h", ctypes.c_int64), ("kv_stride_t", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float)]


class ScoreAux(ctypes.Structure):
    _fields_ = [("kmin", ctypes.c_void_p), ("kmax", ctypes.c_void_p),
                ("block_size", ctypes.c_int32), ("q_idx", ctypes.c_void_p),
                ("k_idx", ctypes.c_void_p), ("idx_w", ctypes.c_void_p),
                ("n_idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("desc", KVDesc), ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("score_kind", ctypes.c_int),
                ("aux", ScoreAux), ("k", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libsa.so is not built (expected at %s); run `python -m top_sparse_decode_sa_amd.build`"
            % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    P = ctypes.POINTER
    L.sa_score.argtypes = [P(KVDesc), st, vp, vp, P(ScoreAux), vp, vp]
    L.sa_block_summarize.argtypes = [P(KVDesc), i32, vp, vp, vp, vp]
    L.sa_topk.argtypes = [vp, i64, i64, i64, i32, vp, vp, sz, vp]
    L.sa_topk_workspace_size.argtypes = [i64, i64, i32]
    L.sa_topk_workspace_size.restype = sz
    L.sa_select.argtypes = [P(KVDesc), st, vp, vp, P(ScoreAux), i32, vp, vp, sz, vp]
    L.sa_select_workspace_size.argtypes = [P(KVDesc), st, i32]
    L.sa_select_workspace_size.restype = sz
    L.sa_stream_read.argtypes = [vp, sz, vp, vp]
    L.sa_gather_read.argtypes = [P(KVDesc), vp, vp, st, vp, i32, i32, vp, vp]
    L.sa_sparse_decode.argtypes = [P(KVDesc), vp, vp, vp, st, vp, i32, i32, vp, vp, sz, vp]
    L.sa_sparse_decode_noalloc.argtypes = [P(KVDesc), vp, vp, vp, st, vp, i32, i32, vp, vp]
    L.sa_check_indices.argtypes = [P(KVDesc), st, vp, i32, i32, vp, vp]
    L.sa_sparse_workspace_size.argtypes = [P(KVDesc), st, i32, i32]
    L.sa_sparse_workspace_size.restype = sz
    L.sa_dense_decode.argtypes = [P(KVDesc), vp, vp, vp, vp, vp, sz, vp]
    L.sa_dense_workspace_size.argtypes = [P(KVDesc)]
    L.sa_dense_workspace_size.restype = sz
    L.sa_dense_decode_scored.argtypes = [P(KVDesc), vp, vp, vp, vp, vp, vp, sz, vp]
    L.sa_dense_scored_workspace_size.argtypes = [P(KVDesc)]
    L.sa_dense_scored_workspace_size.restype = sz
    L.sa_index_overlap.argtypes = [vp, vp, i64, i32, vp, vp]
    L.sa_plan_reuse.argtypes = [vp, i64, i32, ctypes.c_double, vp, vp, vp]
    L.sa_plan_fixed_jump.argtypes = [i32, i32, vp, vp]
    L.sa_gather_blocks.argtypes = [P(KVDesc), vp, vp, vp, i32, i32, vp, vp, vp]
    L.sa_decode_layer.argtypes = [P(LayerArgs), st, vp, vp]
    L.sa_layer_workspace_size.argtypes = [P(LayerArgs), st]
    L.sa_layer_workspace_size.restype = sz
    L.sa_plan_validate.argtypes = [vp, vp, i32]
    L.sa_workspace_init.argtypes = [vp, sz, vp]
    L.sa_status_string.argtypes = [st]
    L.sa_status_string.restype = ctypes.c_char_p
    L.sa_last_error.argtypes = []
    L.sa_last_error.restype = ctypes.c_char_p
    L.sa_version.restype = ctypes.c_char_p
    for name in ["sa_score", "sa_block_summarize", "sa_topk", "sa_select", "sa_sparse_decode",
                 "sa_sparse_decode_noalloc", "sa_check_indices",
                 "sa_dense_decode",
                 "sa_dense_decode_scored", "sa_decode_layer", "sa_plan_validate",
                 "sa_index_overlap", "sa_plan_reuse", "sa_plan_fixed_jump", "sa_gather_blocks",
                 "sa_workspace_init", "sa_stream_read", "sa_gather_read"]:
        getattr(L, name).restype = st
    _lib = L
    return L


class SAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__("%s (%s)" % (lib().sa_status_string(status).decode(), detail))


def check(status: int):
    if status != SA_OK:
        raise SAError(status, lib().sa_last_error().decode())


# ---------------------------------------------------------------- helpers

_DT = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError("dtype %s not supported (float32 or bfloat16)" % t.dtype)
    return _DT[t.dtype]


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU device (got %s)" % t.device)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors on different devices: %s vs %s" % (dev, t.device))
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_desc(q: torch.Tensor, k_cache: torch.Tensor, softmax_scale: float = 0.0) -> KVDesc:
    """Descriptor from q [B, Hq, d] (contiguous) and a K cache [B, Hkv, N, d]."""
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the cache [B, Hkv, N, d]")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if k_cache.stride(3) != 1:
        raise ValueError("the cache's last dimension must be contiguous")
    B, Hkv, N, d = k_cache.shape
    if q.shape[0] != B or q.shape[2] != d:
        raise ValueError("q shape %s does not match cache shape %s" % (tuple(q.shape), tuple(k_cache.shape)))
    return KVDesc(B, q.shape[1], Hkv, d, N, _dtype(q), _dtype(k_cache), k_cache.stride(0),
                  k_cache.stride(1), k_cache.stride(2), float(softmax_scale))


class Workspaces:
    """Zero-initialised device workspaces, one per (device, call signature).

    A workspace is tied to the call kind and shapes it was sized for (see the
    workspace contract in sa.h), so each signature gets its own buffer.
    """

    def __init__(self):
        self._bufs = {}

    def get(self, dev, key, nbytes: int) -> torch.Tensor | None:
        if nbytes == 0:
            return None
        k = (str(dev), key)
        buf = self._bufs.get(k)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device=dev)
            off = (-buf.data_ptr()) % 256
            buf = buf[off:off + nbytes]
            self._bufs[k] = buf
        return buf

    def clear(self):
        self._bufs.clear()


WORKSPACES = Workspaces()


def _desc_key(desc: KVDesc):
    return tuple(getattr(desc, f[0]) for f in KVDesc._fields_)


# ---------------------------------------------------------------- C calls

def sa_score(q, k_cache, kind=SA_SCORE_EXACT, *, kmin=None, kmax=None, block_size=0, q_idx=None,
             k_idx=None, idx_w=None, scores=None, softmax_scale=0.0):
    """sa_score: returns fp32 scores ([B, Hkv, N], [B, Hkv, nb] or [B, N])."""
    dev = _dev(q, k_cache, kmin, kmax, q_idx, k_idx, idx_w)
    desc = make_desc(q, k_cache, softmax_scale)
    aux = ScoreAux()
    B, Hkv, N = desc.batch, desc.n_kv_heads, desc.ctx_len
    if kind == SA_SCORE_BLOCK_MINMAX:
        aux.kmin, aux.kmax, aux.block_size = kmin.data_ptr(), kmax.data_ptr(), block_size
        shape = (B, Hkv, (N + block_size - 1) // block_size)
    elif kind in (SA_SCORE_INDEXER, SA_SCORE_INDEXER_PER_KV_HEAD):
        aux.q_idx, aux.k_idx, aux.idx_w = q_idx.data_ptr(), k_idx.data_ptr(), idx_w.data_ptr()
        H, Di = q_idx.shape[-2], q_idx.shape[-1]
        aux.n_idx_heads, aux.idx_dim = H, Di
        lead = (B,) if kind == SA_SCORE_INDEXER else (B, Hkv)
        if (tuple(q_idx.shape) != lead + (H, Di) or tuple(k_idx.shape) != lead + (N, Di)
                or tuple(idx_w.shape) != lead + (H,)):
            raise ValueError("indexer tensors: q_idx %s+[H,Di], k_idx %s+[N,Di], idx_w %s+[H]"
                             % (list(lead), list(lead), list(lead)))
        for t in (q_idx, k_idx, idx_w):
            if not t.is_contiguous():
                raise ValueError("indexer tensors must be contiguous")
        shape = lead + (N,)
    elif kind == SA_SCORE_EXACT_PER_Q_HEAD:
        shape = (B, desc.n_q_heads, N)
    else:
        shape = (B, Hkv, N)
    if scores is None:
        scores = torch.empty(shape, dtype=torch.float32, device=dev)
    check(lib().sa_score(ctypes.byref(desc), kind, _ptr(q), _ptr(k_cache), ctypes.byref(aux),
                         _ptr(scores), ctypes.c_void_p(_stream(dev))))
    return scores


def sa_block_summarize(k_cache, block_size, q_like=None, kmin=None, kmax=None):
    """sa_block_summarize: returns (kmin, kmax) [B, Hkv, nb, d] in the cache dtype
    (written into kmin / kmax when given)."""
    dev = _dev(k_cache, kmin, kmax)
    B, Hkv, N, d = k_cache.shape
    q = q_like if q_like is not None else torch.empty((B, Hkv, d), dtype=k_cache.dtype, device=dev)
    desc = make_desc(q, k_cache)
    nb = (N + block_size - 1) // block_size
    if kmin is None:
        kmin = torch.empty((B, Hkv, nb, d), dtype=k_cache.dtype, device=dev)
    if kmax is None:
        kmax = torch.empty_like(kmin)
    for t in (kmin, kmax):
        if t.shape != (B, Hkv, nb, d) or t.dtype != k_cache.dtype or not t.is_contiguous():
            raise ValueError("kmin / kmax must be contiguous [B, Hkv, nb, d] in the cache dtype")
    check(lib().sa_block_summarize(ctypes.byref(desc), block_size, _ptr(k_cache), _ptr(kmin),
                                   _ptr(kmax), ctypes.c_void_p(_stream(dev))))
    return kmin, kmax


def sa_select(q, k_cache, k, kind=SA_SCORE_EXACT, idx_out=None, softmax_scale=0.0, *, q_idx=None,
              k_idx=None, idx_w=None):
    """sa_select: the top-k positions without the score array; int32
    [B, Hkv, k] (EXACT, INDEXER_PER_KV_HEAD), [B, Hq, k] (EXACT_PER_Q_HEAD)
    or [B, k] (INDEXER).  The indexer kinds take q_idx / k_idx / idx_w as
    sa_score does (q and k_cache give the shapes)."""
    dev = _dev(q, k_cache, q_idx, k_idx, idx_w)
    desc = make_desc(q, k_cache, softmax_scale)
    aux = ScoreAux()
    if kind in (SA_SCORE_INDEXER, SA_SCORE_INDEXER_PER_KV_HEAD):
        aux.q_idx, aux.k_idx, aux.idx_w = q_idx.data_ptr(), k_idx.data_ptr(), idx_w.data_ptr()
        aux.n_idx_heads, aux.idx_dim = q_idx.shape[-2], q_idx.shape[-1]
        for t in (q_idx, k_idx, idx_w):
            if not t.is_contiguous():
                raise ValueError("indexer tensors must be contiguous")
    if kind == SA_SCORE_EXACT_PER_Q_HEAD:
        shape = (desc.batch, desc.n_q_heads, k)
    elif kind == SA_SCORE_INDEXER:
        shape = (desc.batch, k)
    else:
        shape = (desc.batch, desc.n_kv_heads, k)
    if idx_out is None:
        idx_out = torch.empty(shape, dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sa_select_workspace_size(ctypes.byref(desc), kind, k)
    ws = WORKSPACES.get(dev, ("select", kind, k) + _desc_key(desc), nbytes)
    check(L.sa_select(ctypes.byref(desc), kind, _ptr(q), _ptr(k_cache), ctypes.byref(aux), k,
                      _ptr(idx_out), _ptr(ws), nbytes, ctypes.c_void_p(_stream(dev))))
    return idx_out


def sa_stream_read(data, sink):
    """sa_stream_read: a plain streaming read of a device tensor (measurement
    reference, not a step of the method)."""
    dev = _dev(data, sink)
    check(lib().sa_stream_read(_ptr(data), data.numel() * data.element_size(), _ptr(sink),
                               ctypes.c_void_p(_stream(dev))))


def sa_gather_read(q, k_cache, v_cache, idx, sink, index_kind=SA_IDX_TOKEN_PER_KV_HEAD,
                   block_size=0):
    """sa_gather_read: the reads of sa_sparse_decode on the same arguments
    without its arithmetic (measurement reference); q only gives the
    descriptor its head counts."""
    dev = _dev(q, k_cache, v_cache, idx, sink)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    desc = make_desc(q, k_cache)
    check(lib().sa_gather_read(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), index_kind,
                               _ptr(idx), idx.shape[-1], block_size, _ptr(sink),
                               ctypes.c_void_p(_stream(dev))))


def sa_topk(scores, k, idx_out=None):
    """sa_topk over the last dimension of a 2-D (or higher) fp32 tensor."""
    dev = _dev(scores)
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    n = scores.shape[-1]
    rows = scores.numel() // n if n else 0
    if scores.stride(-1) != 1:
        raise ValueError("scores rows must be contiguous")
    flat = scores.reshape(rows, n)
    row_stride = flat.stride(0) if rows > 1 else n
    if idx_out is None:
        idx_out = torch.empty(scores.shape[:-1] + (k,), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.sa_topk_workspace_size(rows, n, k)
    ws = WORKSPACES.get(dev, ("topk", rows, n, k), nbytes)
    check(L.sa_topk(_ptr(flat), rows, n, row_stride, k, _ptr(idx_out), _ptr(ws), nbytes,
                    ctypes.c_void_p(_stream(dev))))
    return idx_out


def sa_sparse_decode(q, k_cache, v_cache, idx, index_kind=SA_IDX_TOKEN_PER_KV_HEAD, block_size=0,
                     out=None, softmax_scale=0.0, ws=None):
    """sa_sparse_decode: returns out [B, Hq, d] fp32."""
    dev = _dev(q, k_cache, v_cache, idx)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("K and V caches must share shape and strides")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    desc = make_desc(q, k_cache, softmax_scale)
    n_idx = idx.shape[-1]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    L = lib()
    nbytes = L.sa_sparse_workspace_size(ctypes.byref(desc), index_kind, n_idx, block_size)
    if ws is None:
        ws = WORKSPACES.get(dev, ("sparse", _desc_key(desc), index_kind, n_idx, block_size), nbytes)
    check(L.sa_sparse_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), index_kind,
                             _ptr(idx), n_idx, block_size, _ptr(out), _ptr(ws), nbytes,
                             ctypes.c_void_p(_stream(dev))))
    return out


def sa_sparse_decode_noalloc(q, k_cache, v_cache, idx, index_kind=SA_IDX_TOKEN_PER_KV_HEAD,
                             block_size=0, out=None, softmax_scale=0.0):
    """sa_sparse_decode_noalloc (no workspace: the library's static scratch).
    `out` must be given for a call that may not allocate; returns out."""
    dev = _dev(q, k_cache, v_cache, idx)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("K and V caches must share shape and strides")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    desc = make_desc(q, k_cache, softmax_scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    check(lib().sa_sparse_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         index_kind, _ptr(idx), idx.shape[-1], block_size,
                                         _ptr(out), ctypes.c_void_p(_stream(dev))))
    return out


def sa_check_indices(q, k_cache, idx, index_kind=SA_IDX_TOKEN_PER_KV_HEAD, block_size=0,
                     counts=None):
    """sa_check_indices: returns counts (int32[2] on the device): rows with an
    out-of-range index, rows with a repeated index."""
    dev = _dev(q, k_cache, idx)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    desc = make_desc(q, k_cache)
    if counts is None:
        counts = torch.empty(2, dtype=torch.int32, device=dev)
    check(lib().sa_check_indices(ctypes.byref(desc), index_kind, _ptr(idx), idx.shape[-1],
                                 block_size, _ptr(counts), ctypes.c_void_p(_stream(dev))))
    return counts


def sa_dense_decode(q, k_cache, v_cache, out=None, softmax_scale=0.0, ws=None):
    """sa_dense_decode: returns out [B, Hq, d] fp32."""
    dev = _dev(q, k_cache, v_cache)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("K and V caches must share shape and strides")
    desc = make_desc(q, k_cache, softmax_scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    L = lib()
    nbytes = L.sa_dense_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = WORKSPACES.get(dev, ("dense", _desc_key(desc)), nbytes)
    check(L.sa_dense_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                            _ptr(ws), nbytes, ctypes.c_void_p(_stream(dev))))
    return out


def sa_dense_decode_scored(q, k_cache, v_cache, out=None, scores=None, softmax_scale=0.0, ws=None):
    """sa_dense_decode_scored: returns (out [B, Hq, d] fp32, scores [B, Hkv, N] fp32)."""
    dev = _dev(q, k_cache, v_cache)
    if v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("K and V caches must share shape and strides")
    desc = make_desc(q, k_cache, softmax_scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if scores is None:
        scores = torch.empty((desc.batch, desc.n_kv_heads, desc.ctx_len), dtype=torch.float32,
                             device=dev)
    L = lib()
    nbytes = L.sa_dense_scored_workspace_size(ctypes.byref(desc))
    if ws is None:
        ws = WORKSPACES.get(dev, ("dense_scored", _desc_key(desc)), nbytes)
    check(L.sa_dense_decode_scored(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(out), _ptr(scores), _ptr(ws), nbytes,
                                   ctypes.c_void_p(_stream(dev))))
    return out, scores


def sa_index_overlap(idx_a, idx_b, counts=None):
    """sa_index_overlap over the last dimension: int32 counts of shape idx_a.shape[:-1]."""
    dev = _dev(idx_a, idx_b)
    for t in (idx_a, idx_b):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("index sets must be contiguous int32 tensors")
    if idx_a.shape != idx_b.shape:
        raise ValueError("index sets differ in shape: %s vs %s" % (tuple(idx_a.shape), tuple(idx_b.shape)))
    k = idx_a.shape[-1]
    rows = idx_a.numel() // k
    if counts is None:
        counts = torch.empty(idx_a.shape[:-1], dtype=torch.int32, device=dev)
    check(lib().sa_index_overlap(_ptr(idx_a), _ptr(idx_b), rows, k, _ptr(counts),
                                 ctypes.c_void_p(_stream(dev))))
    return counts


def sa_gather_blocks(k_host, v_host, idx, block_size, k_out=None, v_out=None):
    """sa_gather_blocks: K/V caches [B, Hkv, N, d] in pinned host memory, idx [B, Hkv, n_blk]
    int32 on the device; returns (k_out, v_out) [B, Hkv, n_blk * block_size, d] on idx's device."""
    for t in (k_host, v_host):
        if t.is_cuda or not t.is_pinned():
            raise ValueError("the host caches must be pinned CPU tensors (pin_memory=True)")
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("host caches must be [B, Hkv, N, d] with a contiguous last dimension")
    if v_host.shape != k_host.shape or v_host.stride() != k_host.stride():
        raise ValueError("K and V caches must share shape and strides")
    dev = _dev(idx)
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor")
    B, Hkv, N, d = k_host.shape
    n_blk = idx.shape[-1]
    if tuple(idx.shape) != (B, Hkv, n_blk):
        raise ValueError("idx must be [B, Hkv, n_blk]")
    dt = _dtype(k_host)
    desc = KVDesc(B, Hkv, Hkv, d, N, dt, dt, k_host.stride(0), k_host.stride(1), k_host.stride(2), 0.0)
    shape = (B, Hkv, n_blk * block_size, d)
    if k_out is None:
        k_out = torch.empty(shape, dtype=k_host.dtype, device=dev)
    if v_out is None:
        v_out = torch.empty(shape, dtype=k_host.dtype, device=dev)
    for t in (k_out, v_out):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("outputs must be contiguous %s" % (shape,))
    check(lib().sa_gather_blocks(ctypes.byref(desc), _ptr(k_host), _ptr(v_host), _ptr(idx), n_blk,
                                 block_size, _ptr(k_out), _ptr(v_out), ctypes.c_void_p(_stream(dev))))
    return k_out, v_out


def _plan_out(n):
    return (ctypes.c_int32 * max(n, 1))(), (ctypes.c_int32 * max(n, 1))()


def sa_plan_reuse(overlap, total: int, theta: float, sensitive=None):
    """sa_plan_reuse on a host [L, L] int64 overlap matrix; returns (modes, src) lists."""
    import numpy as np
    ov = np.ascontiguousarray(np.asarray(overlap, dtype=np.int64))
    n = ov.shape[0]
    if ov.shape != (n, n):
        raise ValueError("overlap must be a square matrix")
    sens = None
    if sensitive is not None:
        sens = (ctypes.c_int32 * max(n, 1))(*[int(bool(x)) for x in sensitive])
    modes, src = _plan_out(n)
    check(lib().sa_plan_reuse(ctypes.c_void_p(ov.ctypes.data), int(total), n, float(theta), sens,
                              modes, src))
    return list(modes)[:n], list(src)[:n]


def sa_plan_fixed_jump(n_layers: int, step: int):
    """sa_plan_fixed_jump; returns (modes, src) lists."""
    modes, src = _plan_out(n_layers)
    check(lib().sa_plan_fixed_jump(n_layers, step, modes, src))
    return list(modes)[:n_layers], list(src)[:n_layers]


def layer_args(q, k_cache, v_cache, score_kind=SA_SCORE_EXACT, k=0, *, kmin=None, kmax=None,
               block_size=0, q_idx=None, k_idx=None, idx_w=None, out=None, softmax_scale=0.0):
    """Build an sa_layer_args structure (and the output tensor) for sa_decode_layer."""
    dev = _dev(q, k_cache, v_cache, kmin, kmax, q_idx, k_idx, idx_w)
    a = LayerArgs()
    a.desc = make_desc(q, k_cache, softmax_scale)
    a.q, a.k_cache, a.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    a.score_kind = score_kind
    if kmin is not None:
        a.aux.kmin, a.aux.kmax = kmin.data_ptr(), kmax.data_ptr()
    a.aux.block_size = block_size
    if q_idx is not None:
        a.aux.q_idx, a.aux.k_idx, a.aux.idx_w = q_idx.data_ptr(), k_idx.data_ptr(), idx_w.data_ptr()
        a.aux.n_idx_heads, a.aux.idx_dim = q_idx.shape[-2], q_idx.shape[-1]
    a.k = k
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    a.out = out.data_ptr()
    return a, out, dev


def sa_layer_workspace_size(args: LayerArgs, mode: int) -> int:
    return int(lib().sa_layer_workspace_size(ctypes.byref(args), mode))


def sa_decode_layer(args: LayerArgs, mode: int, idx=None, dev=None, ws=None):
    """sa_decode_layer: runs one layer under `mode`; SPARSE writes idx, REUSE reads it."""
    if dev is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    nbytes = sa_layer_workspace_size(args, mode)
    if ws is None:
        key = ("layer", mode, _desc_key(args.desc), args.score_kind, args.k, args.aux.block_size)
        ws = WORKSPACES.get(dev, key, nbytes)
    args.ws = None if ws is None else ws.data_ptr()
    args.ws_bytes = nbytes
    check(lib().sa_decode_layer(ctypes.byref(args), mode, _ptr(idx), ctypes.c_void_p(_stream(dev))))


def sa_plan_validate(modes, src):
    """sa_plan_validate on host lists; raises SAError if the plan is invalid."""
    n = len(modes)
    m = (ctypes.c_int32 * max(n, 1))(*modes)
    s = (ctypes.c_int32 * max(n, 1))(*src)
    check(lib().sa_plan_validate(m, s, n))


def sa_workspace_init(ws):
    dev = _dev(ws)
    check(lib().sa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                  ctypes.c_void_p(_stream(dev))))


def sa_version() -> str:
    return lib().sa_version().decode()
