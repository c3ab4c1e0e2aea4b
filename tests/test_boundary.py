"""The C-ABI library: it loads, exports every call declared in include/sa.h,
and rejects invalid arguments on the host with the documented status code
(before anything could reach a GPU).  Runs without a GPU."""
import ctypes
import os
import re

import pytest

import top_sparse_decode_sa_amd as T
from top_sparse_decode_sa_amd import _binding as Bn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "sa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_call():
    L = T.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), "libsa.so lacks %s" % n
    assert set(names) == set(Bn.EXPORTED)
    assert T.sa_version().startswith("sa ")


def _desc(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, ctx_len=1000, q_dtype=Bn.SA_BF16,
             kv_dtype=Bn.SA_BF16, kv_stride_b=2 * 1000 * 128, kv_stride_h=1000 * 128,
             kv_stride_t=128, softmax_scale=0.0)
    d.update(kw)
    return Bn.KVDesc(**d)


FAKE = ctypes.c_void_p(1 << 20)     # aligned, never dereferenced (calls fail first)
MIS = ctypes.c_void_p((1 << 20) + 4)


def _sparse(desc, q=FAKE, k=FAKE, v=FAKE, ik=0, idx=FAKE, n_idx=10, bs=0, out=FAKE, ws=None,
            nbytes=0):
    return T.lib().sa_sparse_decode(ctypes.byref(desc) if desc is not None else None, q, k, v, ik,
                                    idx, n_idx, bs, out, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), Bn.SA_ERR_UNSUPPORTED),
    (dict(n_q_heads=12, n_kv_heads=4), Bn.SA_ERR_UNSUPPORTED),   # group of 3
    (dict(n_q_heads=9), Bn.SA_ERR_SHAPE),
    (dict(batch=0), Bn.SA_ERR_SHAPE),
    (dict(ctx_len=0), Bn.SA_ERR_SHAPE),
    (dict(ctx_len=1 << 31), Bn.SA_ERR_SHAPE),
    (dict(kv_stride_t=64), Bn.SA_ERR_SHAPE),
    (dict(kv_stride_t=132), Bn.SA_ERR_ALIGN),
    (dict(q_dtype=5), Bn.SA_ERR_DTYPE),
    (dict(softmax_scale=-1.0), Bn.SA_ERR_SHAPE),
    (dict(softmax_scale=float("inf")), Bn.SA_ERR_SHAPE),
])
def test_descriptor_errors(kw, code):
    assert _sparse(_desc(**kw)) == code
    assert T.lib().sa_last_error().decode() != ""


def test_pointer_index_and_workspace_errors():
    L = T.lib()
    d = _desc()
    assert _sparse(None) == Bn.SA_ERR_NULL
    assert _sparse(d, q=None) == Bn.SA_ERR_NULL
    assert _sparse(d, k=MIS) == Bn.SA_ERR_ALIGN
    assert _sparse(d, idx=None) == Bn.SA_ERR_NULL
    assert _sparse(d, n_idx=0) == Bn.SA_ERR_SHAPE
    assert _sparse(d, ik=9) == Bn.SA_ERR_SHAPE
    assert _sparse(d, ik=Bn.SA_IDX_BLOCK_PER_KV_HEAD, bs=0) == Bn.SA_ERR_SHAPE
    # a selection long enough to be split across workgroups needs scratch
    need = L.sa_sparse_workspace_size(ctypes.byref(d), 0, 500, 0)
    assert need > 0 and need % 256 == 0
    assert _sparse(d, n_idx=500, ws=None, nbytes=0) == Bn.SA_ERR_WORKSPACE
    assert _sparse(d, n_idx=500, ws=FAKE, nbytes=need - 1) == Bn.SA_ERR_WORKSPACE
    assert _sparse(d, n_idx=500, ws=ctypes.c_void_p((1 << 20) + 16), nbytes=need) == Bn.SA_ERR_ALIGN
    # a long cache is split over several workgroups per row: it needs a workspace
    dl = _desc(ctx_len=100000, kv_stride_b=2 * 100000 * 128, kv_stride_h=100000 * 128)
    assert L.sa_dense_workspace_size(ctypes.byref(dl)) > 0
    assert L.sa_dense_decode(ctypes.byref(dl), FAKE, FAKE, FAKE, FAKE, None, 0, None) == \
        Bn.SA_ERR_WORKSPACE
    assert L.sa_dense_workspace_size(ctypes.byref(_desc(head_dim=96))) == 0


def test_topk_errors():
    L = T.lib()
    assert L.sa_topk(None, 1, 10, 10, 3, FAKE, None, 0, None) == Bn.SA_ERR_NULL
    assert L.sa_topk(FAKE, 1, 10, 10, 0, FAKE, None, 0, None) == Bn.SA_ERR_SHAPE
    assert L.sa_topk(FAKE, 1, 10, 10, 11, FAKE, None, 0, None) == Bn.SA_ERR_SHAPE
    assert L.sa_topk(FAKE, 0, 10, 10, 3, FAKE, None, 0, None) == Bn.SA_ERR_SHAPE
    assert L.sa_topk(FAKE, 1, 10, 9, 3, FAKE, None, 0, None) == Bn.SA_ERR_SHAPE
    assert L.sa_topk(FAKE, 1 << 22, 10, 10, 3, FAKE, None, 0, None) == Bn.SA_ERR_SHAPE
    assert L.sa_topk_workspace_size(1, 10, 11) == 0


def test_select_errors_and_sizes():
    """sa_select rejects every bad argument before anything is enqueued
    (every pointer here is fake: a call that got as far as a launch would
    return SA_ERR_HIP on this machine)."""
    L = T.lib()
    d = _desc()  # 4 rows of 1000 tokens: two parts of 512, 4096 workspace bytes at k = 64
    E, Q = Bn.SA_SCORE_EXACT, Bn.SA_SCORE_EXACT_PER_Q_HEAD
    mis = ctypes.c_void_p((1 << 20) + 2)
    ws_mis = ctypes.c_void_p((1 << 20) + 16)

    def sel(desc=d, kind=E, q=FAKE, k=FAKE, aux=None, kk=64, idx=FAKE, ws=None, nbytes=0):
        return L.sa_select(ctypes.byref(desc) if desc is not None else None, kind, q, k,
                           ctypes.byref(aux) if aux is not None else None, kk, idx, ws, nbytes,
                           None)

    assert sel(desc=None) == Bn.SA_ERR_NULL
    for kind in (Bn.SA_SCORE_BLOCK_MINMAX, 9):
        assert sel(kind=kind) == Bn.SA_ERR_SHAPE
    # the indexer kinds: aux checked as for sa_score, q and k_cache unused
    IX, IXK = Bn.SA_SCORE_INDEXER, Bn.SA_SCORE_INDEXER_PER_KV_HEAD
    for kind in (IX, IXK):
        assert sel(kind=kind) == Bn.SA_ERR_NULL
        aux = Bn.ScoreAux()
        aux.q_idx = aux.k_idx = 1 << 20
        aux.idx_w = 1 << 20
        aux.n_idx_heads, aux.idx_dim = 17, 64
        assert sel(kind=kind, aux=aux, q=None, k=None) == Bn.SA_ERR_SHAPE
        aux.n_idx_heads, aux.idx_dim = 4, 48
        assert sel(kind=kind, aux=aux, q=None, k=None) == Bn.SA_ERR_UNSUPPORTED
        aux.idx_dim = 64
        assert sel(kind=kind, aux=aux, q=None, k=None, idx=None) == Bn.SA_ERR_NULL
        assert sel(kind=kind, aux=aux, q=None, k=None, kk=1001) == Bn.SA_ERR_SHAPE
        assert sel(kind=kind, aux=aux, q=None, k=None) == Bn.SA_ERR_WORKSPACE
        aux.q_idx = (1 << 20) + 2
        assert sel(kind=kind, aux=aux, q=None, k=None) == Bn.SA_ERR_ALIGN
    # rows: one per sequence (shared indexer) or per (sequence, KV head)
    assert L.sa_select_workspace_size(ctypes.byref(d), IX, 64) == 2 * 2 * 128 * 4
    assert L.sa_select_workspace_size(ctypes.byref(d), IXK, 64) == 2 * 4 * 128 * 4
    assert sel(q=None) == Bn.SA_ERR_NULL
    assert sel(q=mis) == Bn.SA_ERR_ALIGN
    assert sel(k=None) == Bn.SA_ERR_NULL
    assert sel(k=mis) == Bn.SA_ERR_ALIGN
    assert sel(idx=None) == Bn.SA_ERR_NULL
    assert sel(kk=0) == Bn.SA_ERR_SHAPE
    assert sel(kk=1001) == Bn.SA_ERR_SHAPE
    need = L.sa_select_workspace_size(ctypes.byref(d), E, 64)
    assert need == 2 * 4 * 128 * 4
    assert sel() == Bn.SA_ERR_WORKSPACE
    assert sel(ws=ws_mis, nbytes=need) == Bn.SA_ERR_ALIGN
    assert sel(ws=FAKE, nbytes=need - 1) == Bn.SA_ERR_WORKSPACE
    big = _desc(batch=4096, n_q_heads=32, n_kv_heads=8, kv_stride_b=8 * 1000 * 128)
    assert sel(desc=big, kind=Q) == Bn.SA_ERR_SHAPE  # batch * n_q_heads > 65535
    # sizes: 0 for an invalid request
    assert L.sa_select_workspace_size(ctypes.byref(d), Bn.SA_SCORE_BLOCK_MINMAX, 64) == 0
    assert L.sa_select_workspace_size(ctypes.byref(d), E, 0) == 0
    assert L.sa_select_workspace_size(ctypes.byref(d), E, 1001) == 0
    # llama-shaped rows (128 rows of 32768): four 8192-token parts, k = 655:
    # 2620 candidates per row, a score and a position each
    ll = _desc(batch=16, n_q_heads=32, n_kv_heads=8, ctx_len=32768, kv_stride_b=8 * 32768 * 128,
               kv_stride_h=32768 * 128)
    assert L.sa_select_workspace_size(ctypes.byref(ll), E, 655) == 2 * 128 * 2620 * 4
    # candidates more than a quarter of the row: scores plus a register top-k
    assert L.sa_select_workspace_size(ctypes.byref(ll), E, 12000) == 128 * 32768 * 4
    # one part per row (512 rows of 4096): the index list is written directly
    one = _desc(batch=64, n_q_heads=8, n_kv_heads=8, ctx_len=4096, kv_stride_b=8 * 4096 * 128,
                kv_stride_h=4096 * 128)
    assert L.sa_select_workspace_size(ctypes.byref(one), E, 100) == 0
    assert sel(desc=one, kk=100, idx=None) == Bn.SA_ERR_NULL


def test_stream_read_errors():
    L = T.lib()
    sink = FAKE
    assert L.sa_stream_read(None, 4096, sink, None) == Bn.SA_ERR_NULL
    assert L.sa_stream_read(ctypes.c_void_p((1 << 20) + 8), 4096, sink, None) == Bn.SA_ERR_ALIGN
    assert L.sa_stream_read(FAKE, 4096, None, None) == Bn.SA_ERR_NULL
    assert L.sa_stream_read(FAKE, 0, sink, None) == Bn.SA_ERR_SHAPE
    assert L.sa_stream_read(FAKE, 4100, sink, None) == Bn.SA_ERR_SHAPE


def test_score_and_summary_errors():
    L = T.lib()
    d = _desc()
    aux = Bn.ScoreAux()
    assert L.sa_score(ctypes.byref(d), 7, FAKE, FAKE, None, FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_score(ctypes.byref(d), 0, FAKE, FAKE, None, None, None) == Bn.SA_ERR_NULL
    assert L.sa_score(ctypes.byref(d), 1, FAKE, FAKE, None, FAKE, None) == Bn.SA_ERR_NULL
    aux.block_size = 0
    assert L.sa_score(ctypes.byref(d), 1, FAKE, FAKE, ctypes.byref(aux), FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_score(ctypes.byref(d), Bn.SA_SCORE_INDEXER_PER_KV_HEAD, FAKE, FAKE, None, FAKE,
                      None) == Bn.SA_ERR_NULL
    aux.n_idx_heads, aux.idx_dim = 17, 64
    assert L.sa_score(ctypes.byref(d), 2, FAKE, FAKE, ctypes.byref(aux), FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_score(ctypes.byref(d), 3, FAKE, FAKE, ctypes.byref(aux), FAKE, None) == Bn.SA_ERR_SHAPE
    aux.n_idx_heads, aux.idx_dim = 4, 48
    assert L.sa_score(ctypes.byref(d), 2, FAKE, FAKE, ctypes.byref(aux), FAKE, None) == \
        Bn.SA_ERR_UNSUPPORTED
    assert L.sa_block_summarize(ctypes.byref(d), 0, FAKE, FAKE, FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_block_summarize(ctypes.byref(d), 128, FAKE, MIS, FAKE, None) == Bn.SA_ERR_ALIGN


def test_layer_errors_and_sizes():
    L = T.lib()
    a = Bn.LayerArgs()
    a.desc = _desc()
    a.q = a.k_cache = a.v_cache = a.out = 1 << 20
    a.score_kind = Bn.SA_SCORE_EXACT
    a.k = 0
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_SPARSE, FAKE, None) == Bn.SA_ERR_SHAPE
    a.k = 1001
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_SPARSE, FAKE, None) == Bn.SA_ERR_SHAPE
    a.k = 64
    assert L.sa_decode_layer(ctypes.byref(a), 5, FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_SPARSE, None, None) == Bn.SA_ERR_NULL
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_SPARSE, FAKE, None) == Bn.SA_ERR_WORKSPACE
    s_sparse = L.sa_layer_workspace_size(ctypes.byref(a), Bn.SA_LAYER_SPARSE)
    s_reuse = L.sa_layer_workspace_size(ctypes.byref(a), Bn.SA_LAYER_REUSE)
    # SPARSE holds the exact selection's workspace on top of what REUSE needs
    s_select = L.sa_select_workspace_size(ctypes.byref(a.desc), Bn.SA_SCORE_EXACT, 64)
    assert s_select > 0 and s_sparse == s_reuse + s_select
    a.score_kind = Bn.SA_SCORE_BLOCK_MINMAX
    a.aux.block_size = 128
    a.k = 9   # 8 blocks of 128 cover 1000 tokens
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_REUSE, FAKE, None) == Bn.SA_ERR_NULL  # kmin
    assert L.sa_layer_workspace_size(None, 0) == 0


def test_plan_validate():
    T.sa_plan_validate([1, 2, 2, 2], [-1, 0, 0, 0])
    T.sa_plan_validate([0, 0, 1, 1, 1, 1, 1, 1], [-1] * 8)
    T.sa_plan_validate([1, 2, 0, 2], [-1, 0, -1, 1])
    for modes, src in [([2], [0]), ([1, 2], [-1, 1]), ([0, 2], [-1, 0]), ([1, 7], [-1, -1]),
                       ([1, 2], [-1, -5])]:
        with pytest.raises(T.SAError):
            T.sa_plan_validate(modes, src)
    assert T.lib().sa_plan_validate(None, None, 3) == Bn.SA_ERR_NULL
    assert T.lib().sa_plan_validate(FAKE, FAKE, 0) == Bn.SA_ERR_SHAPE


def test_status_strings():
    for s in range(8):
        assert T.lib().sa_status_string(s).decode().startswith("SA_")


# ---------------------------------------------------------------------------
# layer-reuse planner (host-only calls): the C dynamic programme against the
# oracle's exhaustive search, bit-exact, plus its error paths
# ---------------------------------------------------------------------------

def test_plan_reuse_matches_exhaustive_search():
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(11)
    cases = 0
    for n in range(1, 10):
        for trial in range(40):
            total = int(rng.integers(1, 1000))
            m = np.triu(rng.integers(0, total + 1, (n, n)), 1).astype(np.int64)
            if trial % 4 == 0:       # coarse values: many exact ties
                m = np.triu(rng.integers(0, 3, (n, n)) * (total // 2), 1).astype(np.int64)
            theta = float(rng.choice([-0.1, 0.0, 0.3, 0.5, 0.7, 0.95, 1.0]))
            sens = (rng.random(n) < 0.2).astype(int).tolist() if trial % 3 == 0 else None
            want = O.reuse_plan_bruteforce(m, total, theta, sens)
            got = T.sa_plan_reuse(m, total, theta, sens)
            assert got == (list(want[0]), list(want[1])), (n, trial, theta)
            T.sa_plan_validate(*got)
            cases += 1
    assert cases == 9 * 40


def test_plan_fixed_jump_matches_oracle():
    import oracle as O
    for n in range(1, 12):
        for step in range(1, 6):
            want = O.fixed_jump_plan(n, step)
            assert T.sa_plan_fixed_jump(n, step) == (list(want[0]), list(want[1]))


def test_planner_errors():
    import numpy as np
    L = T.lib()
    m = (ctypes.c_int32 * 4)()
    s = (ctypes.c_int32 * 4)()
    ov = np.zeros((4, 4), dtype=np.int64)
    p = ctypes.c_void_p(ov.ctypes.data)
    assert L.sa_plan_reuse(None, 10, 4, 0.5, None, m, s) == Bn.SA_ERR_NULL
    assert L.sa_plan_reuse(p, 10, 0, 0.5, None, m, s) == Bn.SA_ERR_SHAPE
    assert L.sa_plan_reuse(p, 10, 257, 0.5, None, m, s) == Bn.SA_ERR_SHAPE
    assert L.sa_plan_reuse(p, 0, 4, 0.5, None, m, s) == Bn.SA_ERR_SHAPE
    assert L.sa_plan_reuse(p, 10, 4, float("nan"), None, m, s) == Bn.SA_ERR_SHAPE
    ov[0, 3] = 11
    assert L.sa_plan_reuse(p, 10, 4, 0.5, None, m, s) == Bn.SA_ERR_SHAPE
    ov[0, 3] = -1
    assert L.sa_plan_reuse(p, 10, 4, 0.5, None, m, s) == Bn.SA_ERR_SHAPE
    ov[0, 3] = 0
    ov[3, 0] = 99            # below the diagonal: never read
    assert L.sa_plan_reuse(p, 10, 4, 0.5, None, m, s) == Bn.SA_OK
    assert L.sa_plan_fixed_jump(4, 0, m, s) == Bn.SA_ERR_SHAPE
    assert L.sa_plan_fixed_jump(0, 1, m, s) == Bn.SA_ERR_SHAPE
    assert L.sa_plan_fixed_jump(4, 1, None, s) == Bn.SA_ERR_NULL
    assert L.sa_index_overlap(None, FAKE, 4, 8, FAKE, None) == Bn.SA_ERR_NULL
    assert L.sa_index_overlap(FAKE, FAKE, 0, 8, FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_index_overlap(FAKE, FAKE, 4, 0, FAKE, None) == Bn.SA_ERR_SHAPE
    assert L.sa_index_overlap(FAKE, ctypes.c_void_p((1 << 20) + 2), 4, 8, FAKE,
                              None) == Bn.SA_ERR_ALIGN


def test_dense_scored_and_dense_select_errors():
    L = T.lib()
    d = _desc()
    nb = L.sa_dense_scored_workspace_size(ctypes.byref(d))
    ws = ctypes.c_void_p(1 << 24) if nb else None
    assert L.sa_dense_decode_scored(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, ws, nb,
                                    None) == Bn.SA_ERR_NULL
    assert L.sa_dense_decode_scored(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE,
                                    ctypes.c_void_p((1 << 20) + 2), ws, nb, None) == Bn.SA_ERR_ALIGN
    assert L.sa_dense_decode_scored(ctypes.byref(_desc(head_dim=96)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                    ws, nb, None) == Bn.SA_ERR_UNSUPPORTED
    a = Bn.LayerArgs()
    a.desc = d
    a.q = a.k_cache = a.v_cache = a.out = 1 << 20
    a.score_kind = Bn.SA_SCORE_EXACT
    a.k = 10
    need = L.sa_layer_workspace_size(ctypes.byref(a), Bn.SA_LAYER_DENSE_SELECT)
    # scores [B, Hkv, N] fp32 on top of what DENSE needs
    assert need >= 2 * 2 * 1000 * 4 + L.sa_layer_workspace_size(ctypes.byref(a), Bn.SA_LAYER_DENSE)
    a.ws, a.ws_bytes = 1 << 24, need
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_DENSE_SELECT, None, None) == Bn.SA_ERR_NULL
    a.ws_bytes = need - 256
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_DENSE_SELECT, FAKE,
                             None) == Bn.SA_ERR_WORKSPACE
    a.ws_bytes = need
    a.k = 1001
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_DENSE_SELECT, FAKE, None) == Bn.SA_ERR_SHAPE
    a.k = 10
    a.score_kind = Bn.SA_SCORE_BLOCK_MINMAX
    assert L.sa_decode_layer(ctypes.byref(a), Bn.SA_LAYER_DENSE_SELECT, FAKE,
                             None) == Bn.SA_ERR_UNSUPPORTED
    assert L.sa_decode_layer(ctypes.byref(a), 4, FAKE, None) == Bn.SA_ERR_SHAPE
    T.sa_plan_validate([Bn.SA_LAYER_DENSE_SELECT, Bn.SA_LAYER_REUSE], [-1, 0])


def test_per_query_head_row_limit():
    """Per-query-head rows are batch * n_q_heads grid rows: above 65535 the
    calls refuse on the host."""
    L = T.lib()
    d = _desc(batch=2049, n_q_heads=32, n_kv_heads=8)     # 16392 KV rows, 65568 query rows
    assert _sparse(d, ik=Bn.SA_IDX_TOKEN_PER_Q_HEAD) == Bn.SA_ERR_SHAPE
    assert L.sa_score(ctypes.byref(d), Bn.SA_SCORE_EXACT_PER_Q_HEAD, FAKE, FAKE, None, FAKE,
                      None) == Bn.SA_ERR_SHAPE
    assert _sparse(_desc(), ik=4) == Bn.SA_ERR_SHAPE        # unknown index kind


def test_gather_blocks_errors():
    """Offload gather: shapes and block sizes are checked, and host pointers
    that are not pinned host memory are refused, before any launch."""
    import numpy as np
    L = T.lib()
    d = _desc(ctx_len=1024)

    def call(desc=d, kh=FAKE, vh=FAKE, idx=FAKE, n_blk=4, bs=128, ko=FAKE, vo=FAKE):
        return L.sa_gather_blocks(ctypes.byref(desc) if desc is not None else None, kh, vh, idx,
                                  n_blk, bs, ko, vo, None)

    assert call(desc=None) == Bn.SA_ERR_NULL
    assert call(bs=0) == Bn.SA_ERR_SHAPE
    assert call(bs=4097) == Bn.SA_ERR_SHAPE
    assert call(bs=100) == Bn.SA_ERR_SHAPE             # 1024 is not a multiple of 100
    assert call(n_blk=0) == Bn.SA_ERR_SHAPE
    assert call(n_blk=9) == Bn.SA_ERR_SHAPE            # only 8 blocks of 128
    assert call(kh=None) == Bn.SA_ERR_NULL
    assert call(ko=ctypes.c_void_p((1 << 20) + 8)) == Bn.SA_ERR_ALIGN
    assert call(idx=ctypes.c_void_p((1 << 20) + 2)) == Bn.SA_ERR_ALIGN
    import torch
    if not torch.cuda.is_available():
        # pageable host memory is refused (without a GPU every lookup of a
        # device address fails the same way; with one, the GPU tests cover it
        # on real buffers, since outputs here are placeholders)
        plain = np.zeros(1 << 16, dtype=np.uint8)
        p = ctypes.c_void_p((plain.ctypes.data + 255) // 256 * 256)
        assert call(kh=p, vh=p) == Bn.SA_ERR_MEMORY
        assert "pinned" in T.lib().sa_last_error().decode()


def test_bench_select_bytes_follow_the_library_plan():
    """bench.py prices the fused selection by its candidate count; that count
    must be the library's: the workspace is a score and a position per
    candidate slot (rows rounded to 4 slots, 256-byte aligned halves), none
    for one part, the score array when the candidates exceed a quarter of
    the row."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(__file__), "..", "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    L = T.lib()
    for B, Hkv, N, k in [(16, 8, 32768, 655), (2, 2, 32768, 655), (1, 8, 65536, 1500),
                         (32, 8, 17152, 300), (1, 1, 20000, 300), (3, 3, 100, 10),
                         (2, 2, 32768, 12000), (64, 8, 4096, 100), (16, 8, 131072, 2621),
                         (16, 8, 32768, 3276), (16, 8, 32768, 6553)]:
        d = _desc(batch=B, n_q_heads=Hkv, n_kv_heads=Hkv, ctx_len=N, kv_stride_b=Hkv * N * 128,
                  kv_stride_h=N * 128)
        rows = B * Hkv
        C, fused = bench.select_candidates(rows, N, k)
        got = L.sa_select_workspace_size(ctypes.byref(d), Bn.SA_SCORE_EXACT, k)
        if not fused:
            want = -(-rows * N * 4 // 256) * 256 + L.sa_topk_workspace_size(rows, N, k)
        elif C == min(k, N) and got == 0:
            want = 0  # one part per row
        else:
            want = 2 * (-(-rows * (-(-C // 4) * 4) * 4 // 256) * 256)
        assert got == want, (B, Hkv, N, k, C, fused, got, want)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why,
    before touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(__file__), "..", "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_bench_summarize_percentiles(tmp_path):
    """The kernel-trace summary gives count, mean, min, max, median, p10 and
    p90 per kernel name (durations in ns in, microseconds out)."""
    import importlib.util
    import sqlite3
    spec = importlib.util.spec_from_file_location(
        "bench_mod", os.path.join(os.path.dirname(__file__), "..", "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    db = tmp_path / "t_results.db"
    con = sqlite3.connect(str(db))
    con.execute("create table kernels (name text, start integer, end integer)")
    for i in range(1, 11):  # 1..10 us
        con.execute("insert into kernels values (?, ?, ?)", ("k_a", 0, i * 1000))
    con.execute("insert into kernels values (?, ?, ?)", ("k_b", 0, 500))
    con.commit()
    con.close()
    text, rows, counters = bench.summarize(str(db))
    lines = {l.split()[0]: l.split()[1:] for l in text.splitlines()[1:]}
    n, avg, mn, mx, med, p10, p90 = lines["k_a"]
    assert int(n) == 10 and float(avg) == 5.5 and float(mn) == 1.0 and float(mx) == 10.0
    assert float(med) == 5.5 and abs(float(p10) - 1.9) < 1e-9 and abs(float(p90) - 9.1) < 1e-9
    assert lines["k_b"][0] == "1" and float(lines["k_b"][4]) == 0.5
    assert counters == {}


def test_noalloc_rejects_plans_beyond_its_scratch():
    """sa_sparse_decode_noalloc: the same argument checks as sa_sparse_decode,
    and a plan whose split partials exceed the 16 MiB static scratch is
    refused on the host with SA_ERR_WORKSPACE (every pointer is fake)."""
    L = T.lib()
    d = _desc()

    def na(desc, q=FAKE, n_idx=10, ik=0):
        return L.sa_sparse_decode_noalloc(ctypes.byref(desc) if desc is not None else None, q,
                                          FAKE, FAKE, ik, FAKE, n_idx, 0, FAKE, None)

    assert na(None) == Bn.SA_ERR_NULL
    assert na(d, q=None) == Bn.SA_ERR_NULL
    assert na(d, q=MIS) == Bn.SA_ERR_ALIGN
    assert na(d, n_idx=0) == Bn.SA_ERR_SHAPE
    big = _desc(batch=128, n_q_heads=32, n_kv_heads=8, ctx_len=65536,
                kv_stride_b=8 * 65536 * 128, kv_stride_h=65536 * 128)
    need = L.sa_sparse_workspace_size(ctypes.byref(big), 0, 16384, 0)
    assert need > 16 << 20
    assert na(big, n_idx=16384) == Bn.SA_ERR_WORKSPACE
    assert "16777216" in L.sa_last_error().decode()


def test_check_indices_errors():
    """sa_check_indices: index-kind, pointer and size checks on the host."""
    L = T.lib()
    d = _desc()

    def ci(desc, idx=FAKE, n_idx=10, ik=0, bs=0, counts=FAKE):
        return L.sa_check_indices(ctypes.byref(desc) if desc is not None else None, ik, idx,
                                  n_idx, bs, counts, None)

    assert ci(None) == Bn.SA_ERR_NULL
    assert ci(d, idx=None) == Bn.SA_ERR_NULL
    assert ci(d, counts=None) == Bn.SA_ERR_NULL
    assert ci(d, n_idx=0) == Bn.SA_ERR_SHAPE
    assert ci(d, ik=9) == Bn.SA_ERR_SHAPE
    assert ci(d, ik=Bn.SA_IDX_BLOCK_PER_KV_HEAD, bs=0) == Bn.SA_ERR_SHAPE
    assert ci(d, n_idx=8193) == Bn.SA_ERR_UNSUPPORTED
    assert "8192" in L.sa_last_error().decode()


_PLAN_PROBE = r"""
import ctypes, json, sys
sys.path.insert(0, %r)
import top_sparse_decode_sa_amd as T
from top_sparse_decode_sa_amd import _binding as Bn
L = T.lib()
out = []
for B, Hkv, N, k in [(1, 8, 32768, 655), (16, 8, 32768, 655), (128, 8, 131072, 262),
                     (1, 1, 1048576, 2048), (4, 2, 5000, 61)]:
    d = Bn.KVDesc(batch=B, n_q_heads=4 * Hkv, n_kv_heads=Hkv, head_dim=128, ctx_len=N,
                  q_dtype=Bn.SA_BF16, kv_dtype=Bn.SA_BF16, kv_stride_b=Hkv * N * 128,
                  kv_stride_h=N * 128, kv_stride_t=128)
    out.append([L.sa_sparse_workspace_size(ctypes.byref(d), 0, k, 0),
                L.sa_dense_workspace_size(ctypes.byref(d))])
print(json.dumps(out))
"""


def test_launch_plans_ignore_the_environment():
    """The library is stateless: no environment variable steers its launch
    plans (the workspace sizes follow from the plan's split counts), and its
    sources read none."""
    import subprocess
    import sys
    src = os.path.join(ROOT, "top_sparse_decode_sa_amd", "csrc")
    for f in os.listdir(src):
        assert "getenv" not in open(os.path.join(src, f)).read(), f
    probe = _PLAN_PROBE % ROOT

    def run(env):
        e = dict(os.environ)
        e.update(env)
        return subprocess.run([sys.executable, "-c", probe], env=e, check=True,
                              capture_output=True, text=True).stdout
    knobs = {"SA_SPARSE_CHUNK": "64", "SA_SPARSE_WAVES": "1", "SA_DENSE_WAVES": "2",
             "SA_DENSE_ROUNDS": "7"}
    assert run({}) == run(knobs)


def test_bench_oracle_baseline_on_small_workloads(tmp_path):
    """The per-workload cpu_baseline leg of bench.py (oracle worker processes
    behind a barrier, makespans scaled to a step) on shrunken copies of the
    three workloads: every figure is positive and finite, and the units
    reported are the ones dealt out."""
    import dataclasses
    import math

    import numpy as np

    import bench
    import sa_synth as S
    C = S.CONFIGS
    small = {
        "batch128k": dataclasses.replace(C["batch128k"], batch=4, ctx_len=2048, k=8, n_planted=8),
        "block61k": dataclasses.replace(C["block61k"], batch=2, ctx_len=1024, k=3),
        "indexer1m": dataclasses.replace(C["indexer1m"], ctx_len=4096, k=64),
    }
    for name, c in small.items():
        shm = None
        if name == "indexer1m":
            w = S.Workload(c, 0)
            shm = str(tmp_path)
            for l in range(c.n_layers):
                if c.modes[l] == "sparse":
                    k, q = w.k(l), w.q(l)
                    np.savez(os.path.join(shm, "layer%d.npz" % l), qi=w.indexer_q(l, q),
                             ki=w.indexer_k(l, k), wi=w.indexer_w(l), q=q)
        cpu = bench.config_cpu_baseline(name, 0, 10 ** 6, shm=shm, cfg=c, workers=2)
        assert cpu["cores"] == 2 and cpu["kind"] == "oracle"
        for v in (cpu["value"], cpu["steps_per_s"], cpu["one_thread"]["steps_per_s"],
                  cpu["one_thread"]["attend_gbps"]):
            assert v > 0 and math.isfinite(v), (name, cpu)
        want = {"batch128k": 2 * max(1, 64 // 2), "block61k": c.batch * c.n_kv_heads,
                "indexer1m": 6 + 2 * c.n_kv_heads}[name]
        assert "%d units" % want in cpu["sample"], (name, cpu["sample"])


def test_bench_perhead_oracle_baseline_on_a_small_workload():
    """The cpu_baseline leg of bench.py --perhead (the oracle's per-query-head
    step: each head's exact scores, its top-k and its attention) on a
    shrunken llama32k workload: every row timed, the figures positive and
    finite, and each head's set is its own top-k (the planted keys of its KV
    head lead every head of the group)."""
    import dataclasses
    import math

    import numpy as np

    import bench
    import oracle as O
    import sa_synth as S
    c = dataclasses.replace(S.CONFIGS["llama32k"], batch=2, ctx_len=2048, k=40, n_planted=20)
    w = S.Workload(c, 0)
    cpu = bench.perhead_cpu_baseline(w, 10 ** 6, 60.0)
    rows = c.batch * c.n_q_heads
    assert cpu["cores"] == 1 and cpu["kind"] == "oracle"
    assert "%d of the %d query-head rows" % (rows, rows) in cpu["sample"], cpu["sample"]
    for v in (cpu["value"], cpu["steps_per_s"], cpu["attend_steps_per_s"]):
        assert v > 0 and math.isfinite(v), cpu
    # the unit the leg times, for one head: its own top-k holds its KV head's planted keys
    scale = O.default_scale(c.head_dim)
    qf = O.widen(w.q(0, batch=(0, 1))[0])
    kf = O.widen(w.k(0, batch=(0, 1))[0])
    for h in (0, c.n_q_heads - 1):
        sel = O.topk(O.scores_exact(qf[h:h + 1], kf[h // c.group], scale), c.k)
        planted = np.asarray(w.planted(0, 0, h // c.group))
        assert np.isin(planted, sel).all(), h


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_compiles_as_c_and_cxx(tmp_path, lang, compiler):
    """include/sa.h is a C header usable from C and C++, and its enumerations
    have the size of int32_t in both."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(compiler + " missing")
    src = tmp_path / "t.c"
    src.write_text('#include "sa.h"\n'
                   'typedef char enum_is_32_bit[sizeof(sa_dtype) == 4 && sizeof(sa_status) == 4 '
                   '? 1 : -1];\n'
                   'int main(void) { sa_kv_desc d; d.q_dtype = SA_BF16; return (int)d.q_dtype; }\n')
    r = subprocess.run([compiler, "-fsyntax-only", "-Wall", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-x", lang,
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_gather_read_errors():
    """sa_gather_read: argument checks on the host, and SA_ERR_UNSUPPORTED
    where sa_sparse_decode would not run the pair-pipelined gather-attend."""
    L = T.lib()
    d = _desc()

    def gr(desc, k=FAKE, sink=FAKE, n_idx=10, ik=0, bs=0, idx=FAKE):
        return L.sa_gather_read(ctypes.byref(desc) if desc is not None else None, k, FAKE, ik,
                                idx, n_idx, bs, sink, None)

    assert gr(None) == Bn.SA_ERR_NULL
    assert gr(d, k=None) == Bn.SA_ERR_NULL
    assert gr(d, sink=None) == Bn.SA_ERR_NULL
    assert gr(d, k=MIS) == Bn.SA_ERR_ALIGN
    assert gr(d, n_idx=0) == Bn.SA_ERR_SHAPE
    assert gr(d, idx=None) == Bn.SA_ERR_NULL
    f32 = _desc(q_dtype=Bn.SA_F32, kv_dtype=Bn.SA_F32)
    assert gr(f32) == Bn.SA_ERR_UNSUPPORTED
    assert "pair-pipelined" in L.sa_last_error().decode()


def test_bench_oracle_pool_reports_a_failed_worker():
    """A worker of the oracle baseline that fails (here: an unknown unit)
    makes the pool raise instead of leaving the others at the barrier."""
    import bench
    import sa_synth as S
    with pytest.raises(RuntimeError, match="oracle worker failed"):
        bench.oracle_pool(S.CONFIGS["tiny"], 0, [[("no such unit",)], [("no such unit",)]])
