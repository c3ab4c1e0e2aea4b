"""GPU parity of each C-ABI call against the CPU oracle on small and ragged
inputs: every kernel family, every index kind, dtype, head size and group
size, edge cases (k = 1, k = n, ties, -0.0, NaN, partial blocks, strided
caches), at sizes the oracle finishes in seconds."""
import numpy as np
import pytest
import torch

import oracle as O
import sa_synth as S
import top_sparse_decode_sa_amd as T
from gpu_util import check_out, dev, say, score_tol, to_dev, to_host_bits, verdicts

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(7)


def _rand_cache(B, Hq, Hkv, N, d, dtype, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(tdt)
    return q, k, v


def _f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


# --------------------------------------------------------------------- top-k

@pytest.mark.parametrize("n", [1, 2, 7, 100, 480, 511, 512, 513, 1000, 1025, 3000, 4097, 8192, 8193, 32768, 32773])
def test_topk_bit_exact(n):
    say("topk n=%d" % n)
    rows = 5
    vals = RNG.standard_normal((rows, n)).astype(np.float32)
    vals[1] = np.round(vals[1] * 2) / 2          # heavy ties
    vals[2, ::3] = -0.0
    vals[2, 1::3] = 0.0
    if n > 4:
        vals[3, :4] = [np.inf, -np.inf, np.nan, np.nan]
    vals[4] = 1.0                                 # all equal
    x = torch.from_numpy(vals).to(dev())
    for k in sorted({1, max(1, n // 50), max(1, n // 3), n}):
        got = T.sa_topk(x, k).cpu().numpy()
        for r in range(rows):
            want = O.topk(vals[r].astype(np.float64), k)
            assert np.array_equal(got[r], want), (n, k, r)


@pytest.mark.parametrize("rows,n,k", [(3, 40000, 1), (3, 200003, 2048), (2, 200003, 8192),
                                       (2, 100000, 9000), (1, 1048576, 2048), (70, 40004, 300),
                                       (66, 65536, 5000), (65, 131072, 12000)])
def test_topk_long_rows(rows, n, k):
    """Rows longer than the register-resident limit: few rows take the
    multi-workgroup path (k <= 8192), more rows or larger k the row path --
    its short-list finish when the keys of the threshold bin and above fit in
    LDS (with a partial last chunk), its LDS tiles otherwise; tied rows whose
    candidate bin overflows exercise the in-kernel fallbacks."""
    say("topk long rows=%d n=%d k=%d" % (rows, n, k))
    rng = np.random.default_rng(n + k)
    vals = rng.standard_normal((rows, n)).astype(np.float32)
    if rows > 1:
        vals[1] = np.round(vals[1] * 2) / 2      # heavy ties: bin overflow
    if rows > 2:
        vals[2, ::7] = 5.0                       # ties above everything else
    x = torch.from_numpy(vals).to(dev())
    got = T.sa_topk(x, k).cpu().numpy()
    for r in range(rows):
        want = O.topk(vals[r].astype(np.float64), k)
        assert np.array_equal(got[r], want), (rows, n, k, r)


@pytest.mark.parametrize("n,k", [(150001, 2048), (1048576, 2048), (40000, 8192)])
def test_topk_long_rows_ties_at_the_threshold(n, k):
    """Multi-workgroup rows whose k-th largest score is shared by a few
    hundred positions spread over every chunk: only the lowest positions of
    the tie are kept, and the kept set is written in ascending order."""
    say("topk long rows, ties at the threshold n=%d k=%d" % (n, k))
    rng = np.random.default_rng(n + 3 * k)
    vals = rng.standard_normal((2, n)).astype(np.float32)
    for r in range(2):
        v = np.sort(vals[r])[::-1][k - 100 + 50 * r]
        vals[r, rng.choice(n, 400, replace=False)] = v
    vals[1, rng.choice(n, 50, replace=False)] = -0.0   # signed zeros tie with +0.0
    vals[1, rng.choice(n, 50, replace=False)] = 0.0
    got = T.sa_topk(torch.from_numpy(vals).to(dev()), k).cpu().numpy()
    for r in range(2):
        assert np.array_equal(got[r], O.topk(vals[r].astype(np.float64), k)), (n, k, r)


def test_topk_row_stride():
    say("topk row_stride")
    base = RNG.standard_normal((6, 3000)).astype(np.float32)
    view = torch.from_numpy(base).to(dev())[:, :2500]  # rows 3000 apart, n = 2500
    got = T.sa_topk(view, 40).cpu().numpy()
    for r in range(6):
        assert np.array_equal(got[r], O.topk(base[r, :2500].astype(np.float64), 40))


# ------------------------------------------------------------------- scoring

@pytest.mark.parametrize("dtype,d,G", [("f32", 64, 4), ("bf16", 128, 4), ("bf16", 64, 8),
                                       ("f32", 128, 1), ("bf16", 128, 2)])
def test_score_exact(dtype, d, G):
    say("score_exact", dtype, d, G)
    B, Hkv, N = 2, 2, 1000
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, 11)
    s = T.sa_score(q.to(dev()), k.to(dev())).cpu().numpy()
    qf, kf = _f64(q), _f64(k)
    for b in range(B):
        for r in range(Hkv):
            want = O.scores_exact(qf[b, r * G:(r + 1) * G], kf[b, r], O.default_scale(d))
            assert np.max(np.abs(s[b, r] - want)) <= score_tol(want)


@pytest.mark.parametrize("dtype,d,bs,N", [("bf16", 128, 128, 1000), ("f32", 64, 16, 257),
                                          ("bf16", 64, 128, 128)])
def test_block_summaries_and_scores(dtype, d, bs, N):
    say("block", dtype, d, bs, N)
    B, Hkv, G = 2, 2, 4
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, 12)
    kd = k.to(dev())
    kmin, kmax = T.sa_block_summarize(kd, bs)
    sb = T.sa_score(q.to(dev()), kd, T.SA_SCORE_BLOCK_MINMAX, kmin=kmin, kmax=kmax,
                    block_size=bs).cpu().numpy()
    qf, kf = _f64(q), _f64(k)
    mn_g, mx_g = _f64(kmin), _f64(kmax)
    for b in range(B):
        for r in range(Hkv):
            mn, mx = O.block_summaries(kf[b, r], bs)
            assert np.array_equal(mn_g[b, r], mn) and np.array_equal(mx_g[b, r], mx)
            want = O.scores_block(qf[b, r * G:(r + 1) * G], mn, mx)
            assert np.max(np.abs(sb[b, r] - want)) <= score_tol(want)


@pytest.mark.parametrize("H,Di", [(4, 64), (3, 128), (16, 32)])
def test_score_indexer(H, Di):
    say("indexer", H, Di)
    B, N = 2, 3001
    rng = np.random.default_rng(13)
    qi = torch.from_numpy(rng.standard_normal((B, H, Di)).astype(np.float32)).to(torch.bfloat16)
    ki = torch.from_numpy(rng.standard_normal((B, N, Di)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.uniform(size=(B, H)).astype(np.float32))
    q, kc, vc = _rand_cache(B, 8, 2, N, 128, "bf16", 1)
    s = T.sa_score(q.to(dev()), kc.to(dev()), T.SA_SCORE_INDEXER, q_idx=qi.to(dev()),
                   k_idx=ki.to(dev()), idx_w=w.to(dev())).cpu().numpy()
    for b in range(B):
        want = O.scores_indexer(_f64(qi)[b], _f64(ki)[b], w.numpy()[b].astype(np.float64))
        assert np.max(np.abs(s[b] - want)) <= score_tol(want)


@pytest.mark.parametrize("N,k", [(3001, 60), (8192, 17)])
def test_indexer_per_kv_head_layer(N, k):
    """The indexer applied per (sequence, KV head): scores against the oracle
    row by row, then one SPARSE layer through sa_decode_layer (indexer ->
    top-k -> attend) judged on its index sets and outputs."""
    say("indexer per KV head", N, k)
    B, Hq, Hkv, d, H, Di = 2, 8, 2, 128, 4, 64
    rng = np.random.default_rng(N + k)
    q, kc, vc = _rand_cache(B, Hq, Hkv, N, d, "bf16", 31)
    qi = torch.from_numpy(rng.standard_normal((B, Hkv, H, Di)).astype(np.float32)).to(torch.bfloat16)
    ki = torch.from_numpy(rng.standard_normal((B, Hkv, N, Di)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.uniform(size=(B, Hkv, H)).astype(np.float32))
    qd, kd, vd = q.to(dev()), kc.to(dev()), vc.to(dev())
    qid, kid, wd = qi.to(dev()), ki.to(dev()), w.to(dev())
    s = T.sa_score(qd, kd, T.SA_SCORE_INDEXER_PER_KV_HEAD, q_idx=qid, k_idx=kid,
                   idx_w=wd).cpu().numpy()
    want = np.empty((B, Hkv, N))
    for b in range(B):
        for r in range(Hkv):
            want[b, r] = O.scores_indexer(_f64(qi)[b, r], _f64(ki)[b, r],
                                          w.numpy()[b, r].astype(np.float64))
            assert np.max(np.abs(s[b, r] - want[b, r])) <= score_tol(want[b, r])
    a, out, dv = T.layer_args(qd, kd, vd, T.SA_SCORE_INDEXER_PER_KV_HEAD, k, q_idx=qid, k_idx=kid,
                              idx_w=wd)
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev())
    T.sa_decode_layer(a, T.SA_LAYER_SPARSE, idx, dv)
    got = idx.cpu().numpy()
    counts, fails = verdicts(want.reshape(B * Hkv, N), got.reshape(B * Hkv, k), k)
    assert not fails, fails[:3]
    scale = O.default_scale(d)
    ref = _oracle_out(_f64(q), _f64(kc), _f64(vc), got, Hq // Hkv, scale)
    check_out(out.cpu().numpy(), ref, "bf16", "indexer per KV head layer")


@pytest.mark.parametrize("x", [2, 5, 20, 100, 500])
def test_sparse_across_sparsity(x):
    """Exact step (score -> top-k -> attend) at k = N/x, 2x to 500x: every
    launch plan of the gather kernel (split rows with a combine, whole-row
    workgroups) against the oracle."""
    say("sparsity sweep x=%d" % x)
    B, Hq, Hkv, d, N = 2, 8, 2, 128, 8192
    k = N // x
    q, kc, vc = _rand_cache(B, Hq, Hkv, N, d, "bf16", 40 + x)
    qd, kd, vd = q.to(dev()), kc.to(dev()), vc.to(dev())
    s = T.sa_score(qd, kd, T.SA_SCORE_EXACT)
    idx = T.sa_topk(s, k)
    out = T.sa_sparse_decode(qd, kd, vd, idx).cpu().numpy()
    scale = O.default_scale(d)
    qf, kf, vf = _f64(q), _f64(kc), _f64(vc)
    rows_s, rows_g = [], []
    for b in range(B):
        for r in range(Hkv):
            rows_s.append(O.scores_exact(qf[b, r * (Hq // Hkv):(r + 1) * (Hq // Hkv)], kf[b, r], scale))
    got = idx.cpu().numpy()
    counts, fails = verdicts(rows_s, got.reshape(B * Hkv, k), k)
    assert not fails, fails[:3]
    check_out(out, _oracle_out(qf, kf, vf, got, Hq // Hkv, scale), "bf16", "x=%d" % x)


# ---------------------------------------------------------------- attention

def _oracle_out(qf, kf, vf, sets, G, scale):
    B, Hq, d = qf.shape
    out = np.empty((B, Hq, d))
    for b in range(B):
        for r in range(Hq // G):
            out[b, r * G:(r + 1) * G] = O.attend(qf[b, r * G:(r + 1) * G], kf[b, r], vf[b, r],
                                                 sets[b][r], scale)
    return out


@pytest.mark.parametrize("dtype,d,G,N,n_idx", [("bf16", 128, 4, 5000, 655), ("f32", 64, 4, 1024, 64),
                                               ("bf16", 64, 8, 777, 1), ("f32", 128, 2, 3000, 1500),
                                               ("bf16", 128, 1, 2048, 333)])
def test_sparse_token_per_head(dtype, d, G, N, n_idx):
    say("sparse per-head", dtype, d, G, N, n_idx)
    B, Hkv = 3, 2
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, 21)
    rng = np.random.default_rng(22)
    idx = np.stack([np.stack([np.sort(rng.choice(N, n_idx, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    out = T.sa_sparse_decode(q.to(dev()), k.to(dev()), v.to(dev()),
                             torch.from_numpy(idx).to(dev())).cpu().numpy()
    want = _oracle_out(_f64(q), _f64(k), _f64(v), [[idx[b, r] for r in range(Hkv)] for b in range(B)],
                       G, O.default_scale(d))
    check_out(out, want, dtype, "sparse per-head")


@pytest.mark.parametrize("G,B,Hkv,N,n_idx,qmul", [
    (1, 32, 4, 1024, 655, 1.0), (2, 32, 4, 1024, 655, 1.0), (4, 32, 4, 1024, 768, 1.0),
    (2, 32, 4, 1024, 300, 8.0), (4, 32, 4, 1024, 33, 8.0), (2, 2, 4, 4096, 2048, 1.0),
    (1, 2, 4, 4096, 1500, 8.0)])
def test_pair_kernel_groups_and_plans(G, B, Hkv, N, n_idx, qmul):
    """The pair-pipelined gather-attend at 1, 2 and 4 query heads per KV head,
    in both of its plans: 128 whole rows with two workgroups per row (value
    halves; one or two pairs per wave, a partial last wave, a full twelfth
    wave) and 8 rows split over many workgroups with the combine; queries
    scaled by 8 make most of a row's probabilities underflow against its
    maximum."""
    say("pair kernel", G, B, Hkv, N, n_idx, qmul)
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, 128, "bf16", 50 + G + n_idx)
    q = (q.to(torch.float32) * qmul).to(torch.bfloat16)
    rng = np.random.default_rng(51 + n_idx)
    idx = np.stack([np.stack([np.sort(rng.choice(N, n_idx, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    out = T.sa_sparse_decode(q.to(dev()), k.to(dev()), v.to(dev()),
                             torch.from_numpy(idx).to(dev())).cpu().numpy()
    want = _oracle_out(_f64(q), _f64(k), _f64(v), [[idx[b, r] for r in range(Hkv)] for b in range(B)],
                       G, O.default_scale(128))
    check_out(out, want, "bf16", "pair kernel G=%d rows=%d n_idx=%d" % (G, B * Hkv, n_idx))


def test_sparse_shared_and_unsorted_indices():
    say("sparse shared")
    B, Hkv, G, N, d, n_idx = 2, 4, 4, 4000, 128, 700
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, "bf16", 31)
    rng = np.random.default_rng(32)
    idx = np.stack([rng.choice(N, n_idx, replace=False) for _ in range(B)]).astype(np.int32)
    out = T.sa_sparse_decode(q.to(dev()), k.to(dev()), v.to(dev()), torch.from_numpy(idx).to(dev()),
                             T.SA_IDX_TOKEN_SHARED).cpu().numpy()
    want = _oracle_out(_f64(q), _f64(k), _f64(v), [[idx[b]] * Hkv for b in range(B)], G,
                       O.default_scale(d))
    check_out(out, want, "bf16", "sparse shared")


def _bad_rows(idx, limit):
    """Rows with an index outside [0, limit), rows with a repeated index."""
    rows = idx.reshape(-1, idx.shape[-1])
    return [int(sum(((r < 0) | (r >= limit)).any() for r in rows)),
            int(sum(len(set(r.tolist())) < len(r) for r in rows))]


@pytest.mark.parametrize("kind,n_idx", [(T.SA_IDX_TOKEN_PER_KV_HEAD, 1), (T.SA_IDX_TOKEN_PER_KV_HEAD, 700),
                                        (T.SA_IDX_TOKEN_PER_KV_HEAD, 8192), (T.SA_IDX_TOKEN_SHARED, 33),
                                        (T.SA_IDX_TOKEN_PER_Q_HEAD, 2048), (T.SA_IDX_BLOCK_PER_KV_HEAD, 24)])
def test_check_indices_counts_bad_rows(kind, n_idx):
    """sa_check_indices counts rows with an out-of-range index and rows with a
    repeat, on clean index sets and with mistakes planted at the row ends,
    in the middle, at -1, at the limit and as INT32 extremes."""
    say("check indices", kind, n_idx)
    B, Hkv, G, N, d, bs = 2, 4, 2, 9000, 64, 128
    q, k, _ = _rand_cache(B, Hkv * G, Hkv, N, d, "f32", 41)
    qd, kd = q.to(dev()), k.to(dev())
    limit = -(-N // bs) if kind == T.SA_IDX_BLOCK_PER_KV_HEAD else N
    rows = {T.SA_IDX_TOKEN_SHARED: B, T.SA_IDX_TOKEN_PER_Q_HEAD: B * Hkv * G}.get(kind, B * Hkv)
    rng = np.random.default_rng(n_idx)
    idx = np.stack([rng.choice(limit, n_idx, replace=False) for _ in range(rows)]).astype(np.int32)
    bsz = bs if kind == T.SA_IDX_BLOCK_PER_KV_HEAD else 0

    def run(x):
        got = T.sa_check_indices(qd, kd, torch.from_numpy(x).to(dev()), kind, bsz).cpu().tolist()
        assert got == _bad_rows(x, limit), (got, _bad_rows(x, limit))
        return got

    assert run(idx) == [0, 0]
    bad = idx.copy()
    bad[0, -1] = limit
    bad[rows - 1, 0] = -1
    if rows > 2:
        bad[1, n_idx // 2] = np.iinfo(np.int32).min
    if n_idx > 2:
        bad[rows - 1, -1] = bad[rows - 1, n_idx // 2]       # repeat in a row already out of range
    if n_idx > 3:
        bad[rows // 2, 1] = bad[rows // 2, 2]
    if rows > 3 and n_idx > 1:
        bad[2, 0] = bad[2, 1] = np.iinfo(np.int32).max       # out of range and repeated
    got = run(bad)
    assert got[0] >= 1 and (n_idx < 3 or got[1] >= 1)


@pytest.mark.parametrize("N,bs,n_blk", [(1000, 128, 3), (61440, 128, 24), (300, 16, 19),
                                         (8192, 128, 64), (4096, 16, 256), (2048, 128, 16)])
def test_sparse_blocks_with_partial_last_block(N, bs, n_blk):
    say("sparse blocks", N, bs, n_blk)
    B, Hkv, G, d = 2, 2, 4, 128
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, "bf16", 41)
    nb = (N + bs - 1) // bs
    rng = np.random.default_rng(42)
    # every row holds the last (possibly partial) block plus random others
    idx = np.stack([np.stack([rng.permutation(np.r_[rng.choice(nb - 1, n_blk - 1, replace=False), nb - 1])
                              for _ in range(Hkv)]) for _ in range(B)]).astype(np.int32)
    out = T.sa_sparse_decode(q.to(dev()), k.to(dev()), v.to(dev()), torch.from_numpy(idx).to(dev()),
                             T.SA_IDX_BLOCK_PER_KV_HEAD, block_size=bs).cpu().numpy()
    sets = [[O.block_tokens(idx[b, r], bs, N) for r in range(Hkv)] for b in range(B)]
    want = _oracle_out(_f64(q), _f64(k), _f64(v), sets, G, O.default_scale(d))
    check_out(out, want, "bf16", "sparse blocks")


@pytest.mark.parametrize("dtype,d,G,B,Hkv,N,bs,k,zero_q", [
    ("bf16", 128, 4, 2, 2, 61440, 128, 24, False),   # block61k rows
    ("bf16", 128, 4, 1, 2, 1000, 128, 3, False),     # partial last block
    ("f32", 64, 4, 2, 2, 5000, 16, 40, False),
    ("bf16", 64, 2, 1, 1, 4096 * 128, 128, 100, False),  # 4096 blocks: the fused limit
    ("bf16", 128, 4, 1, 1, 4097 * 16, 16, 50, False),    # one block more: score, then top-k
    ("bf16", 128, 4, 2, 2, 8192, 128, 10, True),     # every score 0: the first k blocks
])
def test_block_layer_selection(dtype, d, G, B, Hkv, N, bs, k, zero_q):
    """A SPARSE layer on block scores selects, in one launch where the row's
    blocks fit it, the same blocks as sa_score followed by sa_topk, and
    attends over them as sa_sparse_decode does."""
    say("block layer selection", dtype, d, G, B, Hkv, N, bs, k, zero_q)
    q, kc, vc = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, 43)
    if zero_q:
        q.zero_()
    qd, kd, vd = q.to(dev()), kc.to(dev()), vc.to(dev())
    kmin, kmax = T.sa_block_summarize(kd, bs, q_like=qd)
    args, out, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_BLOCK_MINMAX, k, kmin=kmin, kmax=kmax,
                                 block_size=bs)
    idx = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_)
    want = T.sa_topk(T.sa_score(qd, kd, T.SA_SCORE_BLOCK_MINMAX, kmin=kmin, kmax=kmax,
                                block_size=bs), k)
    ref = T.sa_sparse_decode(qd, kd, vd, want, T.SA_IDX_BLOCK_PER_KV_HEAD, block_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(idx, want)
    assert torch.equal(out, ref)
    if zero_q:
        assert torch.equal(idx.cpu(), torch.arange(k, dtype=torch.int32).expand(B, Hkv, k))


@pytest.mark.parametrize("dtype,d,G,N", [("f32", 64, 4, 1024), ("bf16", 128, 4, 20000),
                                         ("bf16", 64, 2, 999), ("f32", 128, 8, 3333)])
def test_dense_and_all_tokens_sparse(dtype, d, G, N):
    say("dense", dtype, d, G, N)
    B, Hkv = 2, 2
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, 51)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    dense = T.sa_dense_decode(qd, kd, vd).cpu().numpy()
    want = _oracle_out(_f64(q), _f64(k), _f64(v), [[np.arange(N)] * Hkv] * B, G, O.default_scale(d))
    check_out(dense, want, dtype, "dense")
    allidx = torch.arange(N, dtype=torch.int32, device=dev()).repeat(B, Hkv, 1).contiguous()
    sparse = T.sa_sparse_decode(qd, kd, vd, allidx).cpu().numpy()
    check_out(sparse, want, dtype, "sparse k=N")
    tol = 1e-5 if dtype == "f32" else 1e-4
    assert np.max(np.abs(sparse - dense)) <= tol


def test_window_equals_dense_on_window_and_strided_cache():
    """Top-k on recency is a sliding window: sparse over the last W tokens
    equals dense decode over a strided view holding only those tokens."""
    say("window")
    B, Hkv, G, N, d, W = 2, 2, 4, 5000, 128, 300
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, "bf16", 61)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    rec = torch.arange(N, dtype=torch.float32, device=dev()).repeat(B, Hkv, 1).contiguous()
    idx = T.sa_topk(rec, W)
    assert np.array_equal(idx.cpu().numpy()[0, 0], np.arange(N - W, N))
    sparse = T.sa_sparse_decode(qd, kd, vd, idx).cpu().numpy()
    dense_w = T.sa_dense_decode(qd, kd[:, :, N - W:], vd[:, :, N - W:]).cpu().numpy()
    assert np.max(np.abs(sparse - dense_w)) <= 1e-4
    # token-major cache [B, N, Hkv, d] viewed as [B, Hkv, N, d]
    ktm = kd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vtm = vd.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    sparse_tm = T.sa_sparse_decode(qd, ktm, vtm, idx).cpu().numpy()
    assert np.max(np.abs(sparse_tm - sparse)) <= 1e-5


# -------------------------------------------------------------- tiny config

def test_tiny_config_end_to_end():
    """Tiny exact-top-k decode (fp32, 8/2 heads, d 64, N 1024, k 64) through
    every call, plus k = N against dense."""
    say("tiny config")
    w = S.Workload("tiny", 0)
    c = w.cfg
    q_h, k_h, v_h = w.q(), w.k(), w.v()
    qd, kd, vd = to_dev(q_h), to_dev(k_h), to_dev(v_h)
    qf, kf, vf = O.widen(q_h), O.widen(k_h), O.widen(v_h)
    scale = O.default_scale(c.head_dim)
    scores = T.sa_score(qd, kd)
    s_gpu = scores.cpu().numpy()
    s64 = [O.scores_exact(qf[0, r * c.group:(r + 1) * c.group], kf[0, r], scale)
           for r in range(c.n_kv_heads)]
    for r in range(c.n_kv_heads):
        assert np.max(np.abs(s_gpu[0, r] - s64[r])) <= score_tol(s64[r])
    idx = T.sa_topk(scores, c.k)
    idx_h = idx.cpu().numpy()
    for r in range(c.n_kv_heads):
        assert np.array_equal(idx_h[0, r], O.topk(s_gpu[0, r].astype(np.float64), c.k))
        assert set(w.planted(0, 0, r)).issubset(idx_h[0, r])
    counts, fails = verdicts(s64, idx_h[0], c.k)
    assert not fails, fails
    out = T.sa_sparse_decode(qd, kd, vd, idx).cpu().numpy()
    want = _oracle_out(qf, kf, vf, [[idx_h[0, r] for r in range(c.n_kv_heads)]], c.group, scale)
    check_out(out, want, "f32", "tiny sparse")
    # the same through the layer entry point
    args, out2, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_EXACT, c.k)
    idx2 = torch.full((1, c.n_kv_heads, c.k), -1, dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx2, d_)
    assert torch.equal(idx2, idx)
    assert np.max(np.abs(out2.cpu().numpy() - out)) <= 1e-6
    # k = N equals dense
    dense = T.sa_dense_decode(qd, kd, vd).cpu().numpy()
    wantd = _oracle_out(qf, kf, vf, [[np.arange(c.ctx_len)] * c.n_kv_heads], c.group, scale)
    check_out(dense, wantd, "f32", "tiny dense")
    idx_all = T.sa_topk(scores, c.ctx_len)
    assert np.array_equal(idx_all.cpu().numpy()[0, 0], np.arange(c.ctx_len))
    full = T.sa_sparse_decode(qd, kd, vd, idx_all).cpu().numpy()
    check_out(full, wantd, "f32", "tiny k=N")
    assert np.max(np.abs(full - dense)) <= 1e-5


# ---------------------------------------------------- per-query-head index sets

@pytest.mark.parametrize("dtype,d,G,B,N,k", [
    ("bf16", 128, 4, 2, 3000, 61), ("bf16", 128, 4, 40, 2000, 40), ("bf16", 128, 1, 2, 777, 100),
    ("f32", 64, 8, 1, 1500, 33), ("bf16", 64, 2, 2, 999, 999), ("f32", 128, 4, 2, 2500, 50),
    ("f32", 64, 2, 3, 1300, 20)])
def test_per_query_head_selection(dtype, d, G, B, N, k):
    """Every query head scores, selects and attends on its own: scores
    against the oracle, sa_topk bit-exact on the GPU's scores, outputs
    against oracle attention of each head over its own set; the layer entry
    point equals the single calls."""
    say("per-q-head %s d=%d G=%d B=%d N=%d k=%d" % (dtype, d, G, B, N, k))
    Hkv = 2
    q, kc, vc = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, N + k)
    q, kc, vc = q.to(dev()), kc.to(dev()), vc.to(dev())
    scores = T.sa_score(q, kc, T.SA_SCORE_EXACT_PER_Q_HEAD)
    idx = T.sa_topk(scores, k)
    out = T.sa_sparse_decode(q, kc, vc, idx, T.SA_IDX_TOKEN_PER_Q_HEAD)
    args, out2, d_ = T.layer_args(q, kc, vc, T.SA_SCORE_EXACT_PER_Q_HEAD, k)
    idx2 = torch.empty((B, Hkv * G, k), dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx2, d_)
    torch.cuda.synchronize()
    assert tuple(scores.shape) == (B, Hkv * G, N)
    assert torch.equal(idx, idx2) and torch.equal(out, out2)
    qf, kf, vf = _f64(q), _f64(kc), _f64(vc)
    s, ih, o = scores.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy()
    scale = O.default_scale(d)
    for b in range(min(B, 3)):
        for h in range(Hkv * G):
            r = h // G
            s64 = O.scores_per_query_head(qf[b, h], kf[b, r], scale)
            assert np.max(np.abs(s[b, h] - s64)) <= score_tol(s64), (b, h)
            assert np.array_equal(ih[b, h], O.topk(s[b, h].astype(np.float64), k)), (b, h)
            v = O.index_set_verdict(s64, ih[b, h], k)
            assert not v.startswith("failed"), (b, h, v)
            want = O.attend(qf[b, h][None], kf[b, r], vf[b, r], ih[b, h], scale)
            check_out(o[b, h][None], want, dtype, "per-q-head %d,%d" % (b, h))


def test_per_query_head_with_shared_sets_equals_per_kv_head():
    """When the G query heads of a group hold the same set, per-query-head
    decode is per-KV-head decode (to fp32 rounding)."""
    say("per-q-head == per-kv-head on shared sets")
    B, Hkv, G, N, d, k = 3, 8, 4, 5000, 128, 100
    q, kc, vc = _rand_cache(B, Hkv * G, Hkv, N, d, "bf16", 23)
    q, kc, vc = q.to(dev()), kc.to(dev()), vc.to(dev())
    idx = T.sa_topk(T.sa_score(q, kc), k)
    per_q = idx.repeat_interleave(G, dim=1).contiguous()
    a = T.sa_sparse_decode(q, kc, vc, idx).cpu().numpy()
    b = T.sa_sparse_decode(q, kc, vc, per_q, T.SA_IDX_TOKEN_PER_Q_HEAD).cpu().numpy()
    assert np.max(np.abs(a - b)) <= 1e-5


# ------------------------------------------------------------ graph replay

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("B,Hkv,N,k", [(2, 4, 5000, 61), (1, 2, 40000, 300)])
def test_step_graph_replay(B, Hkv, N, k, fused):
    """A decode step (score -> top-k, or the fused sa_select, -> gather-attend)
    captured as a HIP graph and replayed several times, with new queries
    copied in eagerly and the stream synchronised between replays: every
    replay equals the eager step.  The shapes take the split attend plan with
    its combine launch, the multi-workgroup top-k with its zeroing kernel, and
    the fused selection's part and merge launches."""
    say("graph replay B=%d Hkv=%d N=%d k=%d fused=%s" % (B, Hkv, N, k, fused))
    G, d = 4, 128
    q, kc, vc = _rand_cache(B, Hkv * G, Hkv, N, d, "bf16", N)
    q, kc, vc = q.to(dev()), kc.to(dev()), vc.to(dev())
    scores = torch.empty((B, Hkv, N), dtype=torch.float32, device=dev())
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev())
    out = torch.empty((B, Hkv * G, d), dtype=torch.float32, device=dev())

    def step():
        if fused:
            T.sa_select(q, kc, k, idx_out=idx)
        else:
            T.sa_score(q, kc, T.SA_SCORE_EXACT, scores=scores)
            T.sa_topk(scores, k, idx_out=idx)
        T.sa_sparse_decode(q, kc, vc, idx, out=out)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rng = np.random.default_rng(N + 1)
    for rep in range(4):
        q.copy_(torch.from_numpy(rng.standard_normal(tuple(q.shape)).astype(np.float32)).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gi, go = idx.clone(), out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(gi, idx), "replay %d selects differently" % rep
        assert torch.equal(go, out), "replay %d attends differently" % rep


def test_layer_graph_replay_with_merge_attend():
    """A SPARSE layer whose merge and gather-attend share one launch (128
    rows of 32768 tokens, k = 655) captured as a HIP graph and replayed four
    times with new queries copied in eagerly between replays: every replay
    selects and attends as the eager layer call."""
    say("graph replay: SPARSE layer with merge-attend")
    B, Hkv, G, N, d, k = 16, 8, 4, 32768, 128, 655
    gen = torch.Generator(device=dev()).manual_seed(7)
    q = torch.randn((B, Hkv * G, d), generator=gen, device=dev()).to(torch.bfloat16)
    kc = torch.randn((B, Hkv, N, d), generator=gen, device=dev()).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, N, d), generator=gen, device=dev()).to(torch.bfloat16)
    args, out, d_ = T.layer_args(q, kc, vc, T.SA_SCORE_EXACT, k)
    ws = T.WORKSPACES.get(d_, ("graph-layer", T.SA_LAYER_SPARSE),
                          T.sa_layer_workspace_size(args, T.SA_LAYER_SPARSE))
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev())

    def layer():
        T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_, ws)

    layer()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    for rep in range(4):
        q.copy_(torch.randn(tuple(q.shape), generator=gen, device=dev()).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gi, go = idx.clone(), out.clone()
        layer()
        torch.cuda.synchronize()
        assert torch.equal(gi, idx), "replay %d selects differently" % rep
        assert torch.equal(go, out), "replay %d attends differently" % rep
        assert torch.equal(gi, T.sa_select(q, kc, k)), "replay %d differs from sa_select" % rep


# ------------------------------------------------------- index-guided offload

@pytest.mark.parametrize("dtype,d,B,Hkv,N,bs,n_blk,token_major", [
    ("bf16", 128, 2, 4, 4096, 128, 5, False), ("f32", 64, 1, 2, 2048, 64, 7, True),
    ("bf16", 64, 3, 2, 1000, 8, 60, False)])
def test_gather_blocks_from_pinned_host(dtype, d, B, Hkv, N, bs, n_blk, token_major):
    """Selected blocks copied from a pinned host cache are bit-exact; dense
    decode over them equals block-sparse decode of the device-resident cache
    and the oracle's attention over the blocks' tokens."""
    say("gather blocks %s d=%d B=%d Hkv=%d N=%d bs=%d n_blk=%d tm=%s" % (
        dtype, d, B, Hkv, N, bs, n_blk, token_major))
    G = 4
    q, kc, vc = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, N + bs)
    if token_major:   # [B, N, Hkv, d] storage seen as [B, Hkv, N, d]
        kc = kc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vc = vc.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    kh = torch.empty_strided(kc.shape, kc.stride(), dtype=kc.dtype, pin_memory=True)
    vh = torch.empty_strided(vc.shape, vc.stride(), dtype=vc.dtype, pin_memory=True)
    kh.copy_(kc)
    vh.copy_(vc)
    rng = np.random.default_rng(n_blk)
    nb = N // bs
    blocks = np.stack([rng.choice(nb, n_blk, replace=False) for _ in range(B * Hkv)])
    blocks = blocks.reshape(B, Hkv, n_blk).astype(np.int32)       # unsorted ids
    idx = torch.from_numpy(blocks).to(dev())
    ko, vo = T.sa_gather_blocks(kh, vh, idx, bs)
    qd, kd, vd = q.to(dev()), kc.to(dev()), vc.to(dev())
    dense = T.sa_dense_decode(qd, ko, vo)
    ref = T.sa_sparse_decode(qd, kd, vd, idx, T.SA_IDX_BLOCK_PER_KV_HEAD, block_size=bs)
    torch.cuda.synchronize()
    kg, vg = ko.cpu(), vo.cpu()
    for b in range(B):
        for r in range(Hkv):
            want_k = torch.cat([kc[b, r, j * bs:(j + 1) * bs] for j in blocks[b, r]])
            want_v = torch.cat([vc[b, r, j * bs:(j + 1) * bs] for j in blocks[b, r]])
            assert torch.equal(kg[b, r], want_k) and torch.equal(vg[b, r], want_v), (b, r)
    o, rf = dense.cpu().numpy(), ref.cpu().numpy()
    assert np.max(np.abs(o - rf)) <= 1e-5
    qf, kf, vf = _f64(q), _f64(kc), _f64(vc)
    scale = O.default_scale(d)
    for b in range(B):
        for r in range(Hkv):
            toks = O.block_tokens(blocks[b, r], bs, N)
            want = O.attend(qf[b, r * G:(r + 1) * G], kf[b, r], vf[b, r], toks, scale)
            check_out(o[b, r * G:(r + 1) * G], want, dtype, "offload %d,%d" % (b, r))


def test_gather_blocks_refuses_pageable_memory_and_clamps_ids():
    """The C call refuses host memory that is not pinned (nothing is
    launched), and clamps block ids outside the cache into it."""
    import ctypes
    from top_sparse_decode_sa_amd import _binding as Bn
    say("gather blocks: pageable memory refused; out-of-range ids clamped")
    B, Hkv, N, d, bs = 1, 2, 1024, 128, 128
    kc = torch.randn((B, Hkv, N, d)).to(torch.bfloat16)          # pageable
    ids = [[-3, 2, 8], [7, 100, 0]]
    idx = torch.tensor([ids], dtype=torch.int32, device=dev())
    out = torch.empty((B, Hkv, 3 * bs, d), dtype=torch.bfloat16, device=dev())
    desc = T.KVDesc(B, Hkv, Hkv, d, N, T.SA_BF16, T.SA_BF16, kc.stride(0), kc.stride(1),
                    kc.stride(2), 0.0)
    p = ctypes.c_void_p
    st = T.lib().sa_gather_blocks(ctypes.byref(desc), p(kc.data_ptr()), p(kc.data_ptr()),
                                  p(idx.data_ptr()), 3, bs, p(out.data_ptr()), p(out.data_ptr()),
                                  None)
    assert st == Bn.SA_ERR_MEMORY
    kh = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, pin_memory=True)
    kh.copy_(kc)
    ko, _ = T.sa_gather_blocks(kh, kh, idx, bs)
    torch.cuda.synchronize()
    kg = ko.cpu()
    nb = N // bs
    for r in range(Hkv):
        want = torch.cat([kc[0, r, min(max(j, 0), nb - 1) * bs:(min(max(j, 0), nb - 1) + 1) * bs]
                          for j in ids[r]])
        assert torch.equal(kg[0, r], want)


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 64 << 20])
def test_stream_read_covers_every_word(nbytes):
    """The streaming read folds every 32-bit word it loads and writes the
    fold only when it equals 0x9e3779b9; with one such word in a zero buffer
    the sink is written wherever the word sits (first, middle, last), so no
    part of the buffer goes unread, and a zero buffer leaves it alone."""
    say("stream read %d bytes" % nbytes)
    marker = np.uint32(0x9E3779B9).view(np.int32)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    T.sa_stream_read(buf, sink)
    assert int(sink.item()) == 0
    for w in sorted({0, nbytes // 8, nbytes // 4 - 1}):
        buf.zero_()
        buf[w] = int(marker)
        sink.zero_()
        T.sa_stream_read(buf, sink)
        assert int(sink.item()) == int(marker), w


@pytest.mark.parametrize("B,Hkv,N,k,kind,bs", [(16, 8, 32768, 655, T.SA_IDX_TOKEN_PER_KV_HEAD, 0),
                                                (1, 8, 100000, 2048, T.SA_IDX_TOKEN_SHARED, 0),
                                                (2, 2, 8192, 24, T.SA_IDX_BLOCK_PER_KV_HEAD, 128)])
def test_gather_read_reads_the_selected_rows(B, Hkv, N, k, kind, bs):
    """sa_gather_read folds every word of the selected key and value rows it
    loads: with zero caches, a 0x9e3779b9 word in a selected row (the first
    selected token of a row; any of the key's or the value's words) reaches
    the sink, and the same word in a row that is not selected does not."""
    say("gather read", B, Hkv, N, k, kind, bs)
    marker = int(np.uint32(0x9E3779B9).view(np.int32))
    G, d = 4, 128
    q = torch.zeros((B, Hkv * G, d), dtype=torch.bfloat16, device=dev())
    kc = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    rng = np.random.default_rng(N + k)
    nsel = N // bs if bs else N
    rows = B if kind == T.SA_IDX_TOKEN_SHARED else B * Hkv
    sel = np.stack([np.sort(rng.choice(np.arange(1, nsel), k, replace=False)) for _ in range(rows)])
    idx = torch.from_numpy(sel.astype(np.int32).reshape((B, k) if kind == T.SA_IDX_TOKEN_SHARED
                                                         else (B, Hkv, k))).to(dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    T.sa_gather_read(q, kc, vc, idx, sink, kind, bs)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    b, r = B - 1, Hkv - 1
    t = int(sel[b if kind == T.SA_IDX_TOKEN_SHARED else b * Hkv + r, 0]) * (bs or 1)
    for cache, word, tok in [(kc, 0, t), (kc, 63, t), (vc, 5, t), (vc, 60, t), (kc, 0, 0)]:
        kc.zero_()
        vc.zero_()
        cache.view(torch.int32)[b, r, tok, word] = marker
        sink.zero_()
        T.sa_gather_read(q, kc, vc, idx, sink, kind, bs)
        torch.cuda.synchronize()
        want = 0 if tok == 0 else marker   # token 0 is never selected
        assert int(sink.item()) == want, (word, tok)


@pytest.mark.parametrize("N,dtype,want_splits,want_sparse",
                         [(25677, "bf16", 101, 313), (51277, "bf16", 201, 313),
                          (153677, "bf16", 601, 313), (40000, "f32", 625, 625)])
def test_combine_across_split_counts(N, dtype, want_splits, want_sparse):
    """Few rows over a long context split into 101, 201, 601 and 625
    partials per row (the combine's 8-, 16- and 32-lane variants, the last
    two in two rounds of loads, each with a ragged last split); dense decode and a
    20000-token selection (bf16: 313 one-wave partials in the interleaved
    layout) against the oracle."""
    from top_sparse_decode_sa_amd import _binding as Bn
    import ctypes
    say("combine N=%d %s" % (N, dtype))
    B, Hkv, G, d = 1, 2, 4, 128
    q, k, v = _rand_cache(B, Hkv * G, Hkv, N, d, dtype, N)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    desc = Bn.make_desc(qd, kd)
    ws = int(T.lib().sa_dense_workspace_size(ctypes.byref(desc)))
    def padded(splits):  # partials [rows, nsplit, G, d + 2] fp32, in 256-byte units
        return -(-B * Hkv * splits * G * (d + 2) * 4 // 256) * 256

    assert ws == padded(want_splits)
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    scale = O.default_scale(d)
    dense = T.sa_dense_decode(qd, kd, vd).cpu().numpy()
    check_out(dense, _oracle_out(qf, kf, vf, [[np.arange(N)] * Hkv], G, scale), dtype, "dense")
    rng = np.random.default_rng(N + 1)
    sets = [np.sort(rng.choice(N, 20000, replace=False)).astype(np.int32) for _ in range(Hkv)]
    idx = torch.from_numpy(np.stack(sets)[None]).to(dev())
    ws_s = int(T.lib().sa_sparse_workspace_size(ctypes.byref(desc), T.SA_IDX_TOKEN_PER_KV_HEAD,
                                                20000, 0))
    assert ws_s == padded(want_sparse)
    sparse = T.sa_sparse_decode(qd, kd, vd, idx).cpu().numpy()
    check_out(sparse, _oracle_out(qf, kf, vf, [sets], G, scale), dtype, "sparse 20000")
