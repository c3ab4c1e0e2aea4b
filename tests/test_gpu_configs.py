"""Full-size parity of the five decode workloads, run through the C ABI in the
launch configuration the benchmark times (sa_decode_layer / sa_score /
sa_topk / sa_sparse_decode / sa_dense_decode).

The caches are generated at their real sizes (up to 68.7 GB), uploaded and run
whole on the GPU.  The oracle then checks, on sampled (sequence, KV head)
rows it regenerates on the host:
  * selected index sets against its fp64 scores (exact outside the near-tie
    band, band rule inside; failures must be 0),
  * sa_topk bit-exactly against the oracle's top-k of the same fp32 scores,
  * attention outputs against oracle attention over the GPU's own set, and
    dense outputs against oracle dense attention (fp32: max-abs 1e-5; bf16:
    max-abs 1e-2 and mean-abs 1e-3),
plus properties that hold at any size (planted keys selected, reused index
sets byte-identical to their source layer).
"""
import numpy as np
import pytest
import torch

import oracle as O
import sa_synth as S
import top_sparse_decode_sa_amd as T
from gpu_util import check_out, dev, say, score_tol, to_dev

pytestmark = pytest.mark.gpu


def _upload_cache(w, which, layer, chunk=8):
    """Generate a [B, Hkv, N, d] cache in batch slices straight into device memory."""
    c = w.cfg
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    out = torch.empty((c.batch, c.n_kv_heads, c.ctx_len, c.head_dim), dtype=tdt, device=dev())
    for b0 in range(0, c.batch, chunk):
        b1 = min(c.batch, b0 + chunk)
        host = w.k(layer, batch=(b0, b1)) if which == "k" else w.v(layer, batch=(b0, b1))
        t = torch.from_numpy(host)
        out[b0:b1].copy_(t.view(torch.bfloat16) if t.dtype == torch.uint16 else t)
        del host, t
    return out


def _sample_rows(c, n, seed=0):
    rng = np.random.default_rng(1000 + seed)
    rows = {(0, 0), (c.batch - 1, c.n_kv_heads - 1)}
    while len(rows) < min(n, c.batch * c.n_kv_heads):
        rows.add((int(rng.integers(c.batch)), int(rng.integers(c.n_kv_heads))))
    return sorted(rows)


def _report(capsys, msg):
    """A summary line that shows in the test log even when output is captured."""
    say(msg)
    if capsys is not None:
        with capsys.disabled():
            print("\n" + msg, flush=True)


def _check_exact_layer(w, layer, qd, kd, vd, rows, label, capsys=None):
    """SPARSE layer with exact scoring: decode_layer == score+topk+sparse, and
    every sampled row against the oracle."""
    c = w.cfg
    scale = O.default_scale(c.head_dim)
    args, out, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_EXACT, c.k)
    idx = torch.empty((c.batch, c.n_kv_heads, c.k), dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_)
    scores = T.sa_score(qd, kd)
    idx2 = T.sa_topk(scores, c.k)
    out2 = T.sa_sparse_decode(qd, kd, vd, idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "%s: layer entry point and single calls select differently" % label
    assert torch.equal(out, out2), "%s: layer entry point and single calls differ" % label
    assert T.sa_check_indices(qd, kd, idx).tolist() == [0, 0], label
    idx_h = idx.cpu().numpy()
    out_h = out.cpu().numpy()
    q_h = O.widen(qd.cpu().view(torch.uint16).numpy() if c.dtype == "bf16" else qd.cpu().numpy())
    # sa_topk bit-exact on the GPU's own fp32 scores, every row
    s_gpu = scores.cpu().numpy()
    for b in range(c.batch):
        for r in range(c.n_kv_heads):
            assert np.array_equal(idx_h[b, r], O.topk(s_gpu[b, r].astype(np.float64), c.k)), (label, b, r)
            if c.planting == "direction":
                assert set(w.planted(layer, b, r)).issubset(idx_h[b, r]), (label, "planted", b, r)
    counts = {"exact": 0, "excused": 0}
    worst = 0.0
    for b, r in rows:
        qg = q_h[b, r * c.group:(r + 1) * c.group]
        kf = O.widen(w.k_row(layer, b, r))
        vf = O.widen(w.v_row(layer, b, r))
        s64 = O.scores_exact(qg, kf, scale)
        assert np.max(np.abs(s_gpu[b, r] - s64)) <= score_tol(s64), (label, "scores", b, r)
        v = O.index_set_verdict(s64, idx_h[b, r], c.k)
        assert not v.startswith("failed"), (label, b, r, v)
        counts[v] += 1
        want = O.attend(qg, kf, vf, idx_h[b, r], scale)
        mx, _ = check_out(out_h[b, r * c.group:(r + 1) * c.group], want, c.dtype, "%s row %d,%d" % (label, b, r))
        worst = max(worst, mx)
    _report(capsys, "%s: %d/%d checked rows exact or excused %s (of %d rows); worst output "
                    "error %.2e" % (label, counts["exact"] + counts["excused"], len(rows), counts,
                                    c.batch * c.n_kv_heads, worst))
    return idx, out


def _check_dense(w, layer, qd, kd, vd, rows, label):
    c = w.cfg
    scale = O.default_scale(c.head_dim)
    args, out, d_ = T.layer_args(qd, kd, vd)
    T.sa_decode_layer(args, T.SA_LAYER_DENSE, None, d_)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()
    q_h = O.widen(qd.cpu().view(torch.uint16).numpy() if c.dtype == "bf16" else qd.cpu().numpy())
    for b, r in rows:
        qg = q_h[b, r * c.group:(r + 1) * c.group]
        want = O.dense(qg, O.widen(w.k_row(layer, b, r)), O.widen(w.v_row(layer, b, r)), scale)
        check_out(out_h[b, r * c.group:(r + 1) * c.group], want, c.dtype, "%s dense %d,%d" % (label, b, r))
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("seed", [0, 1])
def test_llama32k_exact_topk_at_50x(seed, capsys):
    """Batch 16, 32/8 heads, d 128, bf16 32K cache, k = 655 (50x)."""
    w = S.Workload("llama32k", seed)
    c = w.cfg
    say("llama32k seed %d: generating %.2f GB" % (seed, c.kv_bytes() / 1e9))
    kd, vd = _upload_cache(w, "k", 0), _upload_cache(w, "v", 0)
    qd = to_dev(w.q(0))
    # seed 0: every (sequence, KV head) row against the oracle
    rows = _sample_rows(c, c.batch * c.n_kv_heads if seed == 0 else 12, seed)
    _check_exact_layer(w, 0, qd, kd, vd, rows, "llama32k/%d" % seed, capsys)
    _check_dense(w, 0, qd, kd, vd, rows[:4], "llama32k/%d" % seed)
    if seed == 0:
        _check_per_q_head(w, qd, kd, vd, rows[:4], "llama32k/%d per-q-head" % seed)


def _check_per_q_head(w, qd, kd, vd, rows, label):
    """The same cache with one selection per query head (512 rows of 655):
    sa_topk bit-exact on the GPU's scores for every row, and on sampled
    (sequence, KV head) rows every grouped head's scores, set and output
    against the oracle."""
    c = w.cfg
    scale = O.default_scale(c.head_dim)
    args, out, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_EXACT_PER_Q_HEAD, c.k)
    idx = torch.empty((c.batch, c.n_q_heads, c.k), dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_)
    scores = T.sa_score(qd, kd, T.SA_SCORE_EXACT_PER_Q_HEAD)
    assert T.sa_check_indices(qd, kd, idx, T.SA_IDX_TOKEN_PER_Q_HEAD).tolist() == [0, 0]
    torch.cuda.synchronize()
    idx_h, out_h, s_gpu = idx.cpu().numpy(), out.cpu().numpy(), scores.cpu().numpy()
    for b in range(c.batch):
        for h in range(c.n_q_heads):
            assert np.array_equal(idx_h[b, h], O.topk(s_gpu[b, h].astype(np.float64), c.k)), (b, h)
    q_h = O.widen(qd.cpu().view(torch.uint16).numpy())
    counts = {"exact": 0, "excused": 0}
    for b, r in rows:
        kf = O.widen(w.k_row(0, b, r))
        vf = O.widen(w.v_row(0, b, r))
        for h in range(r * c.group, (r + 1) * c.group):
            s64 = O.scores_per_query_head(q_h[b, h], kf, scale)
            assert np.max(np.abs(s_gpu[b, h] - s64)) <= score_tol(s64), (label, b, h)
            v = O.index_set_verdict(s64, idx_h[b, h], c.k)
            assert not v.startswith("failed"), (label, b, h, v)
            counts[v] += 1
            want = O.attend(q_h[b, h][None], kf, vf, idx_h[b, h], scale)
            check_out(out_h[b, h][None], want, c.dtype, "%s %d,%d" % (label, b, h))
    say("%s: index sets %s" % (label, counts))


@pytest.mark.timeout(600)
def test_block61k_block_selection_and_reuse():
    """Batch 8, 61440 tokens in 480 blocks of 128, top 24 blocks chosen at
    layer 0 from min/max summaries and reused unchanged at layers 1-3;
    layer 0 also run dense."""
    w = S.Workload("block61k", 0)
    c = w.cfg
    bs = c.block_size
    nb = (c.ctx_len + bs - 1) // bs
    rows = _sample_rows(c, 6)
    scale = O.default_scale(c.head_dim)
    modes = [T.SA_LAYER_SPARSE, T.SA_LAYER_REUSE, T.SA_LAYER_REUSE, T.SA_LAYER_REUSE]
    T.sa_plan_validate(modes, list(c.src))
    idx = torch.full((c.batch, c.n_kv_heads, c.k), -1, dtype=torch.int32, device=dev())
    idx_src = None
    counts = {"exact": 0, "excused": 0}
    for layer in range(c.n_layers):
        say("block61k layer %d: generating" % layer)
        kd, vd = _upload_cache(w, "k", layer), _upload_cache(w, "v", layer)
        qd = to_dev(w.q(layer))
        q_h = O.widen(w.q(layer))
        kmin, kmax = T.sa_block_summarize(kd, bs, q_like=qd)
        args, out, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_BLOCK_MINMAX, c.k, kmin=kmin, kmax=kmax,
                                     block_size=bs)
        T.sa_decode_layer(args, modes[layer], idx, d_)
        assert T.sa_check_indices(qd, kd, idx, T.SA_IDX_BLOCK_PER_KV_HEAD, bs).tolist() == [0, 0]
        torch.cuda.synchronize()
        idx_h = idx.cpu().numpy()
        if layer == 0:
            idx_src = idx_h.copy()
            sb = T.sa_score(qd, kd, T.SA_SCORE_BLOCK_MINMAX, kmin=kmin, kmax=kmax, block_size=bs).cpu().numpy()
            assert np.array_equal(idx_h, np.stack([[O.topk(sb[b, r].astype(np.float64), c.k)
                                                    for r in range(c.n_kv_heads)] for b in range(c.batch)]))
        else:
            # reuse: the index buffer the layer attended over is byte-identical
            assert np.array_equal(idx_h, idx_src)
        out_h = out.cpu().numpy()
        mn_h, mx_h = kmin.cpu().to(torch.float64).numpy(), kmax.cpu().to(torch.float64).numpy()
        for b, r in rows:
            qg = q_h[b, r * c.group:(r + 1) * c.group]
            kf = O.widen(w.k_row(layer, b, r))
            mn, mx = O.block_summaries(kf, bs)
            assert np.array_equal(mn_h[b, r], mn) and np.array_equal(mx_h[b, r], mx), ("summaries", layer, b, r)
            if layer == 0:
                s64 = O.scores_block(qg, mn, mx)
                v = O.index_set_verdict(s64, idx_h[b, r], c.k)
                assert not v.startswith("failed"), (b, r, v)
                counts[v] += 1
            toks = O.block_tokens(idx_h[b, r], bs, c.ctx_len)
            assert len(toks) == c.k * bs and idx_h[b, r].max() < nb
            want = O.attend(qg, kf, O.widen(w.v_row(layer, b, r)), toks, scale)
            check_out(out_h[b, r * c.group:(r + 1) * c.group], want, "bf16", "block61k L%d %d,%d" % (layer, b, r))
        if layer == 0:
            _check_dense(w, 0, qd, kd, vd, rows[:3], "block61k L0")
        if layer == 1:
            # index-guided offload: the same layer with its cache in pinned
            # host memory; only the 24 reused blocks per row cross the host
            # link, and attention over them equals the device-resident reuse
            kh = torch.empty(kd.shape, dtype=kd.dtype, pin_memory=True)
            vh = torch.empty(vd.shape, dtype=vd.dtype, pin_memory=True)
            kh.copy_(kd)
            vh.copy_(vd)
            ko, vo = T.sa_gather_blocks(kh, vh, idx, bs)
            off = T.sa_dense_decode(qd, ko, vo)
            torch.cuda.synchronize()
            assert ko.shape == (c.batch, c.n_kv_heads, c.k * bs, c.head_dim)
            assert np.max(np.abs(off.cpu().numpy() - out_h)) <= 1e-5, "offload differs from reuse"
            for b, r in rows[:2]:
                toks = torch.from_numpy(O.block_tokens(idx_h[b, r], bs, c.ctx_len))
                assert torch.equal(ko[b, r].cpu(), kh[b, r][toks]), ("offload K", b, r)
                assert torch.equal(vo[b, r].cpu(), vh[b, r][toks]), ("offload V", b, r)
            say("block61k L1: offload gather of %d blocks per row equals the reuse decode" % c.k)
            del kh, vh, ko, vo
        del kd, vd, kmin, kmax
        torch.cuda.empty_cache()
    say("block61k: layer-0 block sets %s over %d sampled rows; layers 1-3 reused them" % (counts, len(rows)))


@pytest.mark.timeout(900)
def test_batch128k_exact_topk_at_500x(capsys):
    """Batch 128, 131072 tokens (68.7 GB of KV), k = 262 (500x): the top-262 is
    exactly the planted set; dense decode on the same cache."""
    w = S.Workload("batch128k", 0)
    c = w.cfg
    say("batch128k: generating %.1f GB" % (c.kv_bytes() / 1e9))
    kd = _upload_cache(w, "k", 0, chunk=4)
    vd = _upload_cache(w, "v", 0, chunk=4)
    qd = to_dev(w.q(0))
    rows = _sample_rows(c, 32)
    idx, _ = _check_exact_layer(w, 0, qd, kd, vd, rows, "batch128k", capsys)
    idx_h = idx.cpu().numpy()
    for b in range(c.batch):
        for r in range(c.n_kv_heads):
            assert np.array_equal(idx_h[b, r], w.planted(0, b, r))
    _check_dense(w, 0, qd, kd, vd, rows[:2], "batch128k")


@pytest.mark.timeout(900)
def test_indexer1m_mixed_plan(capsys):
    """One 1M-token sequence, 8 layers: dense at layers 0-1, then indexer
    top-2048 shared by the 8 KV heads at layers 2-7."""
    w = S.Workload("indexer1m", 0)
    c = w.cfg
    modes = [T.SA_LAYER_DENSE if m == "dense" else T.SA_LAYER_SPARSE for m in c.modes]
    T.sa_plan_validate(modes, list(c.src))
    scale = O.default_scale(c.head_dim)
    counts = {"exact": 0, "excused": 0}
    for layer in range(c.n_layers):
        say("indexer1m layer %d (%s): generating" % (layer, c.modes[layer]))
        k_h = w.k(layer)
        kd = to_dev(k_h)
        vd = _upload_cache(w, "v", layer)
        q_h = w.q(layer)
        qd = to_dev(q_h)
        qf = O.widen(q_h)
        if modes[layer] == T.SA_LAYER_DENSE:
            _check_dense(w, layer, qd, kd, vd, [(0, 0), (0, c.n_kv_heads - 1)], "indexer1m L%d" % layer)
        else:
            qi_h, ki_h, wi_h = w.indexer_q(layer, q_h), w.indexer_k(layer, k_h), w.indexer_w(layer)
            qi, ki = to_dev(qi_h), to_dev(ki_h)
            wi = torch.from_numpy(wi_h[None, :].copy()).to(dev())
            args, out, d_ = T.layer_args(qd, kd, vd, T.SA_SCORE_INDEXER, c.k, q_idx=qi, k_idx=ki, idx_w=wi)
            idx = torch.empty((c.batch, c.k), dtype=torch.int32, device=dev())
            T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_)
            si = T.sa_score(qd, kd, T.SA_SCORE_INDEXER, q_idx=qi, k_idx=ki, idx_w=wi).cpu().numpy()[0]
            assert T.sa_check_indices(qd, kd, idx, T.SA_IDX_TOKEN_SHARED).tolist() == [0, 0]
            torch.cuda.synchronize()
            idx_h = idx.cpu().numpy()[0]
            assert np.array_equal(idx_h, O.topk(si.astype(np.float64), c.k))
            s64 = O.scores_indexer(O.widen(qi_h[0]), O.widen(ki_h[0]), wi_h.astype(np.float64))
            assert np.max(np.abs(si - s64)) <= score_tol(s64)
            v = O.index_set_verdict(s64, idx_h, c.k)
            assert not v.startswith("failed"), (layer, v)
            counts[v] += 1
            out_h = out.cpu().numpy()
            sel = np.sort(idx_h)
            # every KV head on the first sparse layer, the first and last on the others
            heads = range(c.n_kv_heads) if layer == 2 else [0, c.n_kv_heads - 1]
            for r in heads:
                qg = qf[0, r * c.group:(r + 1) * c.group]
                # only the selected rows are widened; attention over them is the same
                want = O.attend(qg, O.widen(k_h[0, r][sel]), O.widen(w.kv_tokens("v", layer, 0, r, sel)),
                                np.arange(c.k), scale)
                check_out(out_h[0, r * c.group:(r + 1) * c.group], want, "bf16", "indexer1m L%d head %d" % (layer, r))
        del kd, vd, k_h
        torch.cuda.empty_cache()
    _report(capsys, "indexer1m: sparse-layer index sets %s over the 6 sparse layers; outputs "
                    "of all 8 KV heads at layer 2, heads 0 and 7 elsewhere" % counts)


def test_split_counts_agree():
    """The same selection decoded with different split counts -- one sequence
    versus the sequence repeated 64 times, which changes the planned chunking
    (41 splits per row vs one whole-row workgroup sparse, 16 vs 2 splits
    dense) -- agrees within fp32
    rounding: the split-K log-sum-exp combine gives the same result."""
    say("split invariance")
    rng = np.random.default_rng(5)
    B, Hkv, G, N, d, k = 1, 8, 4, 4096, 128, 655
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(torch.bfloat16).to(dev())
    kc = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(torch.bfloat16).to(dev())
    vc = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(torch.bfloat16).to(dev())
    idx = T.sa_topk(T.sa_score(q, kc), k)
    one = T.sa_sparse_decode(q, kc, vc, idx).cpu().numpy()
    rep = 64
    qr, kr, vr = (x.repeat(rep, *([1] * (x.dim() - 1))).contiguous() for x in (q, kc, vc))
    many = T.sa_sparse_decode(qr, kr, vr, idx.repeat(rep, 1, 1).contiguous()).cpu().numpy()
    assert np.max(np.abs(many - one)) <= 1e-5
    dense_one = T.sa_dense_decode(q, kc, vc).cpu().numpy()
    dense_many = T.sa_dense_decode(qr, kr, vr).cpu().numpy()
    assert np.max(np.abs(dense_many - dense_one)) <= 1e-5
