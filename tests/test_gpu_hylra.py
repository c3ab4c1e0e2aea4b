"""GPU parity of the layer-reuse path ("HyLRA", sections 2.2-2.3): full
attention that also hands on its top-k (sa_dense_decode_scored and the
DENSE_SELECT layer mode), the top-k overlap of two layers (sa_index_overlap),
the offline policy (sa_plan_reuse, checked against the oracle's exhaustive
search on the overlaps the GPU measured) and a whole 8-layer decode under that
policy, against the CPU oracle."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import sa_synth as S
import top_sparse_decode_sa_amd as T
from gpu_util import check_out, dev, say, score_tol, to_dev

pytestmark = pytest.mark.gpu


def _rand(B, Hq, Hkv, N, d, dtype, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(tdt)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(tdt)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, N, d)).astype(np.float32)).to(tdt)
    return q.to(dev()), k.to(dev()), v.to(dev())


def _f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


# The fused path (bf16, d 128, G <= 4; whole-row and split plans) and the
# two-launch path (fp32, d 64, G 8), with ragged context lengths.
@pytest.mark.parametrize("dtype,d,G,B,N", [
    ("bf16", 128, 4, 2, 5000), ("bf16", 128, 4, 40, 700), ("bf16", 128, 2, 1, 33),
    ("bf16", 128, 1, 3, 2049), ("f32", 64, 8, 2, 1500), ("bf16", 64, 4, 2, 999)])
def test_dense_decode_scored(dtype, d, G, B, N):
    say("dense scored %s d=%d G=%d B=%d N=%d" % (dtype, d, G, B, N))
    Hkv = 4
    q, k, v = _rand(B, Hkv * G, Hkv, N, d, dtype, N + G)
    out, scores = T.sa_dense_decode_scored(q, k, v)
    plain = T.sa_dense_decode(q, k, v)
    exact = T.sa_score(q, k)
    torch.cuda.synchronize()
    o, s, p, e = out.cpu().numpy(), scores.cpu().numpy(), plain.cpu().numpy(), exact.cpu().numpy()
    assert np.max(np.abs(o - p)) <= 1e-6, "scored and plain dense decode differ"
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    scale = O.default_scale(d)
    for b in range(B):
        for r in range(Hkv):
            qg = qf[b, r * G:(r + 1) * G]
            s64 = O.scores_exact(qg, kf[b, r], scale)
            assert np.max(np.abs(s[b, r] - s64)) <= score_tol(s64), ("scores", b, r)
            assert np.max(np.abs(e[b, r] - s64)) <= score_tol(s64)
            if b < 2:
                want = O.dense(qg, kf[b, r], vf[b, r], scale)
                check_out(o[b, r * G:(r + 1) * G], want, dtype, "dense scored %d,%d" % (b, r))


@pytest.mark.parametrize("rows,k,n", [(1, 1, 10), (37, 655, 32768), (5, 8192, 20000),
                                      (3, 9000, 30000), (64, 7, 7)])
def test_index_overlap(rows, k, n):
    """Bit-exact against the oracle's set intersection, including the rows
    staged in LDS (k <= 8192) and the rows searched in global memory."""
    say("overlap rows=%d k=%d n=%d" % (rows, k, n))
    rng = np.random.default_rng(rows * 7 + k)
    a = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(rows)]).astype(np.int32)
    b = np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(rows)]).astype(np.int32)
    b[0] = a[0]                       # identical sets
    if rows > 2 and k * 2 <= n:
        b[1] = np.sort(np.setdiff1d(np.arange(n), a[1])[:k])   # disjoint sets
    got = T.sa_index_overlap(torch.from_numpy(a).to(dev()), torch.from_numpy(b).to(dev()))
    got = got.cpu().numpy()
    want = np.array([O.index_overlap(a[r], b[r]) for r in range(rows)])
    assert np.array_equal(got, want)
    assert got[0] == k


def test_dense_select_layer_small():
    say("dense-select layer small")
    B, Hkv, G, N, d, k = 2, 4, 4, 3000, 128, 61
    q, kc, vc = _rand(B, Hkv * G, Hkv, N, d, "bf16", 17)
    args, out, d_ = T.layer_args(q, kc, vc, T.SA_SCORE_EXACT, k)
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev())
    T.sa_decode_layer(args, T.SA_LAYER_DENSE_SELECT, idx, d_)
    _, scores = T.sa_dense_decode_scored(q, kc, vc)
    idx2 = T.sa_topk(scores, k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    qf, kf, vf = _f64(q), _f64(kc), _f64(vc)
    scale = O.default_scale(d)
    o, ih = out.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        for r in range(Hkv):
            qg = qf[b, r * G:(r + 1) * G]
            v = O.index_set_verdict(O.scores_exact(qg, kf[b, r], scale), ih[b, r], k)
            assert not v.startswith("failed"), (b, r, v)
            check_out(o[b, r * G:(r + 1) * G], O.dense(qg, kf[b, r], vf[b, r], scale), "bf16",
                      "dense select %d,%d" % (b, r))


@pytest.mark.timeout(900)
def test_hylra32k_policy_end_to_end():
    """8 layers of the llama32k shape (4 sequences) with layer-correlated
    queries and keys: profile every layer as DENSE_SELECT, measure the
    overlap matrix on the GPU, plan with theta = 0.35, run the plan."""
    c = replace(S.CONFIGS["hylra32k"], batch=4)
    w = S.Workload(c, 0)
    L, rows_n, k = c.n_layers, c.batch * c.n_kv_heads, c.k
    scale = O.default_scale(c.head_dim)
    rows = [(0, 0), (1, 3), (3, 7)]
    qs, ks, vs, qh = [], [], [], []
    for l in range(L):
        say("hylra32k layer %d: generating" % l)
        q_h = w.q(l)
        qh.append(O.widen(q_h))
        qs.append(to_dev(q_h))
        ks.append(to_dev(w.k(l)))
        vs.append(to_dev(w.v(l)))
    # profiling pass: every layer full attention + its top-k
    idx = []
    krows = {}
    for l in range(L):
        say("hylra32k layer %d: dense-select" % l)
        args, out, d_ = T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_EXACT, k)
        il = torch.empty((c.batch, c.n_kv_heads, k), dtype=torch.int32, device=dev())
        T.sa_decode_layer(args, T.SA_LAYER_DENSE_SELECT, il, d_)
        torch.cuda.synchronize()
        idx.append(il)
        ih, oh = il.cpu().numpy(), out.cpu().numpy()
        for b, r in rows:
            kf, vf = O.widen(w.k_row(l, b, r)), O.widen(w.v_row(l, b, r))
            krows[(l, b, r)] = (kf, vf)
            qg = qh[l][b, r * c.group:(r + 1) * c.group]
            v = O.index_set_verdict(O.scores_exact(qg, kf, scale), ih[b, r], k)
            assert not v.startswith("failed"), (l, b, r, v)
            check_out(oh[b, r * c.group:(r + 1) * c.group], O.dense(qg, kf, vf, scale), "bf16",
                      "L%d dense %d,%d" % (l, b, r))
    # overlap matrix
    host = [i.cpu().numpy().reshape(rows_n, k) for i in idx]
    M = np.zeros((L, L), dtype=np.int64)
    for i in range(L):
        for j in range(i + 1, L):
            cnt = T.sa_index_overlap(idx[i], idx[j]).cpu().numpy().reshape(rows_n)
            want = np.array([O.index_overlap(host[i][r], host[j][r]) for r in range(rows_n)])
            assert np.array_equal(cnt, want), (i, j)
            M[i, j] = int(cnt.sum())
    total = rows_n * k
    say("overlap ratios:\n%s" % np.array2string(M / total, precision=2))
    modes, src = T.sa_plan_reuse(M, total, 0.35)
    assert (modes, src) == tuple(list(x) for x in O.reuse_plan_bruteforce(M, total, 0.35))
    T.sa_plan_validate(modes, src)
    assert modes[4] != T.SA_LAYER_REUSE, "the weakly correlated layer 4 must reset"
    assert sum(m != T.SA_LAYER_REUSE for m in modes) < L
    say("plan: modes %s src %s" % (modes, src))
    # decode under the plan
    held = {}
    for l in range(L):
        args, out, d_ = T.layer_args(qs[l], ks[l], vs[l], T.SA_SCORE_EXACT, k)
        if modes[l] == T.SA_LAYER_REUSE:
            il = held[src[l]]
        else:
            il = torch.empty((c.batch, c.n_kv_heads, k), dtype=torch.int32, device=dev())
        T.sa_decode_layer(args, modes[l], il if modes[l] != T.SA_LAYER_DENSE else None, d_)
        torch.cuda.synchronize()
        if modes[l] == T.SA_LAYER_DENSE_SELECT:
            assert torch.equal(il, idx[l]), "layer %d: the policy run selects differently" % l
            held[l] = il
        oh = out.cpu().numpy()
        for b, r in rows:
            kf, vf = krows[(l, b, r)]
            qg = qh[l][b, r * c.group:(r + 1) * c.group]
            if modes[l] == T.SA_LAYER_REUSE:
                want = O.attend(qg, kf, vf, host[src[l]].reshape(c.batch, c.n_kv_heads, k)[b, r], scale)
            else:
                want = O.dense(qg, kf, vf, scale)
            check_out(oh[b, r * c.group:(r + 1) * c.group], want, "bf16", "plan L%d %d,%d" % (l, b, r))
