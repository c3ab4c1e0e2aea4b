"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to something independent of its code:
exhaustive search, closed forms, a library attention routine, invariants the
pages state, values the pages print (``tests/golden``), or properties the
seeded constructions guarantee.  A plausible slip in the oracle (a dropped
term, a wrong sign, a swapped index, a wrong group) fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import sa_synth as S

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------

def _brute_topk(scores_int, k):
    """Maximum-sum k-subset; among equal sums the lexicographically smallest
    sorted index vector (ties toward lower indices)."""
    n = len(scores_int)
    best, best_sum = None, None
    for comb in itertools.combinations(range(n), k):  # lexicographic order
        s = sum(scores_int[i] for i in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    return np.array(best, dtype=np.int32)


@pytest.mark.parametrize("n", [1, 2, 5, 8, 10])
def test_topk_matches_exhaustive_search(n):
    for trial in range(40):
        vals = RNG.integers(-3, 4, size=n)  # small range -> many ties
        for k in range(1, n + 1):
            got = O.topk(vals.astype(np.float64), k)
            assert np.array_equal(got, _brute_topk(list(vals), k)), (vals, k)


def test_topk_ties_signed_zero_nan():
    s = np.array([-0.0, 0.0, -1.0, 0.0, np.nan, 2.0])
    assert O.topk(s, 1).tolist() == [5]
    assert O.topk(s, 2).tolist() == [0, 5]          # -0.0 ties +0.0 -> lower index
    assert O.topk(s, 4).tolist() == [0, 1, 3, 5]
    assert O.topk(s, 5).tolist() == [0, 1, 2, 3, 5]  # NaN ranks below -1.0
    assert O.topk(s, 6).tolist() == [0, 1, 2, 3, 4, 5]
    assert O.topk(np.full(7, 3.5), 3).tolist() == [0, 1, 2]
    with pytest.raises(ValueError):
        O.topk(s, 0)
    with pytest.raises(ValueError):
        O.topk(s, 7)


def test_topk_on_recency_is_sliding_window(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "sliding_window_w4.json")))
    n, w = g["n_tokens"], g["window"]
    recency = np.arange(n, dtype=np.float64)           # newer token, higher score
    assert (O.topk(recency, w) + 1).tolist() == g["window_tokens_1based"]
    assert (O.topk(recency, n) + 1).tolist() == g["full_tokens_1based"]
    for n, w in [(1024, 64), (32768, 655)]:
        assert np.array_equal(O.topk(np.arange(n, dtype=np.float64), w), np.arange(n - w, n))


# ---------------------------------------------------------------------------
# attention over a selected set
# ---------------------------------------------------------------------------

def _rand(*shape):
    return RNG.standard_normal(shape)


def test_attend_closed_forms():
    d, n = 16, 50
    scale = O.default_scale(d)
    q = _rand(3, d)
    v = _rand(n, d)
    sel = np.array([3, 7, 11, 40])
    # all selected keys equal -> uniform weights -> mean of V over S
    k_eq = np.tile(_rand(1, d), (n, 1))
    np.testing.assert_allclose(O.attend(q, k_eq, v, sel, scale), np.tile(v[sel].mean(0), (3, 1)),
                               rtol=0, atol=1e-13)
    # q = 0 -> uniform weights as well
    k = _rand(n, d)
    np.testing.assert_allclose(O.attend(np.zeros((2, d)), k, v, sel, scale),
                               np.tile(v[sel].mean(0), (2, 1)), rtol=0, atol=1e-13)
    # V constant -> the constant
    c = _rand(d)
    np.testing.assert_allclose(O.attend(q, k, np.tile(c, (n, 1)), sel, scale), np.tile(c, (3, 1)),
                               rtol=0, atol=1e-13)
    # one selected token -> its value row
    np.testing.assert_allclose(O.attend(q, k, v, [17], scale), np.tile(v[17], (3, 1)), atol=1e-15)
    # two tokens -> sigmoid mixture
    a, b = 5, 9
    for g in range(3):
        la = q[g] @ k[a] * scale
        lb = q[g] @ k[b] * scale
        sa = 1.0 / (1.0 + math.exp(lb - la))
        want = sa * v[a] + (1.0 - sa) * v[b]
        np.testing.assert_allclose(O.attend(q[g:g + 1], k, v, [a, b], scale)[0], want, atol=1e-13)


def test_attend_large_logits_are_stable():
    d = 8
    k = np.zeros((4, d))
    k[2, 0] = 1.0
    q = np.zeros((1, d))
    q[0, 0] = 5000.0  # logit 5000 for token 2, 0 for the rest
    v = np.eye(4, d)
    out = O.attend(q, k, v, [0, 1, 2, 3], 1.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0], v[2], atol=1e-300)


def test_attend_set_order_does_not_matter():
    d, n = 32, 200
    q, k, v = _rand(4, d), _rand(n, d), _rand(n, d)
    sel = RNG.choice(n, 37, replace=False)
    a = O.attend(q, k, v, sel, 0.3)
    b = O.attend(q, k, v, np.sort(sel), 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_attend_split_logsumexp_identity():
    """Attention over S equals the log-sum-exp merge of attention over a split
    of S (the tiling identity behind split-K decoding)."""
    d, n = 64, 300
    q, k, v = _rand(4, d) * 3, _rand(n, d), _rand(n, d)
    sel = np.sort(RNG.choice(n, 120, replace=False))
    o, lse = O.attend_lse(q, k, v, sel, 0.125)
    parts = [sel[:1], sel[1:50], sel[50:]]
    res = [O.attend_lse(q, k, v, p, 0.125) for p in parts]
    m = np.max([r[1] for r in res], axis=0)
    wts = [np.exp(r[1] - m) for r in res]
    merged = sum(w[:, None] * r[0] for w, r in zip(wts, res)) / sum(wts)[:, None]
    np.testing.assert_allclose(merged, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(m + np.log(sum(wts)), lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("g_size,d,n", [(1, 64, 97), (4, 128, 300), (4, 64, 1024)])
def test_dense_matches_library_attention(g_size, d, n):
    """Dense decode equals torch's scaled_dot_product_attention (float64, CPU),
    whose default scale is 1/sqrt(d)."""
    q, k, v = _rand(g_size, d), _rand(n, d), _rand(n, d)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(np.tile(k, (g_size, 1, 1)))[None],
        torch.from_numpy(np.tile(v, (g_size, 1, 1)))[None])[0, :, 0, :].numpy()
    np.testing.assert_allclose(O.dense(q, k, v, O.default_scale(d)), want, rtol=0, atol=1e-12)


def test_sparse_with_all_tokens_equals_dense():
    d, n = 64, 257
    q, k, v = _rand(4, d), _rand(n, d), _rand(n, d)
    np.testing.assert_array_equal(O.attend(q, k, v, O.topk(RNG.standard_normal(n), n), 0.125),
                                  O.dense(q, k, v, 0.125))


def test_window_attention_is_dense_attention_on_the_window():
    d, n, w = 32, 120, 16
    q, k, v = _rand(4, d), _rand(n, d), _rand(n, d)
    sel = O.topk(np.arange(n, dtype=np.float64), w)
    np.testing.assert_allclose(O.attend(q, k, v, sel, 0.2), O.dense(q, k[-w:], v[-w:], 0.2),
                               rtol=0, atol=1e-14)


def test_attend_traffic_is_linear_in_k_and_flat_in_n():
    for n in (1024, 32768, 1 << 20):
        assert O.attend_bytes(655, 128, 2) == 655 * 128 * 2 * 2
    assert O.attend_bytes(1310, 128, 2) == 2 * O.attend_bytes(655, 128, 2)


# ---------------------------------------------------------------------------
# exact scores
# ---------------------------------------------------------------------------

def test_scores_exact_are_attention_logits():
    """For one query head, softmax(scores) is the attention distribution, so
    attending a one-hot value table through the library routine recovers the
    scores up to a constant."""
    d, n = 64, 80
    q, k = _rand(1, d), _rand(n, d)
    probs = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k)[None, None],
        torch.eye(n, dtype=torch.float64)[None, None])[0, 0, 0].numpy()
    s = O.scores_exact(q, k, O.default_scale(d))
    np.testing.assert_allclose(np.log(probs) - np.log(probs[0]), s - s[0], rtol=0, atol=1e-10)


def test_scores_exact_basis_keys_and_group_sum():
    d = 16
    q = _rand(4, d)
    basis = np.eye(d)
    s = O.scores_exact(q, basis, 0.5)
    np.testing.assert_allclose(s, 0.5 * q.sum(axis=0), rtol=0, atol=1e-15)
    # one query head alone, and a group of identical heads scales by G
    np.testing.assert_allclose(O.scores_exact(np.tile(q[:1], (4, 1)), basis, 1.0), 4 * q[0],
                               atol=1e-14)


def test_planted_keys_rank_first_tiny():
    """The 1024-token fp32 workload plants 16 keys per KV head along its group's
    mean query; exact scoring must put all of them in the top 64."""
    w = S.Workload("tiny", 0)
    c = w.cfg
    q, k = O.widen(w.q()), O.widen(w.k())
    for r in range(c.n_kv_heads):
        s = O.scores_exact(q[0, r * c.group:(r + 1) * c.group], k[0, r], O.default_scale(c.head_dim))
        sel = O.topk(s, c.k)
        assert set(w.planted(0, 0, r)).issubset(sel)
        # and the planted keys are exactly the top 16
        assert np.array_equal(O.topk(s, c.n_planted), w.planted(0, 0, r))


@pytest.mark.parametrize("name,rows", [("llama32k", [(0, 0), (15, 7)]), ("batch128k", [(3, 5)])])
def test_planted_keys_rank_first_full_size(name, rows):
    """At full context length: 327 planted keys lie inside the top-655
    (50x sparsity), and at 500x the top-262 IS the planted set."""
    w = S.Workload(name, 0)
    c = w.cfg
    q = O.widen(w.q())
    for b, r in rows:
        s = O.scores_exact(q[b, r * c.group:(r + 1) * c.group], O.widen(w.k_row(0, b, r)),
                           O.default_scale(c.head_dim))
        sel = O.topk(s, c.k)
        pl = w.planted(0, b, r)
        assert len(pl) == c.n_planted
        assert set(pl).issubset(sel)
        if c.n_planted == c.k:
            assert np.array_equal(sel, pl)
        assert O.index_set_verdict(s, sel, c.k) in ("exact", "excused")


# ---------------------------------------------------------------------------
# block summaries and block scores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,bs", [(1024, 128), (1000, 128), (37, 8)])
def test_block_summaries_bound_every_key(n, bs):
    d = 32
    k = _rand(n, d)
    kmin, kmax = O.block_summaries(k, bs)
    nb = (n + bs - 1) // bs
    assert kmin.shape == (nb, d)
    for j in range(nb):
        blk = k[j * bs:min(n, (j + 1) * bs)]
        assert np.all(kmin[j] <= blk) and np.all(blk <= kmax[j])
        # attained: every dimension's bound is some key's value
        assert np.all(np.any(blk == kmin[j], axis=0)) and np.all(np.any(blk == kmax[j], axis=0))
    q = _rand(4, d)
    sb = O.scores_block(q, kmin, kmax)
    for j in range(nb):
        blk = k[j * bs:min(n, (j + 1) * bs)]
        for g in range(4):
            per_q = O.scores_block(q[g:g + 1], kmin[j:j + 1], kmax[j:j + 1])[0]
            assert np.all(blk @ q[g] <= per_q + 1e-12)        # upper bound per query
        assert np.all(O.scores_exact(q, blk, 1.0) <= sb[j] + 1e-12)  # and for the group sum


def test_block_score_of_single_token_blocks_is_exact():
    d, n = 16, 40
    q, k = _rand(4, d), _rand(n, d)
    kmin, kmax = O.block_summaries(k, 1)
    np.testing.assert_allclose(O.scores_block(q, kmin, kmax), O.scores_exact(q, k, 1.0), atol=1e-12)
    assert np.array_equal(O.block_tokens(np.array([2, 0]), 128, 300),
                          np.r_[np.arange(0, 128), np.arange(256, 300)])


# ---------------------------------------------------------------------------
# indexer scores
# ---------------------------------------------------------------------------

def test_indexer_single_head_basis_query():
    n, di = 500, 64
    kidx = _rand(n, di)
    qidx = np.zeros((4, di))
    qidx[0, 5] = 1.0
    qidx[1:] = _rand(3, di)
    si = O.scores_indexer(qidx, kidx, np.array([1.0, 0.0, 0.0, 0.0]))
    np.testing.assert_array_equal(si, np.maximum(0.0, kidx[:, 5]))
    w = np.array([0.25, 0.5, 0.0, 2.0])
    one_hot = [O.scores_indexer(qidx[h:h + 1], kidx, np.ones(1)) for h in range(4)]
    np.testing.assert_allclose(O.scores_indexer(qidx, kidx, w), sum(w[h] * one_hot[h] for h in range(4)),
                               atol=1e-12)


def test_indexer_all_negative_dots_select_the_first_k():
    n, di = 300, 64
    kidx = np.abs(_rand(n, di))
    qidx = -np.abs(_rand(4, di))
    si = O.scores_indexer(qidx, kidx, RNG.uniform(size=4))
    assert np.all(si == 0.0)
    assert np.array_equal(O.topk(si, 17), np.arange(17))


# ---------------------------------------------------------------------------
# per-layer plan and reuse
# ---------------------------------------------------------------------------

def test_plan_reuse_passes_indices_unchanged():
    d, n, k = 16, 64, 8
    layers = [(_rand(4, d), _rand(n, d), _rand(n, d)) for _ in range(4)]
    modes = [O.SPARSE, O.REUSE, O.DENSE, O.REUSE]
    src = [-1, 0, -1, 1]
    outs, idxs = O.run_plan(modes, src, k,
                            lambda l: O.scores_exact(layers[l][0], layers[l][1], 0.25),
                            lambda l, i: O.attend(*layers[l], i, 0.25),
                            lambda l: O.dense(*layers[l], 0.25))
    assert idxs[1] is idxs[0] and idxs[3] is idxs[0] and idxs[2] is None
    np.testing.assert_array_equal(idxs[0], O.topk(O.scores_exact(layers[0][0], layers[0][1], 0.25), k))
    np.testing.assert_array_equal(outs[3], O.attend(*layers[3], idxs[0], 0.25))
    np.testing.assert_array_equal(outs[2], O.dense(*layers[2], 0.25))


def test_plan_check_rejects_bad_plans():
    assert O.plan_check([O.SPARSE, O.REUSE], [-1, 0]) is None
    assert O.plan_check([O.DENSE, O.DENSE] + [O.SPARSE] * 6, [-1] * 8) is None
    assert O.plan_check([O.REUSE], [0]) is not None          # no earlier layer
    assert O.plan_check([O.SPARSE, O.REUSE], [-1, 1]) is not None
    assert O.plan_check([O.DENSE, O.REUSE], [-1, 0]) is not None  # dense owns no set
    assert O.plan_check([O.SPARSE, 7], [-1, -1]) is not None


def test_plan_dense_select_hands_its_topk_on():
    d, n, k = 16, 64, 8
    layers = [(_rand(4, d), _rand(n, d), _rand(n, d)) for _ in range(3)]
    outs, idxs = O.run_plan([O.DENSE_SELECT, O.REUSE, O.REUSE], [-1, 0, 0], k,
                            lambda l: O.scores_exact(layers[l][0], layers[l][1], 0.25),
                            lambda l, i: O.attend(*layers[l], i, 0.25),
                            lambda l: O.dense(*layers[l], 0.25))
    np.testing.assert_array_equal(outs[0], O.dense(*layers[0], 0.25))
    np.testing.assert_array_equal(idxs[0], O.topk(O.scores_exact(layers[0][0], layers[0][1], 0.25), k))
    assert idxs[1] is idxs[0] and idxs[2] is idxs[0]
    assert O.plan_check([O.DENSE_SELECT, O.REUSE], [-1, 0]) is None


def test_per_query_head_scores():
    # basis query: the score is the matching key coordinate times the scale
    k = _rand(9, 8)
    q = np.zeros(8)
    q[3] = 2.0
    np.testing.assert_allclose(O.scores_per_query_head(q, k, 0.5), k[:, 3], rtol=0, atol=1e-15)
    # a group of G copies of one head selects what that head selects alone
    qg = np.stack([_rand(8)] * 4)
    np.testing.assert_array_equal(O.topk(O.scores_per_query_head(qg[0], k, 0.5), 3),
                                  O.topk(O.scores_exact(qg, k, 0.5), 3))


# ---------------------------------------------------------------------------
# layer-reuse policy (HyLRA, section 2.2)
# ---------------------------------------------------------------------------

DS, RU, DN = O.DENSE_SELECT, O.REUSE, O.DENSE


def _tri(n, entries):
    m = np.zeros((n, n), dtype=np.int64)
    for (i, j), v in entries.items():
        m[i, j] = v
    return m


def test_index_overlap_counts_shared_positions():
    assert O.index_overlap([1, 5, 9, 12], [0, 5, 12, 30]) == 2
    assert O.index_overlap([3], [4]) == 0
    assert O.index_overlap(np.arange(10), np.arange(10)) == 10


def test_reuse_plan_worked_example():
    # total 100, theta 0.5.  Worked by hand: {0} fails (layer 3 shares only
    # 40 with layer 0); {0,3}: 90+60 = 150; {0,1}: 95+70 = 165; {0,2}: 90+80
    # = 170 -> full attention at 0 and 2, layers 1 and 3 reuse them.
    m = _tri(4, {(0, 1): 90, (0, 2): 60, (0, 3): 40, (1, 2): 95, (1, 3): 70, (2, 3): 80})
    assert O.reuse_plan_bruteforce(m, 100, 0.5) == ([DS, RU, DS, RU], [-1, 0, -1, 2])


def test_reuse_plan_limits_of_theta():
    rng = np.random.default_rng(3)
    n = 6
    m = np.triu(rng.integers(0, 101, (n, n)), 1)
    # no reuse possible: every layer runs full attention, no set is handed on
    assert O.reuse_plan_bruteforce(m, 100, 1.0) == ([DN] * n, [-1] * n)
    # every reuse allowed: one reset at layer 0 serves all
    assert O.reuse_plan_bruteforce(m, 100, -1.0) == ([DS] + [RU] * (n - 1), [-1] + [0] * (n - 1))
    # "exceeds theta" is strict: a ratio equal to theta is no reuse
    m2 = _tri(2, {(0, 1): 50})
    assert O.reuse_plan_bruteforce(m2, 100, 0.5) == ([DN, DN], [-1, -1])
    assert O.reuse_plan_bruteforce(m2, 100, 0.49) == ([DS, RU], [-1, 0])


def test_reuse_plan_sensitive_layers_and_ties():
    m = np.full((5, 5), 100, dtype=np.int64)
    # a sensitive layer always resets; the others reuse the latest reset
    assert O.reuse_plan_bruteforce(m, 100, 0.5, sensitive=[0, 0, 1, 0, 0]) == \
        ([DS, RU, DS, RU, RU], [-1, 0, -1, 2, 2])
    # tie: {0,1} and {0,2} both keep 50 -> the later reset wins
    t = _tri(3, {(0, 1): 50, (0, 2): 10, (1, 2): 50})
    assert O.reuse_plan_bruteforce(t, 100, 0.4) == ([DS, RU, DN], [-1, 0, -1])


def test_fixed_jump_plan():
    assert O.fixed_jump_plan(8, 3) == ([DS, RU, RU, DS, RU, RU, DS, RU],
                                       [-1, 0, 0, -1, 3, 3, -1, 6])
    assert O.fixed_jump_plan(4, 1) == ([DN] * 4, [-1] * 4)
    assert O.fixed_jump_plan(7, 3)[0][6] == DN        # a last full layer hands nothing on


# ---------------------------------------------------------------------------
# acceptance rule
# ---------------------------------------------------------------------------

def test_index_set_verdict():
    s = np.array([5.0, 4.0, 3.0, 2.0, 1.0])
    assert O.index_set_verdict(s, [0, 1], 2) == "exact"
    assert O.index_set_verdict(s, [0, 2], 2).startswith("failed")
    near = np.array([5.0, 3.0, 3.0 - 1e-5, 1.0])
    assert O.index_set_verdict(near, [0, 2], 2) == "excused"
    assert O.index_set_verdict(near, [0, 1], 2) == "exact"
    assert O.index_set_verdict(near, [1, 2], 2).startswith("failed")   # misses 5.0
    assert O.index_set_verdict(near, [0, 3], 2).startswith("failed")   # takes 1.0
    assert O.index_set_verdict(near, [0, 0], 2).startswith("failed")
    assert O.index_set_verdict(near, [0, 9], 2).startswith("failed")


# ---------------------------------------------------------------------------
# cost-model arithmetic printed on the pages
# ---------------------------------------------------------------------------

def test_cost_model_figures(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "cost_model.json")))
    sm = g["score_matrix"]
    assert O.score_matrix_bytes(sm["n_tokens"], sm["bytes_per_score"]) == sm["gib"] * 2 ** 30
    dsa = g["dsa_example"]
    total, saved = O.dsa_cost(dsa["context_k"], dsa["indexer_k"], dsa["selected_k"])
    assert total == dsa["total_k"]
    assert round(100 * saved) == dsa["saved_percent"]
    for n, x, k in g["sparsity_to_k"]["cases"]:
        assert n // x == k
    assert S.CONFIGS["llama32k"].k == 655 and S.CONFIGS["batch128k"].k == 262
