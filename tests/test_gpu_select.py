"""GPU parity of sa_select, exact selection without the score array.

Every case must give, position for position, the index list of sa_score
(exact) followed by sa_topk on the same device inputs.  That chain is itself
pinned to the oracle elsewhere; one ragged case here is also checked against
the oracle's fp64 scores directly.  The cases cover the fused path (parts of
8192 tokens, parts shortened for few rows, a ragged last part, an odd and an
even iteration count, each merge variant), the one-part path (which writes
the index list itself), the fallback when the candidates would be more than
a quarter of the row, both dtypes and head sizes, per-query-head rows, and
ties, NaN and -0.0 across part boundaries."""
import numpy as np
import pytest
import torch

import oracle as O
import top_sparse_decode_sa_amd as T
from gpu_util import dev, say, verdicts

pytestmark = pytest.mark.gpu


def _cache(B, Hq, Hkv, N, d, dtype, seed):
    """q and K drawn N(0, 1) on the device (large caches stay off the host)."""
    g = torch.Generator(device=dev()).manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((B, Hq, d), generator=g, device=dev(), dtype=torch.float32).to(tdt)
    k = torch.randn((B, Hkv, N, d), generator=g, device=dev(), dtype=torch.float32).to(tdt)
    return q, k


def _reference(q, k, kk, kind=T.SA_SCORE_EXACT):
    return T.sa_topk(T.sa_score(q, k, kind), kk)


CASES = [
    # B, Hq, Hkv, N, d, dtype, k, what
    (16, 32, 8, 32768, 128, "bf16", 655, "llama-shaped rows: four 8192-token parts, 2620-key merge"),
    (2, 8, 2, 32768, 128, "bf16", 655, "few rows: 4096-token parts, 5240-key merge"),
    (32, 64, 8, 2 * 8192 + 768, 128, "bf16", 300, "parts of 32, 32 and 3 iterations"),
    (1, 4, 1, 20000, 128, "bf16", 300, "ragged last part"),
    (3, 6, 3, 100, 128, "bf16", 10, "one part shorter than one iteration"),
    (1, 2, 2, 1, 128, "bf16", 1, "one token"),
    (2, 4, 2, 300, 64, "bf16", 300, "k = N"),
    (2, 4, 2, 5000, 64, "f32", 37, "f32, head_dim 64"),
    (2, 8, 4, 9000, 128, "f32", 500, "f32, head_dim 128"),
    (2, 4, 2, 3000, 64, "bf16", 64, "bf16, head_dim 64"),
    (1, 8, 8, 65536, 128, "bf16", 1500, "12000 candidates: 1024-thread merge"),
    (2, 8, 2, 32768, 128, "bf16", 12000, "fallback: candidates more than a quarter of the row"),
    (16, 32, 8, 32768, 128, "bf16", 3276, "fallback at 10x sparsity"),
    (32, 64, 8, 2 * 8192 + 768, 64, "f32", 300, "f32, head_dim 64, 768 parts: 256-thread parts"),
    (16, 32, 8, 2 * 8192, 64, "bf16", 300, "bf16, head_dim 64, 256 parts: 512-thread parts"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,k,what", CASES)
def test_select_matches_score_then_topk(B, Hq, Hkv, N, d, dtype, k, what):
    say("select B=%d Hq=%d Hkv=%d N=%d d=%d %s k=%d (%s)" % (B, Hq, Hkv, N, d, dtype, k, what))
    q, kc = _cache(B, Hq, Hkv, N, d, dtype, seed=N + k)
    got = T.sa_select(q, kc, k)
    want = _reference(q, kc, k)
    torch.cuda.synchronize()
    assert torch.equal(got, want), what
    del q, kc
    torch.cuda.empty_cache()


def test_select_per_query_head():
    say("select per query head")
    q, kc = _cache(2, 8, 2, 20000, 128, "bf16", seed=3)
    got = T.sa_select(q, kc, 300, kind=T.SA_SCORE_EXACT_PER_Q_HEAD)
    assert tuple(got.shape) == (2, 8, 300)
    assert torch.equal(got, _reference(q, kc, 300, T.SA_SCORE_EXACT_PER_Q_HEAD))


def test_select_against_oracle():
    """Ragged parts, checked against fp64 scores: the selected set is the
    exact top-k up to fp32 near-ties, in ascending order."""
    say("select vs oracle")
    B, Hq, Hkv, N, d, k = 1, 8, 2, 20000, 128, 300
    q, kc = _cache(B, Hq, Hkv, N, d, "bf16", seed=11)
    got = T.sa_select(q, kc, k).cpu().numpy()
    qf = q.cpu().to(torch.float64).numpy()
    kf = kc.cpu().to(torch.float64).numpy()
    G = Hq // Hkv
    s64 = [O.scores_exact(qf[0, r * G:(r + 1) * G], kf[0, r], O.default_scale(d)) for r in range(Hkv)]
    counts, fails = verdicts(s64, [got[0, r] for r in range(Hkv)], k)
    assert counts["failed"] == 0, fails


@pytest.mark.parametrize("pattern", ["zero query", "integer scores", "nan and signed zero"])
def test_select_ties_and_specials(pattern):
    """Equal scores across part boundaries go to the lower position; NaN
    ranks below every number; -0.0 equals +0.0."""
    say("select specials: %s" % pattern)
    B, Hq, Hkv, N, d, k = 2, 8, 2, 20000, 128, 300
    q, kc = _cache(B, Hq, Hkv, N, d, "bf16", seed=5)
    if pattern == "zero query":
        q.zero_()
    elif pattern == "integer scores":
        q = torch.round(q.float()).to(q.dtype)
        kc = torch.round(kc.float().clamp(-1, 1)).to(kc.dtype)
    else:
        kc[:, :, 17::97, :] = float("nan")
        q[:, :, 0] = 0.0
        kc[:, :, 5::13, :] = 0.0
        kc[:, :, 6::13, :] = -0.0
    got = T.sa_select(q, kc, k)
    want = _reference(q, kc, k)
    assert torch.equal(got, want), pattern
    if pattern == "zero query":
        assert torch.equal(got.cpu(), torch.arange(k, dtype=torch.int32).expand(B, Hkv, k))


# ------------------------------------------------------------ indexer kinds

IDX_CASES = [
    # B, Hkv, N, H, Di, k, shared, what
    (16, 8, 32768, 4, 64, 655, False, "llama-shaped per-KV-head indexer, four 8192-token parts"),
    (2, 2, 20000, 4, 64, 300, False, "ragged last part"),
    (3, 2, 9000, 16, 128, 200, True, "shared indexer, 16 heads of 128 dims"),
    (2, 4, 5000, 3, 32, 40, False, "3 heads of 32 dims"),
    (4, 2, 100, 8, 64, 10, True, "one part shorter than one iteration"),
    (2, 2, 32768, 4, 64, 12000, False, "fallback: candidates more than a quarter of the row"),
    (128, 8, 131072, 4, 64, 262, False, "batch128k shape at 500x: 1024 rows of sixteen 8192-token parts"),
    # few long rows: the scoring launch counts the top-k's histogram
    (1, 8, 1 << 20, 4, 64, 2048, True, "indexer1m shape: one 1M-token row, histogram counted"),
    (2, 2, 200003, 4, 64, 8192, True, "counted histogram, ragged last chunk, k = 8192"),
    (3, 1, 65536 + 77, 4, 64, 1, True, "counted histogram, k = 1"),
    (2, 2, 40000, 16, 128, 700, True, "counted histogram, 16 heads of 128 dims"),
]


def _indexer_inputs(B, Hkv, N, H, Di, shared, seed):
    """Indexer tensors drawn on the device; q and a cache view that only give
    the call its shapes (the indexer kinds read neither)."""
    g = torch.Generator(device=dev()).manual_seed(seed)
    lead = (B,) if shared else (B, Hkv)
    qi = torch.randn(lead + (H, Di), generator=g, device=dev()).to(torch.bfloat16)
    ki = torch.randn(lead + (N, Di), generator=g, device=dev()).to(torch.bfloat16)
    w = torch.rand(lead + (H,), generator=g, device=dev())
    q = torch.zeros((B, Hkv * 4, 128), dtype=torch.bfloat16, device=dev())
    kc = torch.zeros((N, 128), dtype=torch.bfloat16, device=dev()).as_strided(
        (B, Hkv, N, 128), (0, 0, 128, 1))
    return q, kc, qi, ki, w


@pytest.mark.parametrize("B,Hkv,N,H,Di,k,shared,what", IDX_CASES)
def test_select_indexer_matches_score_then_topk(B, Hkv, N, H, Di, k, shared, what):
    say("select indexer B=%d Hkv=%d N=%d H=%d Di=%d k=%d shared=%s (%s)" % (
        B, Hkv, N, H, Di, k, shared, what))
    kind = T.SA_SCORE_INDEXER if shared else T.SA_SCORE_INDEXER_PER_KV_HEAD
    q, kc, qi, ki, w = _indexer_inputs(B, Hkv, N, H, Di, shared, seed=N + H)
    got = T.sa_select(q, kc, k, kind, q_idx=qi, k_idx=ki, idx_w=w)
    want = T.sa_topk(T.sa_score(q, kc, kind, q_idx=qi, k_idx=ki, idx_w=w), k)
    torch.cuda.synchronize()
    assert tuple(got.shape) == ((B, k) if shared else (B, Hkv, k))
    assert torch.equal(got, want), what
    del q, kc, qi, ki, w, got, want
    torch.cuda.empty_cache()


def test_select_indexer_against_oracle():
    """Indexer selection checked against the oracle's fp64 indexer scores:
    the exact top-k up to fp32 near-ties, in ascending order."""
    say("select indexer vs oracle")
    B, Hkv, N, H, Di, k = 1, 2, 20000, 4, 64, 300
    q, kc, qi, ki, w = _indexer_inputs(B, Hkv, N, H, Di, False, seed=21)
    got = T.sa_select(q, kc, k, T.SA_SCORE_INDEXER_PER_KV_HEAD, q_idx=qi, k_idx=ki, idx_w=w)
    got = got.cpu().numpy()
    qf = qi.cpu().to(torch.float64).numpy()
    kf = ki.cpu().to(torch.float64).numpy()
    wf = w.cpu().to(torch.float64).numpy()
    s64 = [O.scores_indexer(qf[0, r], kf[0, r], wf[0, r]) for r in range(Hkv)]
    counts, fails = verdicts(s64, [got[0, r] for r in range(Hkv)], k)
    assert counts["failed"] == 0, fails


def test_select_indexer_long_row_against_oracle():
    """One 200003-token row (the multi-workgroup top-k with its histogram
    counted by the indexer launch) against the oracle's fp64 indexer scores."""
    say("select indexer long row vs oracle")
    B, Hkv, N, H, Di, k = 1, 2, 200003, 4, 64, 2048
    q, kc, qi, ki, w = _indexer_inputs(B, Hkv, N, H, Di, True, seed=23)
    got = T.sa_select(q, kc, k, T.SA_SCORE_INDEXER, q_idx=qi, k_idx=ki, idx_w=w).cpu().numpy()
    s64 = O.scores_indexer(qi.cpu().to(torch.float64).numpy()[0], ki.cpu().to(torch.float64).numpy()[0],
                           w.cpu().to(torch.float64).numpy()[0])
    counts, fails = verdicts([s64], [got[0]], k)
    assert counts["failed"] == 0, fails


@pytest.mark.parametrize("what", ["zero weights", "all dots negative"])
def test_select_indexer_long_row_all_ties(what):
    """Every score equal (0): the top-k is the first k positions; bin d1 then
    holds the whole row, more than the candidate list takes, so the last
    launch runs the row path."""
    say("select indexer long row ties: %s" % what)
    B, Hkv, N, H, Di, k = 2, 2, 300001, 4, 64, 3000
    q, kc, qi, ki, w = _indexer_inputs(B, Hkv, N, H, Di, True, seed=29)
    if what == "zero weights":
        w.zero_()
    else:
        ki = ki.abs()
        qi = -qi.abs()
    got = T.sa_select(q, kc, k, T.SA_SCORE_INDEXER, q_idx=qi, k_idx=ki, idx_w=w)
    assert torch.equal(got.cpu(), torch.arange(k, dtype=torch.int32).expand(B, k))
