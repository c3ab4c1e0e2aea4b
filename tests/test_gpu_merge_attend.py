"""GPU parity of the SPARSE layer's merge-then-attend launch.

When the selection is fused (parts scored and pre-selected on chip) and the
gather-attend plan gives each row one workgroup, sa_decode_layer(SPARSE)
runs the selection's merge and the gather-attend in one launch.  Its index
list must equal sa_select's and its output sa_sparse_decode's over that
list, value for value: the launch does the same merge and the same per-wave
attention work.  The cases cover 64, 48 and 32 slots per wave, 4 and 8
candidate keys per thread, groups of 4 and 2 query heads, a ragged last part
and the per-KV-head indexer.  Per-query-head rows split into parts are not
fused (their scoring reads each key row once for the KV head's query heads,
then a top-k per query head): that case checks the same equality through
the shared-row scoring launch."""
import pytest
import torch

import top_sparse_decode_sa_amd as T
from gpu_util import dev, say

pytestmark = pytest.mark.gpu

EX, EXQ, IXK = T.SA_SCORE_EXACT, T.SA_SCORE_EXACT_PER_Q_HEAD, T.SA_SCORE_INDEXER_PER_KV_HEAD

CASES = [
    # B, Hq, Hkv, N, k, kind, what
    (16, 32, 8, 32768, 655, EX, "llama shape: 4 parts, 2620 candidates, 11 waves of 64 slots"),
    (16, 32, 8, 40960, 655, EX, "5 parts: 3275 candidates, 8 keys per thread"),
    (16, 32, 8, 32768, 500, EX, "48 slots per wave"),
    (16, 32, 8, 20000, 300, EX, "32 slots per wave, ragged last part"),
    (32, 16, 8, 32768, 655, EX, "groups of 2 query heads"),
    (4, 32, 8, 32768, 655, EXQ, "per query head: 128 rows of one head, scored four to a key load"),
    (16, 32, 8, 32768, 655, IXK, "per-KV-head indexer"),
    (16, 32, 8, 32768, 1, EX, "k = 1: one wave with slots, eleven idle"),
    (16, 32, 8, 32768, 768, EX, "k = 768: twelve full waves, 3072 candidates (register capacity)"),
]


def _kernels_seen(fn):
    """Names of the device kernels fn launches, from the torch profiler
    (empty if the profiler records no device activity here)."""
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    return {e.name for e in prof.events()}


@pytest.mark.parametrize("B,Hq,Hkv,N,k,kind,what", CASES)
def test_layer_merge_attend_equals_select_then_decode(B, Hq, Hkv, N, k, kind, what):
    say("merge-attend B=%d Hq=%d Hkv=%d N=%d k=%d kind=%d (%s)" % (B, Hq, Hkv, N, k, kind, what))
    g = torch.Generator(device=dev()).manual_seed(N + k + kind)
    q = torch.randn((B, Hq, 128), generator=g, device=dev()).to(torch.bfloat16)
    kc = torch.randn((B, Hkv, N, 128), generator=g, device=dev()).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, N, 128), generator=g, device=dev()).to(torch.bfloat16)
    extra = {}
    if kind == IXK:
        extra = {"q_idx": torch.randn((B, Hkv, 4, 64), generator=g, device=dev()).to(torch.bfloat16),
                 "k_idx": torch.randn((B, Hkv, N, 64), generator=g, device=dev()).to(torch.bfloat16),
                 "idx_w": torch.rand((B, Hkv, 4), generator=g, device=dev())}
    want_idx = T.sa_select(q, kc, k, kind, **extra)
    ik = T.SA_IDX_TOKEN_PER_Q_HEAD if kind == EXQ else T.SA_IDX_TOKEN_PER_KV_HEAD
    want_out = T.sa_sparse_decode(q, kc, vc, want_idx, index_kind=ik)
    args, out, d_ = T.layer_args(q, kc, vc, kind, k, **extra)
    idx = torch.empty_like(want_idx)
    names = _kernels_seen(lambda: T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_))
    expect = "score_exact_heads_kernel" if kind == EXQ else "merge_attend_kernel"
    if names:
        assert any(expect in n for n in names), sorted(names)
    else:
        say("  (the profiler recorded no device kernels; launch path not checked)")
    torch.cuda.synchronize()
    assert torch.equal(idx, want_idx), what
    assert torch.equal(out, want_out), what
    del q, kc, vc, extra
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,Hq,Hkv,N,k,what", [
    (2, 8, 2, 32768, 655, "4 rows: the gather-attend splits each row"),
    (16, 32, 8, 32768, 769, "k = 769: more slots than twelve waves of 64"),
])
def test_layer_without_whole_row_plan_keeps_two_launches(B, Hq, Hkv, N, k, what):
    """When a row's gather-attend does not fit one workgroup, the layer runs
    the merge and the split gather-attend as before, with the same results
    as the two calls."""
    say("merge-attend fallback: %s" % what)
    g = torch.Generator(device=dev()).manual_seed(3 + k)
    q = torch.randn((B, Hq, 128), generator=g, device=dev()).to(torch.bfloat16)
    kc = torch.randn((B, Hkv, N, 128), generator=g, device=dev()).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, N, 128), generator=g, device=dev()).to(torch.bfloat16)
    want_idx = T.sa_select(q, kc, k)
    want_out = T.sa_sparse_decode(q, kc, vc, want_idx)
    args, out, d_ = T.layer_args(q, kc, vc, EX, k)
    idx = torch.empty_like(want_idx)
    names = _kernels_seen(lambda: T.sa_decode_layer(args, T.SA_LAYER_SPARSE, idx, d_))
    assert not any("merge_attend_kernel" in n for n in names)
    torch.cuda.synchronize()
    assert torch.equal(idx, want_idx)
    assert torch.equal(out, want_out)
