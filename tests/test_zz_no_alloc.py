"""The allocation-free entry point, sa_sparse_decode_noalloc, through the C
ABI: on plans that split rows across workgroups (so its static scratch holds
the split partials) it must write exactly what sa_sparse_decode writes with a
caller workspace -- on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents), and when captured in a HIP
graph and replayed."""
import numpy as np
import pytest
import torch

import top_sparse_decode_sa_amd as T
from top_sparse_decode_sa_amd import _binding as Bn
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, N, k, kind, seed):
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    K = torch.randn(B, Hkv, N, 128, device=dev(), generator=g).to(torch.bfloat16)
    V = torch.randn(B, Hkv, N, 128, device=dev(), generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, 128, device=dev(), generator=g).to(torch.bfloat16)
    rows = B if kind == T.SA_IDX_TOKEN_SHARED else B * Hkv
    idx = torch.stack([torch.randperm(N, device=dev(), generator=g)[:k] for _ in range(rows)])
    idx = idx.sort(dim=-1).values.to(torch.int32)
    idx = idx.view(B, k) if kind == T.SA_IDX_TOKEN_SHARED else idx.view(B, Hkv, k)
    return q, K, V, idx.contiguous()


def _needs_scratch(q, K, idx, kind):
    desc = T.make_desc(q, K)
    import ctypes
    return T.lib().sa_sparse_workspace_size(ctypes.byref(desc), kind, idx.shape[-1], 0)


# (B, Hq, Hkv, N, k, index kind): the first larger than the second
CALLS = [(2, 32, 8, 65536, 2048, T.SA_IDX_TOKEN_PER_KV_HEAD),
         (1, 32, 8, 16384, 700, T.SA_IDX_TOKEN_SHARED)]


def test_noalloc_equals_workspace_call_twice_in_a_row():
    for i, (B, Hq, Hkv, N, k, kind) in enumerate(CALLS):
        say("no-alloc call %d: B %d, %d/%d heads, N %d, k %d, kind %d" % (i, B, Hq, Hkv, N, k, kind))
        q, K, V, idx = _inputs(B, Hq, Hkv, N, k, kind, seed=100 + i)
        need = _needs_scratch(q, K, idx, kind)
        assert 0 < need <= 16 << 20, need   # the plan splits rows: the scratch is in use
        want = T.sa_sparse_decode(q, K, V, idx, kind)
        out = torch.full_like(want, float("nan"))
        T.sa_sparse_decode_noalloc(q, K, V, idx, kind, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, want), "call %d differs" % i


def test_noalloc_in_a_graph():
    B, Hq, Hkv, N, k, kind = CALLS[0]
    say("no-alloc graph: B %d, N %d, k %d" % (B, N, k))
    q, K, V, idx = _inputs(B, Hq, Hkv, N, k, kind, seed=7)
    want = T.sa_sparse_decode(q, K, V, idx, kind)
    out = torch.zeros_like(want)
    T.sa_sparse_decode_noalloc(q, K, V, idx, kind, out=out)   # first call on the device: lookup
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        T.sa_sparse_decode_noalloc(q, K, V, idx, kind, out=out)
    for rep in range(3):
        out.zero_()
        # other work of the program between replays, on the same scratch
        T.sa_sparse_decode_noalloc(q[:1], K[:1], V[:1], idx[:1], kind, out=torch.empty_like(want[:1]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), "replay %d differs" % rep
