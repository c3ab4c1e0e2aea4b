"""The seeded input generator: slices and single rows regenerate the same
stored values as the whole tensor (what lets the tests and the benchmark's
oracle leg rebuild any row of a large cache on the host)."""
import dataclasses

import numpy as np
import pytest

import sa_synth as S


def _small(name, **kw):
    return dataclasses.replace(S.CONFIGS[name], batch=2, ctx_len=1000, n_layers=3, **kw)


@pytest.mark.parametrize("name", ["llama32k", "block61k", "indexer1m", "hylra32k"])
def test_rows_and_batch_slices_match_the_whole_cache(name):
    c = _small(name, n_planted=10, planted_frac=0.01) if S.CONFIGS[name].planting != "none" \
        else _small(name)
    w = S.Workload(c, 3)
    for layer in (0, 2):
        k, v = w.k(layer), w.v(layer)
        assert np.array_equal(w.k(layer, batch=(1, 2))[0], k[1])
        for b, r in [(0, 0), (1, c.n_kv_heads - 1)]:
            assert np.array_equal(w.k_row(layer, b, r), k[b, r])
            assert np.array_equal(w.v_row(layer, b, r), v[b, r])


def test_token_rows_match_whole_rows():
    c = _small("indexer1m")
    w = S.Workload(c, 5)
    toks = np.array([0, 1, 17, 500, 999])
    for layer, b, r in [(0, 0, 0), (2, 1, 7)]:
        assert np.array_equal(w.kv_tokens("k", layer, b, r, toks), w.k_row(layer, b, r)[toks])
        assert np.array_equal(w.kv_tokens("v", layer, b, r, toks), w.v_row(layer, b, r)[toks])
    with pytest.raises(ValueError):
        S.Workload(_small("block61k"), 0).kv_tokens("k", 0, 0, 0, toks)
