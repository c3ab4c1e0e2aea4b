"""Top-k sparse decode attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libsa.so`` (hand-written HIP kernels behind the C
ABI of ``include/sa.h``); this package is its Python binding.  Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built (``python -m top_sparse_decode_sa_amd.build``).
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIB_PATH, SA_BF16, SA_F32, SA_IDX_BLOCK_PER_KV_HEAD, SA_IDX_TOKEN_PER_KV_HEAD,
    SA_IDX_TOKEN_PER_Q_HEAD, SA_IDX_TOKEN_SHARED, SA_LAYER_DENSE, SA_LAYER_DENSE_SELECT, SA_LAYER_REUSE, SA_LAYER_SPARSE,
    SA_SCORE_BLOCK_MINMAX, SA_SCORE_EXACT, SA_SCORE_EXACT_PER_Q_HEAD, SA_SCORE_INDEXER, SA_SCORE_INDEXER_PER_KV_HEAD,
    WORKSPACES, KVDesc, LayerArgs, SAError, ScoreAux, layer_args, lib, make_desc,
    sa_block_summarize, sa_decode_layer, sa_dense_decode, sa_dense_decode_scored, sa_gather_blocks,
    sa_index_overlap, sa_layer_workspace_size, sa_plan_fixed_jump, sa_plan_reuse,
    sa_check_indices, sa_plan_validate, sa_score, sa_select, sa_sparse_decode,
    sa_sparse_decode_noalloc,
    sa_gather_read, sa_stream_read, sa_topk,
    sa_version, sa_workspace_init)

__version__ = "0.1.0"
