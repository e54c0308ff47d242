"""MI355X-native Qwen Sparse Attention (QSA): forward path, sparse-attention backward and
the indexer's KL warm-up.

The computation lives in libqsa.so (hand-written HIP kernels for gfx950 behind the C
ABI of include/qsa.h); this package only builds it and marshals torch tensors to it.
"""
from .ops import (  # noqa: F401
    DecodePlan,
    PrefillPlan,
    VarlenPlan,
    prefer_fused_select,
    QSAError,
    abi_version,
    default_row_chunk,
    qsa_decode_forward,
    qsa_decode_forward_noalloc,
    qsa_decode_forward_paged,
    qsa_index_scores,
    qsa_index_scores_bwd,
    qsa_indexer_kl_loss,
    qsa_indexer_kl_target,
    qsa_pool_keys,
    qsa_prefill_forward,
    qsa_prefill_select,
    qsa_prefill_varlen_forward,
    qsa_sparse_attn_bwd,
    qsa_sparse_attn_decode,
    qsa_sparse_attn_fwd,
    qsa_sparse_attn_fwd_launches,
    qsa_sparse_attn_fwd_rows_per_launch,
    qsa_sparse_attn_fwd_tiled,
    qsa_sparse_attn_varlen_fwd,
    qsa_topk_blocks,
    score_ld,
)
