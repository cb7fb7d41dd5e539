"""DeepSeek Sparse Attention hot path on AMD Instinct MI355X (gfx950).

Lightning-indexer scoring -> per-query top-k -> MQA-mode sparse MLA, as hand-written HIP
kernels behind the C ABI of include/dsa.h (libdsa.so).  This package is the thin Python
binding: torch provides device memory and streams, the library does every step.
"""
from ._lib import DSAError, EXPORTS, LIB_PATH, TOPK_NOALLOC_SCRATCH_BYTES, load  # noqa: F401
from .api import (  # noqa: F401
    PagedKV, decode_scores, decode_workspace_size, dsa_append_paged, dsa_decode_paged, dsa_indexer_bwd, dsa_indexer_bwd_listed,
    dsa_indexer_kl_loss, dsa_indexer_kl_loss_sparse,
    dsa_indexer_logits, dsa_indexer_logits_ue8m0, dsa_prefill_paged, dsa_profile_begin, dsa_profile_end,
    dsa_profile_kernel_name, dsa_quantize_fp8_rows,
    dsa_quantize_fp8_rows_ue8m0, dsa_sparse_mla_bwd, dsa_sparse_mla_fwd, dsa_topk, dsa_topk_noalloc, indexer_bwd_workspace_size, ld_for, make_dims,
    prefill_workspace_size,
)
