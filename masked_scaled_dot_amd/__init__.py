"""Masked scaled dot-product attention over a CSR mask, native to AMD MI355X (gfx950).

The computation runs in ``libsa.so`` (hand-written HIP kernels behind a C ABI, declared
in ``include/sa.h``); this package is its thin ctypes binding. Importing it without the
built library raises ImportError: there is no CPU or PyTorch fallback.
"""
from ._lib import (  # noqa: F401
    EXPORTS, LIB_PATH, SA_BF16, SA_ERR_ALIGN, SA_ERR_CSR, SA_ERR_DTYPE, SA_ERR_HIP, SA_ERR_NULL,
    SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_F32, SA_FLAG_VALIDATE, SA_OK, Problem,
    SaError, sa_csr_transpose, sa_fused_backward, sa_fused_backward_noalloc, sa_fused_forward, sa_gather_entries, sa_gather_entries_ordered,
    sa_gather_order_build, sa_plan_build, sa_plan_bytes, sa_plan_bytes_segments, sa_mask_workspace_bytes, sa_coo_to_csr,
    sa_key_mask_from_lengths, sa_varlen_row_ptr, sa_varlen_col_idx, sa_topk_mask,
    sa_bias_grad, sa_problem, sa_sddmm, sa_sparse_softmax, sa_sparse_softmax_backward, sa_spmm,
    sa_status_string, sa_transpose_workspace_bytes, sa_validate_csr,
    BlockCover, block_cover, sa_block_cover, sa_block_cover_row_ptr, sa_block_cover_col_idx,
    sa_block_cover_bits, sa_fused_backward_cover,
)
