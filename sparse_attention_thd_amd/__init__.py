"""MI355X-native DeepSeek-V4 Compressed Sparse Attention on THD packs (forward, sparse-MLA backward,
indexer KL-loss gradient).

The compute lives in ``libcsa.so`` (HIP kernels for gfx950, C ABI in
``include/csa.h``); ``_lib`` is its ctypes binding and ``api`` composes the
four calls into a forward pass.  Importing this package fails when the library
has not been built (``python sparse_attention_thd_amd/build.py``).
"""
from . import _lib
from ._lib import (CSA_IDX_ANY, CSA_IDX_TOPK, CsaError, csa_build_indices, csa_compress, csa_compress_learned,
                   csa_indexer_kl_grad, csa_indexer_kl_grad_noalloc, csa_indexer_kl_grad_workspace_bytes,
                   csa_indexer_topk, csa_indexer_topk_workspace_bytes, csa_last_error, csa_sparse_mla_bwd,
                   csa_sparse_mla_bwd_deterministic, csa_sparse_mla_bwd_deterministic_workspace_bytes,
                   csa_sparse_mla_bwd_workspace_bytes, csa_sparse_mla_fwd, csa_validate_layout,
                   csa_validate_topk_rows, csa_version)
from .api import CsaPlan, LayerCompressMode, LearnedCompressor, ThdLayout, csa_forward, layer_compress_mode

__all__ = ["CSA_IDX_ANY", "CSA_IDX_TOPK", "CsaError", "CsaPlan", "LayerCompressMode", "LearnedCompressor", "ThdLayout", "csa_build_indices", "csa_compress",
           "csa_compress_learned", "csa_forward", "csa_indexer_kl_grad", "csa_indexer_kl_grad_noalloc", "csa_indexer_kl_grad_workspace_bytes", "csa_indexer_topk", "csa_indexer_topk_workspace_bytes",
           "csa_last_error", "csa_sparse_mla_bwd", "csa_sparse_mla_bwd_deterministic",
           "csa_sparse_mla_bwd_deterministic_workspace_bytes", "csa_sparse_mla_bwd_workspace_bytes", "csa_sparse_mla_fwd", "csa_validate_layout", "csa_validate_topk_rows",
           "csa_version", "layer_compress_mode"]
