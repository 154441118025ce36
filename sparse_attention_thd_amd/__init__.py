"""MI355X-native DeepSeek-V4 Compressed Sparse Attention on THD packs (forward, sparse-MLA backward).

The compute lives in ``libcsa.so`` (HIP kernels for gfx950, C ABI in
``include/csa.h``); ``_lib`` is its ctypes binding and ``api`` composes the
four calls into a forward pass.  Importing this package fails when the library
has not been built (``python -m sparse_attention_thd_amd.build``).
"""
from . import _lib
from ._lib import (CsaError, csa_build_indices, csa_compress, csa_indexer_topk, csa_last_error,
                   csa_sparse_mla_bwd, csa_sparse_mla_bwd_workspace_bytes, csa_sparse_mla_fwd,
                   csa_validate_layout, csa_version)
from .api import CsaPlan, LayerCompressMode, ThdLayout, csa_forward, layer_compress_mode

__all__ = ["CsaError", "CsaPlan", "LayerCompressMode", "ThdLayout", "csa_build_indices", "csa_compress",
           "csa_forward", "csa_indexer_topk", "csa_last_error", "csa_sparse_mla_bwd",
           "csa_sparse_mla_bwd_workspace_bytes", "csa_sparse_mla_fwd", "csa_validate_layout",
           "csa_version", "layer_compress_mode"]
