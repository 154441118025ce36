"""CPU fp64 oracle for the THD Compressed Sparse Attention forward and its backward.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain definition that the
HIP library is checked against.  Only the test-suite, the smoke check and the
bench's CPU-baseline leg may import it; the library never calls it and there is
no CPU fallback anywhere in the product path.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or rounding routines).
"""
from .csa_oracle import (  # noqa: F401
    NO_COMPRESS, COMPRESSOR_ONLY, INDEXER,
    layer_compress_mode, segment_table, query_table, build_indices,
    compress, compress_learned, round_to_bf16, round_to_f32, round_to,
    indexer_scores, indexer_topk, indexer_kl_grad, sparse_mla_fwd, sparse_mla_bwd, csa_forward,
)
