"""DeepSeek Sparse Attention (DSA) forward path for AMD MI355X (gfx950).

The computation lives in libdsa.so (hand-written HIP kernels behind the C ABI
of include/dsa.h); this package only binds it."""
from .dsa import (  # noqa: F401
    DSAError, Dims, EXPORTS, dsa_attn_workspace_size, dsa_forward, dsa_forward_workspace_size,
    dsa_indexer_scores, dsa_sparse_mla_attn, dsa_topk, dsa_version, lib,
)
