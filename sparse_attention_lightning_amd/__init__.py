"""DeepSeek Sparse Attention (DSA) hot path for AMD MI355X (gfx950).

Lightning indexer (FP8) -> top-k token selector -> sparse MLA in MQA mode, plus IndexShare
reuse of one index set across layers or draft positions, and the HiSparse hot buffer that
swaps the selected latent pages in from host memory. All compute runs in the HIP
kernels of libdsa.so; this package only marshals torch tensors into the C ABI.
"""
from ._binding import (Cache, DsaError, EXPORTS, HotBuffer, LIB_PATH, OP_FORWARD_SHARED,  # noqa: F401
                       NOALLOC_SCRATCH_BYTES, OP_HISPARSE_SWAP_IN, OP_INDEX_SCORE, OP_SPARSE_MLA, OP_TOPK,
                       csa_forward, csa_workspace_size, forward_shared, forward_shared_noalloc,
                       hisparse_swap_in, index_score, lib, load_library, sparse_mla_fwd, topk, workspace_size)
