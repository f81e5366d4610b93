"""MI355X-native (gfx950) sparse-attention indexer hot path.

The computation lives in libsparse_indexer.so (hand-written HIP, C ABI in
include/sparse_indexer.h); this package only marshals torch tensors into it.
"""
from ._binding import (SparseIndexerError, block_sparse_select, dosa_prune_topk, gather_slots,
                       idx_score, idx_score_topk, idx_score_topk_noalloc, idx_score_topk_prior,
                       idx_score_topk_witness, kvwitness_merge, lib, positions_of_blocks,
                       rows_topk, status_string)

__all__ = ["idx_score_topk", "idx_score_topk_noalloc", "idx_score_topk_witness",
           "idx_score_topk_prior", "idx_score", "rows_topk", "dosa_prune_topk", "kvwitness_merge",
           "block_sparse_select", "positions_of_blocks", "gather_slots", "SparseIndexerError",
           "lib", "status_string"]
