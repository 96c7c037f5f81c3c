"""CPU oracle for the IndexCache hot path — TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package. The HIP library shares no
code with it and never calls it.

Every function is pinned (tests/test_oracle_*.py) by the pages' worked example,
closed forms, brute force or library special cases; none is "parity unpinned".
"""
from .indexcache import (PAD, validate_pattern, nearest_full, indexer_scores,
                         topk_row, topk, sparse_attention, schedule, layer_stack,
                         overlap, jaccard, mean_overlap, greedy_pattern, position_order,
                         overlap_matrix, overlap_proxy_loss, distill_loss, row_position)

__all__ = ["PAD", "validate_pattern", "nearest_full", "indexer_scores", "topk_row",
           "topk", "sparse_attention", "schedule", "layer_stack", "overlap",
           "jaccard", "mean_overlap", "greedy_pattern", "position_order",
           "overlap_matrix", "overlap_proxy_loss", "distill_loss", "row_position"]
