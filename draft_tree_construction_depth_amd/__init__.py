"""MI355X-native draft-tree construction (DDTree-style) for speculative decoding.

The compute lives in libddtree.so (hand-written HIP for gfx950, C ABI in
include/ddtree.h); this package only binds it:

    ddtree_build     logits [batch, L, V] -> top-B prefix tree (+ ancestor mask)
    ddtree_build_noalloc  the same on the library's static scratch (no workspace)
    ddtree_select    stage 2 alone, from stage-1 tables (+ mask)
    ddtree_mask      parents -> bit-packed ancestor-only attention mask
    ddtree_accept    tree + target tokens -> accepted path, new bonus token
    ddtree_compact_kv  KV caches keep only the accepted path's rows (in place)
    ddtree_row_topk  stage 1 alone: per-row sorted top-K and log-sum-exp
    ddtree_read_probe  measurement: stage 1's read path alone (the read ceiling)
    ddtree_ts_load_probe  measurement: a TreeSpark head evaluation's loads alone
    treespark_expand TreeSpark parent-conditioned tree (bf16 MFMA head)
    sparkling_build  SparklingTree conditioned best-first tree (top-C rows, Markov head)
    sparkling_beam   fixed-branching beam tree on SparklingTree's rows (per-depth widths)
    dspark_budget    DSpark survival-ranked verification budget across the batch
"""

from ._lib import (DDT_BF16, DDT_F32, DDTreeError, ddtree_accept, ddtree_build,
                   ddtree_build_noalloc, ddtree_compact_kv,
                   ddtree_mask, ddtree_read_probe, ddtree_row_topk, ddtree_select,
                   ddtree_ts_load_probe,
                   dspark_budget, lib,
                   sparkling_beam, sparkling_build, status_string, treespark_expand)

__all__ = ["DDT_BF16", "DDT_F32", "DDTreeError", "ddtree_accept", "ddtree_build",
           "ddtree_build_noalloc",
           "ddtree_compact_kv", "ddtree_mask", "ddtree_read_probe", "ddtree_row_topk",
           "ddtree_ts_load_probe",
           "ddtree_select", "dspark_budget",
           "lib", "sparkling_beam", "sparkling_build", "status_string",
           "treespark_expand"]
