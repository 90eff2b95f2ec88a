"""Plain float64 CPU oracle of the SuperGlue matching forward pass.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct
definition that the HIP library is checked against.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does, and this package imports nothing from the product.

Two implementations of the same functions, sharing nothing but the pages'
definitions:

* the plain C oracle (sg_oracle.c behind oracle/native.py): float64 loops in
  index order, no BLAS; the functions of this package are its functions;
* oracle.reference_numpy: float64 numpy with library matrix products, the
  independent cross-check.

Both are pinned by tests/test_oracle_*.py (every pin runs against each) to
what the pages and the mathematics fix: the pages' worked examples, closed
forms, invariants, library routines and brute force on tiny inputs.  Parity
unpinned: the end-to-end composition with trained weights, which no page
prints (covered only by the invariants and per-step pins).
"""
from . import native, reference_numpy
from .native import (adaptive_match, attentional_gnn, attentional_propagation, bidirectional_cross_attention,
                     build, confidence_threshold, double_softmax_assignment, double_softmax_from_descriptors,
                     double_softmax_match, extract_matches, final_projection, keypoint_encoder, layer_head,
                     log_optimal_transport, log_sigmoid, log_sinkhorn_iterations, match_from_descriptors,
                     matchability, multi_head_attention, normalize_keypoints, rope_angles, rotate_pairs,
                     score_matrix, set_threads, sinkhorn_knopp_exp, superglue_descriptors, superglue_match,
                     threads, token_confidence)

IMPLEMENTATIONS = {"c": native, "numpy": reference_numpy}

__all__ = ["IMPLEMENTATIONS", "native", "reference_numpy", "adaptive_match", "attentional_gnn",
           "attentional_propagation", "bidirectional_cross_attention", "build", "confidence_threshold",
           "double_softmax_assignment", "double_softmax_from_descriptors", "double_softmax_match",
           "extract_matches", "final_projection", "keypoint_encoder", "layer_head", "log_optimal_transport",
           "log_sigmoid", "log_sinkhorn_iterations", "match_from_descriptors", "matchability",
           "multi_head_attention", "normalize_keypoints", "rope_angles", "rotate_pairs", "score_matrix",
           "set_threads", "sinkhorn_knopp_exp", "superglue_descriptors", "superglue_match", "threads",
           "token_confidence"]
