"""Plain fp64 CPU oracle for topology-scheduled block-sparse causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or executes anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
call it.  It shares no code with the HIP path.

What it computes (all in float64, numpy only):

* ``schedule`` -- the CSR block schedule of the pages "Add topology-derived
  sparse attention kernel" (triton-lang/kernels pull request 22): sink blocks,
  a local window and the top-k key blocks ranked by elder-rule 0-dimensional
  persistence (H0) salience of the key-block centroids, built by brute force
  over ALL centroid pairs (no MST shortcut); plus the dense causal CSR and the
  fixed-segment (block-diagonal causal) CSR.
* ``attention`` -- dense masked attention: every query row takes a full-width
  softmax over the keys its CSR row allows, with the causal constraint
  (key position <= query position).
* ``attention_grad`` -- the gradients (dQ, dK, dV) of that attention and its
  per-row log-sum-exp, by the closed form of the row-softmax chain rule; and
  ``schedule.transpose_schedule``, the column view of a CSR schedule that the
  key/value gradients gather over.

Each function names the passage of the pages it follows.  Readings of points the
pages leave open are listed, with the reason for each, in the repository's
design notes; they are repeated briefly where they are used.
"""
from .schedule import (
    block_centroids,
    centroid_distances,
    elder_rule_salience,
    top_k_blocks,
    schedule_from_salience,
    build_schedule,
    dense_causal_schedule,
    fixed_segment_schedule,
    csr_to_block_sets,
    transpose_schedule,
    refine_schedule,
)
from .attention import allowed_key_mask, masked_attention, masked_attention_rows
from .attention_grad import masked_lse, attention_backward, attention_backward_rows

__all__ = [
    "block_centroids",
    "centroid_distances",
    "elder_rule_salience",
    "top_k_blocks",
    "schedule_from_salience",
    "build_schedule",
    "dense_causal_schedule",
    "fixed_segment_schedule",
    "csr_to_block_sets",
    "transpose_schedule",
    "refine_schedule",
    "allowed_key_mask",
    "masked_attention",
    "masked_attention_rows",
    "masked_lse",
    "attention_backward",
    "attention_backward_rows",
]
