"""CPU oracle for MTraining-style Vertical-Slash dynamic sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the tests, the package's smoke check
and the CPU-baseline leg of the benchmark do.  It shares no code with the HIP
kernels or their host library, and it computes everything in float64 from the
definitions on the pages:

* index estimation (observation window, vertical and slash scores, top-k) —
  MTraining paper note, Algorithm 1 ("dynamic sparse training head") and
  MTraining (arXiv 2510.18830) §4.1 (i)-(ii);
* the Vertical-Slash mask (``sparseformat``) — Algorithm 1, last two steps;
* masked softmax attention forward with log-sum-exp, and its backward —
  MTraining §3.2 Eq. 1-2 and the paper note's Appendix B.1;
* the merge of partial (O, LSE) pairs across KV chunks (``merge_out_and_lse``)
  — the paper note's Appendix E, Algorithm 2;
* effective-mask-area accounting — MagiAttention "Dynamic Attention Solver",
  "Computation Cost Estimation";
* the XAttention block estimator (anti-diagonal block scores, threshold
  selection) — the paper note's appendix, baseline settings, item 2;
* the MoBA block gate (block means, per-query top-k with the own block) —
  the same appendix, item 1;
* the RoPE relative-position property — MTraining Theorem 3.1 and the paper
  note's Appendix B.2, Eq. 14.

Every function names the passage it follows.  Readings of silent or garbled
steps are listed in the repository's design notes.
"""
from .index import (capacities, window_probs, window_scores, select_topk, estimate_index,
                    topp_count, estimate_index_topp,
                    dense_mask, block_selected, row_block_selected)
from .attention import (attn_fwd_dense, attn_bwd_dense, attn_fwd_support, attn_bwd_support,
                        lse_merge, row_groups, support_candidates, bwd_delta,
                        bwd_rounding_bounds)
from .accounting import mask_area_bruteforce, mask_area_formula, dense_causal_area
from . import xattn, moba
from .xattn import antidiag_logits, xattn_block_scores, estimate_index_xattn
from .moba import block_means, gate_scores, select_blocks, estimate_index_moba

__all__ = [
    "capacities", "window_probs", "window_scores", "select_topk", "estimate_index",
    "topp_count", "estimate_index_topp", "dense_mask", "attn_fwd_dense", "attn_bwd_dense", "attn_fwd_support", "attn_bwd_support",
    "lse_merge", "row_groups", "support_candidates", "bwd_delta", "bwd_rounding_bounds",
    "mask_area_bruteforce",
    "mask_area_formula", "dense_causal_area", "xattn", "antidiag_logits", "xattn_block_scores",
    "estimate_index_xattn", "block_selected", "row_block_selected", "moba", "block_means",
    "gate_scores", "select_blocks", "estimate_index_moba",
]
