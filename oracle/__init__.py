"""Plain fp64 CPU oracle for top-p block-routed attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and nothing here imports the product path.

What it computes, and where the definitions come from:

* routing (``routing``): per-block mean pooling of Q and K, block scores as
  the scaled dot product of pooled vectors, a softmax over key blocks, and
  top-p selection -- rank key blocks by probability and keep them until the
  cumulative probability reaches p.  Top-p routing is defined on the FVAttn
  review page, section 1 (Key Terms, "Top-p routing") and used in section 3
  (Method); the page does not define the block score, so the pooled score is
  the reading taken here.  For causal models the routing cuts key blocks
  after the query block before the softmax (``causal_cut``); the pages state
  routing for full attention only, so this block-level cut is a reading too.
* attention (``attention``): S = Q K^T scaled, P = softmax(S) restricted to the
  allowed keys, O = P V, and the log-sum-exp of each row -- the standard
  attention of the FlashAttention review page, Background [3] (Motivation),
  which that page says FlashAttention computes exactly (Introduction).
* scheduling (``schedule``): the longest-first work list, a greedy
  longest-processing-time assignment over workers, and the load-imbalance
  factor (max over mean) -- FVAttn review, section 1 (Runtime Load
  Balancing) and section 3 (load imbalance factor).
* work accounting (``flops``): executed attention FLOPs for a block mask.
* slack-aware augmentation (``sasa``): priced in the key tiles the attention
  kernel runs, every row of a work item takes the blocks of the item's union
  (free), and workers of a batched longest-first model whose load is below
  the makespan buy the most valuable blocks outside the union of their last
  item with their slack; or the union fill alone -- FVAttn review, section 1
  (Key Terms, "Slack-Aware Sparse Augmentation") and section 3 (Method).
* FP8 quantisation (``fp8``): OCP E4M3 codes of Q (one scale per token) and
  K (one scale per 64-token tile), scales from each group's largest
  magnitude, every decision in fp32 -- the ParaAttention/HunyuanVideo post,
  section on FP8 dynamic quantisation (format and groups are readings).  The
  fp8 attention path is exact attention on the dequantised Q and K.

All arithmetic is float64 (inputs are upcast exactly from bf16/fp32), except
that the fp8 quantiser rounds its intermediate steps to fp32 explicitly, as
its definition states.  Nothing
is blocked, fused or reordered beyond what the definitions state.  Every
function is pinned by the CPU tests against brute force, closed forms,
library special cases or invariants.
"""
from .routing import (block_sizes, num_blocks, pool_blocks, block_scores, softmax_rows,
                      top_p_select, causal_eligible, causal_cut, route, ambiguous_blocks, RouteResult)
from .attention import attend, attend_units, attend_dense_masked_logits
from .schedule import group_costs, work_list, lpt_assign, lpt_batched, static_partition_loads, load_imbalance
from .flops import executed_flops, dense_flops
from .sasa import Augmented, augment, UnionFilled, union_fill, retained_mass, item_unions, block_tiles, item_costs
from . import fp8

__all__ = [
    "block_sizes", "num_blocks", "pool_blocks", "block_scores", "softmax_rows",
    "top_p_select", "causal_eligible", "causal_cut", "route", "ambiguous_blocks", "RouteResult",
    "attend", "attend_units", "attend_dense_masked_logits",
    "group_costs", "work_list", "lpt_assign", "static_partition_loads", "load_imbalance",
    "executed_flops", "dense_flops",
    "Augmented", "augment", "UnionFilled", "union_fill", "retained_mass",
    "fp8",
]
