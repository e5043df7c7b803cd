"""Plain fp64 CPU oracle for head-aware sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, links or runs anything in this package; only the test
suite, the smoke check and the benchmark's CPU-baseline leg do.  The oracle
shares no code with the GPU path: it is written from the definitions on the
source pages, in numpy float64, slow and obvious on purpose.

Sources (cited by page title and section in each function):
  * "RBS-Attention: Radius-Bounded Sparse Prefill for Long-Context LLMs"
    (yunkai-blog post) -- "Key technical points": 1. two-branch selector
    (centroid base branch, radius rescue branch), 2. independent thresholds
    and mask merge feeding an unchanged block-sparse FlashAttention.
  * "Kascade sparse attention" (3l3c.ai blog) -- "What Kascade got right:
    anchor-layer Top-k reuse" and "Head-aware is the key to accuracy".
  * "Can language models decide where to look?" (yetianai.com, Declarative
    Attention) -- "Declarative attention protocol" (global/focus/local modes,
    block-aligned masks over a paged KV cache, ~2048-token chunks).
  * "Million-token context: models finally pick what matters" (openai-hub.com)
    -- "Three modes, three reasoning states".
  * "Sparse attention innovation: Meituan LoZA" (aiii.org.cn) -- "2. ZigZag
    architecture" (streaming sparse attention, window 1024) and "4. From food
    delivery to AI" (SplitKV-and-Combine).

Every function is pinned by the fact tests in tests/test_oracle_facts.py
(closed forms, brute force, library special cases, invariants).  Parity
status per function:
  dense_attention, masked_attention, masked_attention_rows,
  index_attention, segment_attention, lse_combine  -- pinned
  block_stats, pool_queries, select_blocks           -- pinned
  kv_head, anchor_scores, topk, anchor_topk           -- pinned
  topk_pooled, union_sets, set_recall                 -- pinned
  gather_pages, build_segments                        -- pinned
  token_block_mass, retention, ideal_rows, index_mass -- pinned
"""

from .attention import (dense_attention, masked_attention, masked_attention_rows,
                        index_attention, segment_attention, lse_combine,
                        attention_partial)
from .blocks import block_stats, pool_queries, select_blocks, visible_count, k_of
from .topk import (kv_head, anchor_scores, topk, anchor_topk, topk_pooled, union_sets,
                   set_recall)
from .paged import gather_pages
from .segments import build_segments, SEG_GLOBAL, SEG_FOCUS, SEG_LOCAL, SEG_STREAMING
from .quality import token_block_mass, retention, ideal_rows, index_mass

__all__ = [
    "dense_attention", "masked_attention", "masked_attention_rows", "index_attention",
    "segment_attention", "lse_combine", "attention_partial", "block_stats", "pool_queries",
    "select_blocks", "visible_count", "k_of", "kv_head", "anchor_scores", "topk", "anchor_topk",
    "topk_pooled", "union_sets", "set_recall", "gather_pages",
    "build_segments", "SEG_GLOBAL", "SEG_FOCUS", "SEG_LOCAL", "SEG_STREAMING",
    "token_block_mass", "retention", "ideal_rows", "index_mass",
]
