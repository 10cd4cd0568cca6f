"""CPU oracle for ring block attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 implementation of what one ring step
computes (blockwise exact softmax attention of a query chunk against one KV
chunk, with a log-sum-exp), of the LSE-weighted merge of per-step partials,
and of the attention backward.  Nothing here is blocked, fused or reordered
beyond computing independent query rows in batches.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and this package imports nothing
from the product path.

Sources (no formula is printed on the pages; the definition is standard
softmax attention):
  * TASP: Topology-aware Sequence Parallelism — abstract: Ring Attention
    splits the queries into chunks across accelerators and every query chunk
    must see every KV chunk, one ring iteration at a time; the result is exact
    attention.  Experiment highlights: Zigzag-Ring Attention is the causal
    load-balanced variant.
  * Same paper, citation map ("Builds on"): Attention Is All You Need (the
    attention definition), FlashAttention / FlashAttention-2 / Self-attention
    Does Not Need O(n^2) Memory (blockwise exact attention with partial
    results), GQA (grouped KV heads).
  * HSAP: A Hierarchical Sequence-aware Parallelism for Hybrid-Context
    Generative Models — abstract and methodology: causal attention on packed
    (hybrid-context) sequences must not cross document boundaries.

Parity pins for every function are in tests/test_oracle_*.py.  Where the
pages are silent, the reading taken is stated at the function that takes it.
"""
from .attn import (MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL, allowed_mask, attention,
                        attention_backward, attention_backward_sampled, count_pairs, doc_of, merge, merge_many)
from .layouts import contiguous_positions, ring_source, striped_positions, zigzag_positions

__all__ = [
    "MASK_NONE", "MASK_CAUSAL", "MASK_DOC_CAUSAL", "allowed_mask", "attention",
    "attention_backward", "attention_backward_sampled", "count_pairs", "doc_of", "merge", "merge_many",
    "contiguous_positions", "ring_source", "zigzag_positions",
]
