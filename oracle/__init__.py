"""CPU oracle for one GPU's share of Ulysses sequence parallelism.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything here: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library and does not import it.

What it computes (plain numpy, fp64 for all floating point):
  pack_ref / unpack_ref   the local sequence->head and head->sequence
                          redistributions, as explicit index arithmetic on raw
                          bits ("Snowflake's Ulysses trick ...", second
                          paragraph: after the all-to-all each GPU holds the full
                          sequence for a subset of heads; "Ulysses Sequence
                          Parallelism ...", the "All-to-All Communication" step:
                          a second all-to-all reverses it)
  pack_heads_ref / unpack_heads_ref
                          the same for any run of heads, e.g. the replicated
                          kv head of a rank when there are fewer kv heads than
                          ranks (replicated_kv_head)
  pack_qkv_ref / unpack_qkv_ref
                          the same redistributions for a fused QKV projection
                          output (query, key, value heads of a token side by
                          side), one packed tensor per section
  merge_ref               attention over a union of disjoint key sets from
                          the per-set results (log-sum-exp merge; the pages
                          compare Ulysses with Ring Attention, which produces
                          such per-chunk results)
  attn_ref                exact masked softmax attention per head and its
                          analytic gradients (the plain definition that tiled
                          attention reproduces; "Ulysses Sequence Parallelism
                          ...", the paragraph on quadratic attention cost and
                          FlashAttention)

Every function is pinned by tests in tests/test_oracle.py against brute force,
closed forms, finite differences and invariants; see the docstrings there.
"""
from .ref import (  # noqa: F401
    attn_ref,
    bf16_bits_to_f64,
    doc_tables,
    f32_bits_to_f64,
    merge_ref,
    pack_heads_ref,
    pack_qkv_ref,
    pack_ref,
    replicated_kv_head,
    unpack_heads_ref,
    unpack_qkv_ref,
    unpack_ref,
)
