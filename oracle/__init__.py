"""CPU oracle for the tree-attention + tree-verification path.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct
restatement of what the verification hot path of EAGLE-2-style dynamic-tree
speculative decoding computes, in numpy fp64 and Python integers. Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it. It shares no code with the HIP library (no kernels, headers,
helpers, tables or constants) and imports nothing from it.

Modules and the passages they follow (page titles as published):

* ``philox``  - Philox4x64-10, Salmon, Moraes, Dror and Shaw, "Parallel Random
  Numbers: As Easy as 1, 2, 3" (SC'11). The pages name no generator; the
  counter-based stream of per-(sequence, node) uniforms is this build's reading.
* ``tree``    - EAGLE-2 dynamic tree expansion and reranking: SGLang
  "Speculative Decoding" page, sections "EAGLE Decoding" (num_steps, eagle_topk,
  num_draft_tokens) and "References" (tree-style branching by topk, stopping
  unlikely branches, reranking to the top num_draft_tokens nodes); lesty.tech
  "EAGLE-2 & Lookahead Decoding", section 4 "Dynamic Tree Construction
  Mechanics" (confidence = product of conditional probabilities).
  Tree mask: tanhdev "Tech Radar: SGLang EAGLE-2", section 2 "Dynamic
  Tree-Attention Verification" (mask equation) and section 5 "FlashAttention-3
  Tree Kernel Design" (64-bit ancestry bitmask).
* ``attention`` - attention of every tree node over the prefix plus its own
  ancestors: the same mask equation; n1n.ai "Speculative Decoding in
  Production: EAGLE-3 Dynamic Trees", section "From Linear Sequences to Dynamic
  Draft Trees" (flattened tree in one forward pass).
* ``verify``  - greedy and rejection-sampling verification of a tree: n1n.ai
  page, section "Mathematical Proof of Lossless Speedup" (steps 1-3) and
  section "From Linear Sequences to Dynamic Draft Trees" (B1 rejected, B2
  accepted); tanhdev page, section 5 "Speculative Rejection Sampling:
  Mathematical Invariance"; lesty.tech page, "Tree Attention Masking and Target
  Verification" (longest valid path).
* ``kvcompact`` - keep the accepted path's KV, drop rejected branches: tanhdev
  page, section 2 sequence diagram ("Retain Accepted Path KV & Discard Rejected
  Branches"); lesty.tech page, section 6 "Paged Tree KV-Cache Allocation".

Every function is pinned by ``tests/test_oracle_*.py`` against library routines,
closed forms, brute force or hand-worked cases. Where the pages leave a step
open, the reading taken is stated at the function.
"""

from . import philox, tree, attention, verify, kvcompact  # noqa: F401
