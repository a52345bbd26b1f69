"""The five workload shapes of the verification path.

Each workload is one attention layer plus one verification over a batch of
draft trees. Shapes follow the model families the pages benchmark on
(Llama-2-7B, Llama-3-8B, Llama-3-70B) and the drafting knobs of the SGLang
"Speculative Decoding" page, section "EAGLE Decoding" (num_steps = tree depth,
eagle_topk = branching factor, num_draft_tokens = nodes kept after reranking).

Per-sequence values (prefix length, topk, depth) may be drawn at random; the
draw happens in ``workloads.synth`` from the workload's seed.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    description: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    # prefix length: fixed int, or (lo, hi) inclusive uniform range per sequence
    prefix: object
    page: int
    contiguous_pages: bool
    # topk / depth: fixed int, or (lo, hi) inclusive uniform range per sequence
    topk: object
    depth: object
    num_draft: int
    vocab: int
    # "greedy", "sample", or "alternate" (even sequences greedy, odd sampling)
    verify: str
    temperature: float
    compact: bool
    seed: int

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def max_topk(self) -> int:
        return self.topk if isinstance(self.topk, int) else self.topk[1]

    @property
    def max_depth(self) -> int:
        return self.depth if isinstance(self.depth, int) else self.depth[1]

    @property
    def max_prefix(self) -> int:
        return self.prefix if isinstance(self.prefix, int) else self.prefix[1]

    @property
    def max_nodes(self) -> int:
        """T = drafts + root."""
        return self.num_draft + 1


CONFIGS: Tuple[WorkloadSpec, ...] = (
    WorkloadSpec(
        name="tiny_gqa4_d64",
        description="batch 1, 8 q / 2 kv heads, head_dim 64, prefix 256 in contiguous pages, "
        "depth 3 topk 2 -> 8 drafts + root, vocab 1000, greedy",
        batch=1, q_heads=8, kv_heads=2, head_dim=64, prefix=256, page=16,
        contiguous_pages=True, topk=2, depth=3, num_draft=8, vocab=1000,
        verify="greedy", temperature=0.0, compact=False, seed=1001,
    ),
    WorkloadSpec(
        name="llama2_7b_layer_b1",
        description="Llama-2-7B-shaped layer: batch 1, 32/32 heads (MHA), head_dim 128, prefix 1024 "
        "in shuffled 16-token pages, depth 3 topk 4 -> 16 drafts, vocab 32000, greedy",
        batch=1, q_heads=32, kv_heads=32, head_dim=128, prefix=1024, page=16,
        contiguous_pages=False, topk=4, depth=3, num_draft=16, vocab=32000,
        verify="greedy", temperature=0.0, compact=False, seed=1002,
    ),
    WorkloadSpec(
        name="llama3_8b_layer_b8",
        description="Llama-3-8B-shaped layer: batch 8, 32 q / 8 kv heads (GQA 4), head_dim 128, prefix "
        "4096 each in shuffled pages, depth 5 topk 4 -> 8 drafts, vocab 128256, rejection sampling T=1.0",
        batch=8, q_heads=32, kv_heads=8, head_dim=128, prefix=4096, page=16,
        contiguous_pages=False, topk=4, depth=5, num_draft=8, vocab=128256,
        verify="sample", temperature=1.0, compact=False, seed=1003,
    ),
    WorkloadSpec(
        name="llama3_70b_layer_b1_tree64",
        description="Llama-3-70B-shaped layer on one GPU: batch 1, 64 q / 8 kv heads (GQA 8), head_dim 128, "
        "prefix 8192 in shuffled pages, depth 6 topk 8 -> 64 drafts, vocab 128256, greedy, then "
        "accepted-path KV compaction",
        batch=1, q_heads=64, kv_heads=8, head_dim=128, prefix=8192, page=16,
        contiguous_pages=False, topk=8, depth=6, num_draft=64, vocab=128256,
        verify="greedy", temperature=0.0, compact=True, seed=1004,
    ),
    WorkloadSpec(
        name="mixed_serving_b32",
        description="mixed serving batch: 32 sequences, prefix U[512,16384] in one shared shuffled page "
        "pool, 64 q / 8 kv heads, head_dim 128, 32 drafts, depth U{4..6}, topk U{4..8}, vocab 128256, "
        "even sequences greedy, odd sequences rejection sampling T=0.7",
        batch=32, q_heads=64, kv_heads=8, head_dim=128, prefix=(512, 16384), page=16,
        contiguous_pages=False, topk=(4, 8), depth=(4, 6), num_draft=32, vocab=128256,
        verify="alternate", temperature=0.7, compact=False, seed=1005,
    ),
)


def get_config(key) -> WorkloadSpec:
    """Look a workload up by index (0-4) or by name."""
    if isinstance(key, int):
        return CONFIGS[key]
    for c in CONFIGS:
        if c.name == key:
            return c
    raise KeyError(f"unknown workload {key!r}; known: {[c.name for c in CONFIGS]}")
