"""Draft-tree construction (EAGLE-2 expansion + reranking) and the tree mask.

Tree construction follows the SGLang "Speculative Decoding" page ("EAGLE
Decoding": num_steps is the drafting depth, eagle_topk the branching factor per
step, num_draft_tokens the nodes kept; "References": the draft is extended in a
tree style with topk branches per step, unlikely branches stop expanding, and a
final reranking keeps the top num_draft_tokens nodes) and the lesty.tech page
"EAGLE-2 & Lookahead Decoding", section 4 "Dynamic Tree Construction Mechanics"
(the confidence of a draft path is the product of its conditional
probabilities, i.e. the sum of its log-probs).

Readings taken where the pages leave the rule open:

* expansion is layer-wise: at step 1 the root spawns its top-k tokens; at step
  d >= 2 each of the k frontier nodes (the k best nodes of step d-1 by
  cumulative score) spawns its top-k tokens, so k*k candidates join the pool
  and the k best of them form the next frontier; nodes outside the frontier
  stop expanding;
* the rerank keeps the N best nodes of the whole pool; kept nodes are numbered
  1..N in pool order (root = node 0);
* ranking keys: vocabulary top-k by (log-prob desc, token asc); frontier and
  rerank by (score desc, pool index asc). A child's score never exceeds its
  parent's and the parent has the smaller pool index, so the kept set is
  closed under taking parents and parents[i] < i;
* draft log-probs are clamped: NaN -> -inf, values >= 0 (including -0) -> +0;
* scores are fp64: score(child) = score(parent) + double(logprob), with
  score(root) = 0;
* truncated draft vocabulary (SGLang page, "EAGLE-2 Decoding via
  Frequency-Ranked Speculative Sampling": the draft's LM head covers only a
  high-frequency token subset, given as a token map): the draft rows hold
  V_draft entries, entry i standing for token token_map[i]; the ranking above
  runs on the draft index i (ties to the smaller index, i.e. the
  higher-ranked token of the subset) and a node's token is token_map[i].
  Without a map the index is the token.

Mask (tanhdev "Tech Radar: SGLang EAGLE-2", section 2 "Dynamic Tree-Attention
Verification": node i attends exactly to its ancestors and itself; section 5
"FlashAttention-3 Tree Kernel Design": one 64-bit word per node, a bitwise AND
decides ancestry). The root is every node's ancestor and is left implicit, so
bit (j - 1) of anc[i] stands for draft node j and N <= 64 drafts fit one word.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

STATUS_INVALID_PARENT = 1


def row_topk(row: np.ndarray, k: int):
    """Top-k (token, value) of one draft row by (value desc, token asc)."""
    vals = np.asarray(row, dtype=np.float32).astype(np.float64)
    vals = np.where(np.isnan(vals), -np.inf, vals)
    vals = np.where(vals >= 0.0, 0.0, vals)
    tokens = np.arange(vals.shape[0])
    order = np.lexsort((tokens, -vals))  # primary: -value ascending, then token
    return [(int(t), float(vals[t])) for t in order[:k]]


@dataclass
class PoolEntry:
    token: int
    parent: int  # pool index, -1 for the root
    score: float
    depth: int
    frontier_slot: int = -1  # f if this entry was frontier slot f at step ``depth``


@dataclass
class BuiltTree:
    tokens: np.ndarray  # int32 [T]
    parents: np.ndarray  # int32 [T], parents[0] = -1
    depth: np.ndarray  # int32 [T]
    anc: np.ndarray  # uint64 [T]
    q_row: np.ndarray  # int32 [T]
    frontier_tokens: List[List[int]]  # per step, in rank order
    pool: List[PoolEntry]
    kept: List[int]  # pool indices of nodes 1..N


def pool_size(k: int, D: int) -> int:
    return k + (D - 1) * k * k


def draft_row_index(step: int, slot: int, max_topk: int) -> int:
    """Row of the per-sequence draft-row array that step ``step`` uses for frontier slot ``slot``."""
    if step == 1:
        return 0
    return 1 + (step - 2) * max_topk + slot


def build_tree(rows, root_token: int, k: int, D: int, N: int, max_topk: int, token_map=None) -> BuiltTree:
    """Build one sequence's draft tree.

    ``rows`` is the per-sequence draft log-prob array [R, V] laid out as in
    ``draft_row_index``: row 0 is the root's row (step 1), and step d's row for
    frontier slot f is ``draft_row_index(d, f, max_topk)``. With ``token_map``
    (int [V]) row entry i stands for token ``token_map[i]`` (truncated draft
    vocabulary); ranking uses i, node tokens are mapped.
    """
    tok_of = (lambda i: int(i)) if token_map is None else (lambda i: int(token_map[i]))
    V = rows.shape[-1]
    if not (1 <= k <= V and D >= 1):
        raise ValueError("need 1 <= topk <= V and depth >= 1")
    if not (1 <= N <= pool_size(k, D)):
        raise ValueError("num_draft must be in [1, topk + (depth - 1) * topk^2]")

    pool: List[PoolEntry] = []
    frontier_tokens: List[List[int]] = []

    # step 1: the root's top-k children
    for rank, (idx, lp) in enumerate(row_topk(rows[draft_row_index(1, 0, max_topk)], k)):
        pool.append(PoolEntry(tok_of(idx), -1, 0.0 + lp, 1, frontier_slot=rank))
    frontier = list(range(k))
    frontier_tokens.append([pool[i].token for i in frontier])

    # steps 2..D: each frontier node spawns its top-k children
    for d in range(2, D + 1):
        base = len(pool)
        for f, parent in enumerate(frontier):
            row = rows[draft_row_index(d, f, max_topk)]
            for idx, lp in row_topk(row, k):
                pool.append(PoolEntry(tok_of(idx), parent, pool[parent].score + lp, d))
        cands = list(range(base, base + k * k))
        ranked = sorted(cands, key=lambda i: (-pool[i].score, i))
        frontier = ranked[:k]
        for f, i in enumerate(frontier):
            pool[i].frontier_slot = f
        frontier_tokens.append([pool[i].token for i in frontier])

    # rerank: keep the N best of the whole pool, number them in pool order
    ranked = sorted(range(len(pool)), key=lambda i: (-pool[i].score, i))
    kept = sorted(ranked[:N])
    node_of = {p: n + 1 for n, p in enumerate(kept)}

    T = N + 1
    tokens = np.empty(T, dtype=np.int32)
    parents = np.empty(T, dtype=np.int32)
    depth = np.empty(T, dtype=np.int32)
    q_row = np.full(T, -1, dtype=np.int32)
    tokens[0], parents[0], depth[0], q_row[0] = root_token, -1, 0, draft_row_index(1, 0, max_topk)
    for n, p in enumerate(kept, start=1):
        e = pool[p]
        tokens[n] = e.token
        parents[n] = 0 if e.parent < 0 else node_of[e.parent]
        depth[n] = e.depth
        if e.frontier_slot >= 0 and e.depth < D:
            # this node was expanded at step depth+1 from frontier slot f
            q_row[n] = draft_row_index(e.depth + 1, e.frontier_slot, max_topk)
    anc, _, _ = tree_mask(parents, T)
    return BuiltTree(tokens, parents, depth, anc, q_row, frontier_tokens, pool, kept)


def tree_mask(parents: Sequence[int], T: int):
    """Ancestor bitmask, depth and status for one tree of T nodes.

    anc[0] = 0; for i >= 1, anc[i] = anc[p] | bit(i - 1) with p = parents[i].
    A parent outside [0, i) sets STATUS_INVALID_PARENT and the node is treated
    as a child of the root (a reading: the pages define no invalid input).
    """
    if not (1 <= T <= 65):
        raise ValueError("a tree has 1..65 nodes (root + at most 64 drafts)")
    anc = np.zeros(T, dtype=np.uint64)
    depth = np.zeros(T, dtype=np.int32)
    status = 0
    for i in range(1, T):
        p = int(parents[i])
        if not (0 <= p < i):
            status |= STATUS_INVALID_PARENT
            p = 0
        anc[i] = np.uint64(int(anc[p]) | (1 << (i - 1)))
        depth[i] = depth[p] + 1
    return anc, depth, status

