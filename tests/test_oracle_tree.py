"""Pins for the oracle's tree construction and tree mask.

Checks against: a hand-worked example (tests/golden/tree_build_handworked.json),
special cases that reduce to plain argmax / top-k / the whole pool, structural
invariants that any layer-wise top-k expansion with reranking must satisfy, and
a brute-force parent walk for the ancestor bitmask.
"""
import json
import os

import numpy as np
import pytest

from oracle.tree import (
    STATUS_INVALID_PARENT,
    build_tree,
    draft_row_index,
    pool_size,
    tree_mask,
)
from workloads import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_handworked_example():
    with open(os.path.join(GOLDEN, "tree_build_handworked.json")) as f:
        g = json.load(f)
    rows = np.array(g["rows"], dtype=np.float32)
    t = build_tree(rows, g["root_token"], g["topk"], g["depth"], g["num_draft"], g["max_topk"])
    e = g["expect"]
    assert t.tokens.tolist() == e["tokens"]
    assert t.parents.tolist() == e["parents"]
    assert t.depth.tolist() == e["depth"]
    assert [int(x) for x in t.anc] == e["anc"]
    assert t.q_row.tolist() == e["q_row"]
    assert t.frontier_tokens == e["frontier_tokens"]


def _rows(seed, R, V):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, 2, size=(R, V))
    lp = z - z.max(axis=1, keepdims=True)
    lp = lp - np.log(np.exp(lp).sum(axis=1, keepdims=True))
    return lp.astype(np.float32)


@pytest.mark.parametrize("D", [1, 2, 5])
def test_topk1_is_argmax_chain(D):
    rows = _rows(D, 1 + (D - 1), 50)
    t = build_tree(rows, 7, 1, D, D, 1)
    assert t.parents.tolist() == [-1] + list(range(D))
    expect = [int(np.argmax(rows[draft_row_index(d, 0, 1)])) for d in range(1, D + 1)]
    assert t.tokens[1:].tolist() == expect


def test_depth1_is_topN_of_root_row():
    rows = _rows(3, 1, 100)
    t = build_tree(rows, 0, 10, 1, 6, 10)
    top = np.argsort(-rows[0].astype(np.float64), kind="stable")[:6]
    # nodes are numbered in pool (= rank) order, so they appear best-first
    assert t.tokens[1:].tolist() == top.tolist()
    assert t.parents.tolist() == [-1] + [0] * 6


@pytest.mark.parametrize("k,D", [(2, 3), (3, 2), (4, 3)])
def test_full_pool_is_kept(k, D):
    rows = _rows(k * 10 + D, 1 + (D - 1) * k, 40)
    n = pool_size(k, D)
    if n > 64:
        pytest.skip("pool larger than one mask word")
    t = build_tree(rows, 0, k, D, n, k)
    assert [t.tokens[i + 1] for i in range(n)] == [e.token for e in t.pool]


def _check_invariants(t, k, D, N):
    T = N + 1
    assert t.parents[0] == -1 and t.depth[0] == 0
    kids = {}
    for i in range(1, T):
        p = int(t.parents[i])
        assert 0 <= p < i
        assert t.depth[i] == t.depth[p] + 1 <= D
        kids.setdefault(p, []).append(int(t.tokens[i]))
    for p, toks in kids.items():
        assert len(toks) <= k
        assert len(set(toks)) == len(toks), "sibling tokens must be distinct"
    for i in range(T):
        assert bin(int(t.anc[i])).count("1") == t.depth[i]
    scores = np.array([e.score for e in t.pool])
    kept = set(t.kept)
    for p in t.kept:  # scores never increase down a path
        par = t.pool[p].parent
        if par >= 0:
            assert t.pool[p].score <= t.pool[par].score
    if len(kept) < len(t.pool):
        lo = min(scores[list(kept)])
        hi = max(scores[[i for i in range(len(t.pool)) if i not in kept]])
        assert lo >= hi


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(1, 6))
    D = int(rng.integers(1, 6))
    n = pool_size(k, D)
    N = int(rng.integers(1, min(n, 64) + 1))
    rows = _rows(seed, 1 + (D - 1) * k, 60)
    t = build_tree(rows, 3, k, D, N, k)
    _check_invariants(t, k, D, N)
    # each step's frontier is the top-k of that step's k*k candidates
    for d in range(2, D + 1):
        base = k + (d - 2) * k * k
        idx = np.arange(base, base + k * k)
        sc = np.array([t.pool[i].score for i in idx])
        order = idx[np.lexsort((idx, -sc))][:k]
        assert t.frontier_tokens[d - 1] == [t.pool[i].token for i in order]


def test_workload_trees_satisfy_invariants():
    w = make_workload(B=3, Hq=4, Hkv=2, d=64, prefix=32, topk=(2, 4), depth=(2, 4), num_draft=10,
                      V=200, seed=5)
    for b in range(w.B):
        t = build_tree(w.draft_logprobs[b], int(w.root_tokens[b]), int(w.topk[b]), int(w.depth[b]),
                       int(w.num_draft[b]), w.max_topk)
        _check_invariants(t, int(w.topk[b]), int(w.depth[b]), int(w.num_draft[b]))


def test_nan_and_positive_logprobs_are_clamped():
    rows = np.array([[np.nan, 0.5, -0.0, -1.0]], dtype=np.float32)
    t = build_tree(rows, 0, 3, 1, 3, 3)
    # +0.5 and -0.0 clamp to 0 (tie -> token order), NaN is -inf and ranks last
    assert t.tokens[1:].tolist() == [1, 2, 3]


@pytest.mark.parametrize("seed", range(20))
def test_mask_equals_parent_walk(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 66))
    parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)])
    anc, depth, status = tree_mask(parents, T)
    assert status == 0
    for i in range(T):
        walk = set()
        j = i
        while j != 0:
            walk.add(j)
            j = parents[j]
        bits = {j for j in range(1, T) if (int(anc[i]) >> (j - 1)) & 1}
        assert bits == walk
        assert depth[i] == len(walk)


def test_mask_invalid_parent_becomes_root_child():
    parents = [-1, 0, 5, 1]
    anc, depth, status = tree_mask(parents, 4)
    assert status == STATUS_INVALID_PARENT
    assert [int(x) for x in anc] == [0, 0b001, 0b010, 0b101]
    assert depth.tolist() == [0, 1, 1, 2]


# ---- truncated draft vocabulary (token map)
def _same_tree(a, b):
    assert a.tokens.tolist() == b.tokens.tolist()
    assert a.parents.tolist() == b.parents.tolist()
    assert a.depth.tolist() == b.depth.tolist()
    assert [int(x) for x in a.anc] == [int(x) for x in b.anc]
    assert a.q_row.tolist() == b.q_row.tolist()
    assert a.frontier_tokens == b.frontier_tokens


def _scatter_rows(rows, token_map, V):
    full = np.full(rows.shape[:-1] + (V,), -np.inf, dtype=np.float32)
    full[..., token_map] = rows
    return full


@pytest.mark.parametrize("seed", range(4))
def test_token_map_identity_changes_nothing(seed):
    w = make_workload(B=1, Hq=2, Hkv=1, d=64, prefix=8, topk=4, depth=4, num_draft=30, V=300, seed=seed)
    plain = build_tree(w.draft_logprobs[0], 5, 4, 4, 30, 4)
    mapped = build_tree(w.draft_logprobs[0], 5, 4, 4, 30, 4, token_map=np.arange(300))
    _same_tree(plain, mapped)


@pytest.mark.parametrize("seed", range(4))
def test_token_map_monotone_equals_full_vocabulary_with_ties(seed):
    """A subset listed in increasing token order ranks ties the same way by index and by token, so the
    truncated build equals the full-vocabulary build on rows that are -inf outside the subset, even with
    ties (log-probs quantised to halves)."""
    rng = np.random.default_rng(seed)
    V, Vd, k, D, N = 1000, 120, 5, 4, 50
    token_map = np.sort(rng.choice(V, size=Vd, replace=False))
    rows = np.round(rng.normal(-6.0, 2.0, size=(1 + (D - 1) * k, Vd)) * 2.0) / 2.0
    rows = np.minimum(rows, 0.0).astype(np.float32)
    t_map = build_tree(rows, 7, k, D, N, k, token_map=token_map)
    t_full = build_tree(_scatter_rows(rows, token_map, V), 7, k, D, N, k)
    _same_tree(t_map, t_full)
    assert set(t_map.tokens[1:].tolist()) <= set(token_map.tolist())


@pytest.mark.parametrize("seed", range(4))
def test_token_map_random_order_equals_full_vocabulary_without_ties(seed):
    w = make_workload(B=1, Hq=2, Hkv=1, d=64, prefix=8, topk=6, depth=5, num_draft=64, V=4000, draft_vocab=512,
                      seed=seed)
    assert w.draft_logprobs.shape[-1] == 512 and len(set(w.token_map.tolist())) == 512
    assert not (np.diff(w.token_map) > 0).all()  # not in token order
    t_map = build_tree(w.draft_logprobs[0], 3, 6, 5, 64, 6, token_map=w.token_map)
    t_full = build_tree(_scatter_rows(w.draft_logprobs[0], w.token_map, 4000), 3, 6, 5, 64, 6)
    _same_tree(t_map, t_full)


def test_truncated_workload_draft_probabilities():
    w = make_workload(B=2, Hq=2, Hkv=1, d=64, prefix=8, topk=4, depth=3, num_draft=12, V=2000, draft_vocab=300,
                      verify="sample", seed=11)
    outside = np.setdiff1d(np.arange(2000), w.token_map)
    assert (w.draft_probs[:, :, outside] == 0).all()
    np.testing.assert_allclose(w.draft_probs.sum(axis=-1), 1.0, rtol=1e-5)
    np.testing.assert_allclose(np.exp(w.draft_logprobs.astype(np.float64)), w.draft_probs[:, :, w.token_map],
                               rtol=1e-6, atol=1e-12)
