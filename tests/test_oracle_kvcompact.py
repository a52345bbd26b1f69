"""Pins for the oracle's accepted-path KV compaction.

After compaction slot L_b + k holds what slot L_b + n_k held before the call
(n_k = k-th accepted draft), every other slot is unchanged, and the new
length is L_b + 1 + accept_len; checked slot by slot with a brute-force
logical view of the cache.
"""
import numpy as np
import pytest

from oracle.kvcompact import kv_compact


def _logical(pages, pt, n, page):
    return np.stack([pages[:, pt[s // page], s % page] for s in range(n)], axis=1)


def test_compaction_moves_accepted_slots_only():
    rng = np.random.default_rng(0)
    page, Hkv, d, layers = 4, 2, 8, 3
    L = [5, 9, 0]
    T = 8
    npg = [-(-(l + T) // page) for l in L]
    P = sum(npg) + 2
    phys = rng.permutation(P)
    pt = np.full((3, max(npg)), -1)
    c = 0
    for b in range(3):
        pt[b, : npg[b]] = phys[c : c + npg[b]]
        c += npg[b]
    k = rng.normal(size=(layers, P, page, Hkv, d))
    v = rng.normal(size=(layers, P, page, Hkv, d))
    accept_nodes = [[0, 1, 3, 6, -1, -1, -1, -1], [0, 2, -1, -1, -1, -1, -1, -1], [0] + [-1] * 7]
    accept_len = [3, 1, 0]
    k2, v2, lens = kv_compact(k, v, pt, L, accept_nodes, accept_len, page)
    assert lens.tolist() == [L[b] + 1 + accept_len[b] for b in range(3)]
    for b in range(3):
        n = L[b] + T
        before_k, after_k = _logical(k, pt[b], n, page), _logical(k2, pt[b], n, page)
        before_v, after_v = _logical(v, pt[b], n, page), _logical(v2, pt[b], n, page)
        moved = {L[b] + j: L[b] + accept_nodes[b][j] for j in range(1, accept_len[b] + 1)}
        for s in range(n):
            src = moved.get(s, s)
            np.testing.assert_array_equal(after_k[:, s], before_k[:, src])
            np.testing.assert_array_equal(after_v[:, s], before_v[:, src])
    # pages owned by nobody are untouched
    spare = [p for p in range(P) if p not in set(pt[pt >= 0].tolist())]
    for p in spare:
        np.testing.assert_array_equal(k2[:, p], k[:, p])


# ---------------------------------------------------------------------------------------------------------------
# Page-table pruning. Pinned against brute force over the logical view: after pruning, the logical slots below the
# new length read exactly what the oracle's (separately pinned) compaction leaves there, no page is both live and
# returned, every page the tree held comes back exactly once or stays live, and nothing outside the tree changes.

from oracle.kvcompact import PRUNE_REMAP, PRUNE_TAIL, kv_prune  # noqa: E402


def _random_path(rng, T):
    """A random root-to-node path of a random tree with T nodes: (parents, accepted nodes n_1 < ... < n_a)."""
    parents = [-1] + [int(rng.integers(0, i)) for i in range(1, T)]
    node = int(rng.integers(0, T))
    path = []
    while node > 0:
        path.append(node)
        node = parents[node]
    return path[::-1]


def _prune_case(rng, B, page, max_T=12, spare=3):
    L = [int(x) for x in rng.integers(0, 3 * page + 5, size=B)]
    T = [int(x) for x in rng.integers(1, max_T + 1, size=B)]
    npg = [-(-(L[b] + T[b]) // page) for b in range(B)]
    max_pages = max(npg) + 1
    P = sum(npg) + spare
    phys = rng.permutation(P)
    pt = np.full((B, max_pages), -1, dtype=np.int64)
    c = 0
    for b in range(B):
        pt[b, : npg[b]] = phys[c : c + npg[b]]
        c += npg[b]
    nodes = np.full((B, max_T), -1, dtype=np.int64)
    alen = np.zeros(B, dtype=np.int64)
    for b in range(B):
        path = _random_path(rng, T[b])
        nodes[b, 0] = 0
        nodes[b, 1 : 1 + len(path)] = path
        alen[b] = len(path)
    return L, T, pt, P, nodes, alen


def _view(pool, pt_row, n, page):
    return np.stack([pool[:, int(pt_row[s // page]), s % page] for s in range(n)], axis=1)


def _check_prune(L, T, pt, P, nodes, alen, page, mode, rng):
    B = len(L)
    layers, Hkv, d = 2, 2, 4
    k = rng.normal(size=(layers, P, page, Hkv, d))
    v = rng.normal(size=(layers, P, page, Hkv, d))
    kc, vc, clens = kv_compact(k, v, pt, L, nodes, alen, page)
    new_pt, freed, count, lens, status = kv_prune(pt, L, T, nodes, alen, page, P, mode)
    assert (status == 0).all()
    np.testing.assert_array_equal(lens, clens)
    # REMAP moves nothing, so the view is read from the untouched pool; TAIL reads the compacted pool
    kk, vv = (k, v) if mode == PRUNE_REMAP else (kc, vc)
    for b in range(B):
        n = int(lens[b])
        np.testing.assert_array_equal(_view(kk, new_pt[b], n, page), _view(kc, pt[b], n, page))
        np.testing.assert_array_equal(_view(vv, new_pt[b], n, page), _view(vc, pt[b], n, page))
        got = freed[b, : count[b]].tolist()
        assert (freed[b, count[b]:] == -1).all()
        assert len(got) == len(set(got))
        live = {int(new_pt[b, s // page]) for s in range(n)}
        before = {int(pt[b, s // page]) for s in range(L[b] + T[b])}
        assert not live & set(got)
        assert live | set(got) == before  # every page the sequence held is live or returned, none twice
        for i in range(-(-n // page), pt.shape[1]):  # past the new length: the tree's entries cleared, others kept
            assert new_pt[b, i] == (-1 if i <= (L[b] + T[b] - 1) // page else pt[b, i])
        if mode == PRUNE_REMAP:
            path = set(nodes[b, : alen[b] + 1].tolist())
            assert got == [int(pt[b, L[b] + i]) for i in range(1, T[b]) if i not in path]
        np.testing.assert_array_equal(new_pt[b, : L[b] // page], pt[b, : L[b] // page])  # prefix pages untouched
    return new_pt, freed, count


def test_prune_remap_matches_compaction_view():
    """page 1: the zero-copy remap reads what compaction wrote, and returns exactly the rejected nodes' slots."""
    rng = np.random.default_rng(11)
    for _ in range(25):
        case = _prune_case(rng, 4, 1)
        _check_prune(*case, 1, PRUNE_REMAP, rng)


def test_prune_tail_after_compaction():
    """Any page size: after compaction the pages past the new length that the tree touched come back."""
    rng = np.random.default_rng(12)
    for page in (1, 2, 4, 16):
        for _ in range(15):
            case = _prune_case(rng, 4, page)
            _check_prune(*case, page, PRUNE_TAIL, rng)


def test_prune_special_cases():
    # all of a chain accepted: REMAP leaves the table as it was and frees nothing
    pt = np.arange(20).reshape(1, 20)
    nodes = np.array([[0, 1, 2, 3, 4, 5]])
    new_pt, freed, count, lens, status = kv_prune(pt, [10], [6], nodes, [5], 1, 20, PRUNE_REMAP)
    np.testing.assert_array_equal(new_pt, pt)
    assert count[0] == 0 and lens[0] == 16 and status[0] == 0
    # nothing accepted: every draft slot is returned, the root's stays
    new_pt, freed, count, lens, status = kv_prune(pt, [10], [6], nodes, [0], 1, 20, PRUNE_REMAP)
    assert freed[0, :5].tolist() == [11, 12, 13, 14, 15] and count[0] == 5 and lens[0] == 11
    assert new_pt[0, 10] == 10 and (new_pt[0, 11:16] == -1).all() and (new_pt[0, 16:] == pt[0, 16:]).all()
    # a root-only tree returns nothing in either mode
    for mode in (PRUNE_REMAP, PRUNE_TAIL):
        _, _, count, lens, _ = kv_prune(pt, [3], [1], nodes, [0], 1, 20, mode)
        assert count[0] == 0 and lens[0] == 4
    # TAIL, page 4, L = 6, T = 9 (slots 6..14, pages 1..3), one accepted: L' = 8, pages 2 and 3 come back
    pt4 = np.array([[7, 3, 9, 1, 5]])
    new_pt, freed, count, lens, _ = kv_prune(pt4, [6], [9], np.array([[0, 4] + [-1] * 7]), [1], 4, 10, PRUNE_TAIL)
    assert freed[0, :2].tolist() == [9, 1] and count[0] == 2 and lens[0] == 8
    assert new_pt[0].tolist() == [7, 3, -1, -1, 5]
    # the same with L' on a page boundary's far side: L = 6, a = 2 -> L' = 9, page 2 (slots 8..11) keeps slot 8
    new_pt, freed, count, lens, _ = kv_prune(pt4, [6], [9], np.array([[0, 4, 7] + [-1] * 6]), [2], 4, 10, PRUNE_TAIL)
    assert freed[0, :1].tolist() == [1] and count[0] == 1 and new_pt[0].tolist() == [7, 3, 9, -1, 5]


def test_prune_invalid_inputs():
    pt = np.arange(20).reshape(1, 20)
    # path not increasing
    new_pt, _, count, lens, status = kv_prune(pt, [4], [6], np.array([[0, 3, 2, 0, 0, 0]]), [2], 1, 20, PRUNE_REMAP)
    assert status[0] == 128 and count[0] == 0 and lens[0] == 4 and (new_pt == pt).all()
    # node past the tree, accept_len past the tree
    assert kv_prune(pt, [4], [3], np.array([[0, 3, 0, 0, 0, 0]]), [1], 1, 20, PRUNE_REMAP)[4][0] == 128
    assert kv_prune(pt, [4], [3], np.array([[0, 1, 2, 0, 0, 0]]), [3], 1, 20, PRUNE_TAIL)[4][0] == 128
    # tree past the table, negative prefix
    assert kv_prune(pt, [16], [5], np.array([[0] * 6]), [0], 1, 20, PRUNE_TAIL)[4][0] == 64
    r = kv_prune(pt, [-2], [5], np.array([[0] * 6]), [0], 1, 20, PRUNE_TAIL)
    assert r[4][0] == 64 and r[3][0] == 0
    # entries outside the pool are cleared but never returned
    bad = pt.copy()
    bad[0, 6] = 99
    new_pt, freed, count, _, status = kv_prune(bad, [4], [5], np.array([[0, 3, 0, 0, 0, 0]]), [1], 1, 20, PRUNE_REMAP)
    assert status[0] == 32 and freed[0, :count[0]].tolist() == [5, 8] and new_pt[0, 5] == 7
    with pytest.raises(ValueError):
        kv_prune(pt, [4], [5], np.array([[0] * 6]), [0], 4, 20, PRUNE_REMAP)
