"""Pins for the oracle's accepted-path KV compaction.

After compaction slot L_b + k holds what slot L_b + n_k held before the call
(n_k = k-th accepted draft), every other slot is unchanged, and the new
length is L_b + 1 + accept_len; checked slot by slot with a brute-force
logical view of the cache.
"""
import numpy as np

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
