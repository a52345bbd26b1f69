"""Accepted-path KV compaction and page-table pruning of rejected branches (test infrastructure: the CPU
oracle the HIP library is checked against; only tests, the smoke check and the bench's CPU baseline use it).

Source: tanhdev "Tech Radar: SGLang EAGLE-2", section 2 sequence diagram (the
target retains the accepted path's KV and discards rejected branches);
lesty.tech "EAGLE-2 & Lookahead Decoding", section 6 "Paged Tree KV-Cache
Allocation" (rejected candidates' blocks are recycled).

Reading: tree node j's K/V sits at slot L_b + j. After verification the root
stays at slot L_b and the k-th accepted draft n_k (k = 1..accept_len, path
order) moves to slot L_b + k, for every layer and KV head; the new length is
L_b + 1 + accept_len. Defined on the cache as it was before the call (all
sources are read before any slot is overwritten).
"""
from __future__ import annotations

import numpy as np


def kv_compact(k_layers, v_layers, page_table, prefix_lens, accept_nodes, accept_len, page):
    """k_layers, v_layers: [num_layers, P, page, Hkv, d] arrays (returned as new copies)."""
    k_old, v_old = np.asarray(k_layers), np.asarray(v_layers)
    k_new, v_new = k_old.copy(), v_old.copy()
    B = len(prefix_lens)
    new_lens = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = int(prefix_lens[b])
        a = int(accept_len[b])
        for j in range(1, a + 1):
            src = L + int(accept_nodes[b][j])
            dst = L + j
            ps, os_ = int(page_table[b][src // page]), src % page
            pd, od = int(page_table[b][dst // page]), dst % page
            k_new[:, pd, od] = k_old[:, ps, os_]
            v_new[:, pd, od] = v_old[:, ps, os_]
        new_lens[b] = L + 1 + a
    return k_new, v_new, new_lens


PRUNE_TAIL = 0
PRUNE_REMAP = 1
STATUS_INVALID_PAGE = 32
STATUS_INVALID_LENGTH = 64
STATUS_INVALID_PATH = 128


def kv_prune(page_table, prefix_lens, T_b, accept_nodes, accept_len, page, num_pages, mode):
    """Page-table pruning of rejected branches: no KV moves, only the logical-to-physical map changes.

    Sources: tanhdev "Tech Radar: SGLang EAGLE-2", section 4 "Production Failure Modes", Failure Mode 2
    "KV Cache Memory Fragmentation" (the tree cache tracks candidate ancestry and prunes discarded branches
    without copying); lesty.tech "EAGLE-2 & Lookahead Decoding", section 6 "Paged Tree KV-Cache Allocation"
    (the physical blocks of rejected candidates go straight back to the free pool).

    Reading: sequence b's tree took logical slots L .. L + T - 1 (node i at L + i). Its accepted path is
    n_0 = 0 (the root) and n_1 < ... < n_a from verification. Afterwards the path must read, in order, at
    logical slots L .. L + a, and the new length is L' = L + 1 + a.

    mode PRUNE_REMAP (page == 1, one slot per table entry): zero-copy. Entry L + j takes the old entry of
    slot L + n_j (j = 1..a); entries L + a + 1 .. L + T - 1 become -1; the old entries of the T - 1 - a
    rejected nodes are returned, in node order.
    mode PRUNE_TAIL (any page size; the accepted KV was already moved to slots L + 1 .. L + a, e.g. by
    kv_compact): the pages whose slots all lie at or past L' but that the tree touched, logical pages
    ceil(L' / page) .. floor((L + T - 1) / page), are returned in logical order and their entries become -1.

    Entries outside [0, num_pages) are never returned (bit 32). A sequence whose length or path is invalid
    (T outside [1, max_T], L < 0, L + T past the table, a outside [0, T - 1], nodes not strictly increasing
    within [1, T - 1]) keeps its table, returns nothing and gets new length max(L, 0) (bit 64 for the length,
    bit 128 for the path).

    Returns (new page table, freed [B, max_T] padded with -1, freed_count [B], new_lens [B], status [B]).
    """
    if mode == PRUNE_REMAP and page != 1:
        raise ValueError("PRUNE_REMAP needs one slot per table entry (page == 1)")
    pt = np.array(page_table, dtype=np.int64)
    B, max_pages = pt.shape
    max_T = np.asarray(accept_nodes).shape[1]
    freed = np.full((B, max_T), -1, dtype=np.int64)
    count = np.zeros(B, dtype=np.int64)
    new_lens = np.zeros(B, dtype=np.int64)
    status = np.zeros(B, dtype=np.int64)
    for b in range(B):
        L, T, a = int(prefix_lens[b]), int(T_b[b]), int(accept_len[b])
        new_lens[b] = max(L, 0)
        if not (1 <= T <= max_T and L >= 0 and L + T <= max_pages * page):
            status[b] |= STATUS_INVALID_LENGTH
            continue
        path = [0] + [int(accept_nodes[b][j]) for j in range(1, a + 1)] if 0 <= a <= T - 1 else None
        if path is None or any(not (path[j - 1] < path[j] < T) for j in range(1, len(path))):
            status[b] |= STATUS_INVALID_PATH
            continue
        new_lens[b] = L + 1 + a
        out = []
        if mode == PRUNE_REMAP:
            old = [int(pt[b, L + i]) for i in range(T)]
            for j in range(1, a + 1):
                pt[b, L + j] = old[path[j]]
            for i in range(a + 1, T):
                pt[b, L + i] = -1
            on_path = set(path)
            for i in range(1, T):
                if not 0 <= old[i] < num_pages:
                    status[b] |= STATUS_INVALID_PAGE
                elif i not in on_path:
                    out.append(old[i])
        else:
            first = -(-(L + 1 + a) // page)
            last = (L + T - 1) // page
            for p in range(first, last + 1):
                e = int(pt[b, p])
                pt[b, p] = -1
                if 0 <= e < num_pages:
                    out.append(e)
                else:
                    status[b] |= STATUS_INVALID_PAGE
        freed[b, : len(out)] = out
        count[b] = len(out)
    return pt, freed, count, new_lens, status
