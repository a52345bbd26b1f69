"""Accepted-path KV compaction.

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
