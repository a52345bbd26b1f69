"""Tree attention over a paged prefix KV cache plus each node's own ancestors.

Definition (tanhdev "Tech Radar: SGLang EAGLE-2", section 2 "Dynamic
Tree-Attention Verification": candidate i attends to j iff j is an ancestor of
i or i itself; n1n.ai "Speculative Decoding in Production: EAGLE-3 Dynamic
Trees", section "From Linear Sequences to Dynamic Draft Trees": the tree is
flattened into one sequence evaluated in a single pass; lesty.tech "EAGLE-2 &
Lookahead Decoding", section 4 "Tree Attention Masking and Target
Verification": the masked tree runs through paged attention).

For sequence b, query head h and tree node i (i < T_b):

* KV head g = h // (Hq / Hkv) (contiguous GQA grouping - a reading);
* keys/values: every prefix slot 0..L_b-1, and the tree slots L_b + j for the
  root j = 0, every ancestor j of i and j = i (node j's K/V sits at slot
  L_b + j of the same paged cache - a reading of the flattened layout);
* slot s lives in page page_table[b, s // page] at offset s % page;
* out = softmax(sm_scale * q.k) @ v over those keys, lse = log-sum-exp of the
  scaled scores (natural log), all in fp64.
"""
from __future__ import annotations

import numpy as np

from .tree import tree_mask


def gather_slots(pages: np.ndarray, page_table_b: np.ndarray, n_slots: int, page: int) -> np.ndarray:
    """[n_slots, Hkv, d] view of a sequence's slots 0..n_slots-1 through its page table."""
    s = np.arange(n_slots)
    phys = page_table_b[s // page]
    if n_slots and (phys.min() < 0 or phys.max() >= pages.shape[0]):
        raise ValueError("page table points outside the KV pool")
    return pages[phys, s % page]


def tree_attention(q, k_pages, v_pages, page_table, prefix_lens, parents, T_b, sm_scale,
                   batch_heads=None, kv_values=None):
    """Reference tree attention.

    q: [B, T_max, Hq, d]; k_pages, v_pages: [P, page, Hkv, d] (any float dtype,
    converted exactly to fp64); page_table: [B, max_pages]; prefix_lens, T_b:
    [B]; parents: [B, T_max]. ``batch_heads`` optionally restricts the work to
    a list of (b, h) pairs (other outputs stay NaN). ``kv_values(slots, which)`` optionally maps a sequence's
    gathered K (which = 0) or V (which = 1) slots [n, Hkv, d] to their fp64 values (default: the stored values).
    Returns (out [B, T_max, Hq, d] fp64, lse [B, T_max, Hq] fp64); entries of
    nodes i >= T_b are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k_pages = np.asarray(k_pages)
    v_pages = np.asarray(v_pages)
    B, T_max, Hq, d = q.shape
    page = k_pages.shape[1]
    Hkv = k_pages.shape[2]
    G = Hq // Hkv
    out = np.full((B, T_max, Hq, d), np.nan)
    lse = np.full((B, T_max, Hq), np.nan)
    todo = {}
    if batch_heads is None:
        for b in range(B):
            todo[b] = list(range(Hq))
    else:
        for b, h in batch_heads:
            todo.setdefault(int(b), []).append(int(h))

    for b, heads in todo.items():
        L = int(prefix_lens[b])
        T = int(T_b[b])
        anc, _, _ = tree_mask(parents[b], T)
        K = gather_slots(k_pages, page_table[b], L + T, page)
        Vv = gather_slots(v_pages, page_table[b], L + T, page)
        K, Vv = (K.astype(np.float64), Vv.astype(np.float64)) if kv_values is None else (kv_values(K, 0), kv_values(Vv, 1))
        # allowed[i, s]: does node i see slot s?
        allowed = np.zeros((T, L + T), dtype=bool)
        allowed[:, :L] = True
        for i in range(T):
            allowed[i, L] = True  # the root
            allowed[i, L + i] = True  # itself
            for j in range(1, T):
                if (int(anc[i]) >> (j - 1)) & 1:
                    allowed[i, L + j] = True
        for h in heads:
            g = h // G
            s = sm_scale * (q[b, :T, h, :] @ K[:, g, :].T)  # [T, L+T]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            out[b, :T, h, :] = (e @ Vv[:, g, :]) / z
            lse[b, :T, h] = (m + np.log(z))[:, 0]
    return out, lse


def tree_attention_fp8(q, k8_pages, v8_pages, k_scale, v_scale, page_table, prefix_lens, parents, T_b, sm_scale,
                       batch_heads=None):
    """The FP8-KV variant: K and V stored as E4M3 codes with one fp32 scale per KV head (value = code value *
    scale[g]), q quantized per row as oracle.fp8 defines; then the same tree attention as above, in fp64.

    Sources and readings: oracle.fp8 (the pages name FP8 targets but fix no format). q: [B, T_max, Hq, d] float;
    k8_pages, v8_pages: uint8 [P, page, Hkv, d]; k_scale, v_scale: [Hkv].
    """
    from .fp8 import e4m3_decode, quantize_q_rows

    scales = (np.asarray(k_scale, dtype=np.float64)[None, :, None], np.asarray(v_scale, dtype=np.float64)[None, :, None])
    return tree_attention(quantize_q_rows(q), k8_pages, v8_pages, page_table, prefix_lens, parents, T_b, sm_scale,
                          batch_heads, kv_values=lambda codes, which: e4m3_decode(codes) * scales[which])
