"""Pins for the oracle's tree attention against torch's own attention routine.

torch.nn.functional.scaled_dot_product_attention (fp64, CPU math path) is an
independent implementation of softmax attention; the cases below reduce tree
attention to it:

* a chain tree is causal attention over prefix + path (bottom-right aligned);
* a single-node tree is plain decode attention over prefix + root;
* every node equals attention of its query over prefix + its own root->node path;
* shuffling physical pages (and the page table with them) changes nothing;
* GQA equals MHA with each KV head repeated for its query group;
* lse equals torch.logsumexp of the scaled visible scores.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.attention import gather_slots, tree_attention
from oracle.tree import tree_mask
from workloads.synth import random_parents


def _case(seed, B=2, Hq=4, Hkv=2, d=16, L=(37, 5), T=(7, 9), page=4, parents_kind="random", shuffle=True):
    rng = np.random.default_rng(seed)
    L = list(L)[:B]
    T = list(T)[:B]
    T_max = max(T)
    npages = [-(-(L[b] + T_max) // page) for b in range(B)]
    P = sum(npages)
    phys = rng.permutation(P) if shuffle else np.arange(P)
    pt = np.full((B, max(npages)), -1, dtype=np.int64)
    c = 0
    for b in range(B):
        pt[b, : npages[b]] = phys[c : c + npages[b]]
        c += npages[b]
    k = rng.normal(size=(P, page, Hkv, d))
    v = rng.normal(size=(P, page, Hkv, d))
    q = rng.normal(size=(B, T_max, Hq, d))
    parents = np.full((B, T_max), -1, dtype=np.int64)
    for b in range(B):
        parents[b, : T[b]] = random_parents(rng, T[b], parents_kind)
    return dict(q=q, k=k, v=v, pt=pt, L=np.array(L), T=np.array(T), parents=parents, page=page,
                scale=1 / np.sqrt(d), Hq=Hq, Hkv=Hkv)


def _run(c):
    return tree_attention(c["q"], c["k"], c["v"], c["pt"], c["L"], c["parents"], c["T"], c["scale"])


def _sdpa(qv, K, V, scale, mask=None):
    q = torch.from_numpy(qv)[None, None]  # [1,1,Tq,d]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("seed", range(3))
def test_chain_tree_is_causal_attention(seed):
    c = _case(seed, parents_kind="chain")
    out, _ = _run(c)
    G = c["Hq"] // c["Hkv"]
    for b in range(2):
        L, T = int(c["L"][b]), int(c["T"][b])
        K = gather_slots(c["k"], c["pt"][b], L + T, c["page"])
        V = gather_slots(c["v"], c["pt"][b], L + T, c["page"])
        mask = np.tril(np.ones((T, L + T), dtype=bool), k=L)  # bottom-right causal
        for h in range(c["Hq"]):
            ref = _sdpa(c["q"][b, :T, h], K[:, h // G], V[:, h // G], c["scale"], mask)
            np.testing.assert_allclose(out[b, :T, h], ref, rtol=0, atol=1e-12)


def test_single_node_tree_is_decode_attention():
    c = _case(11, T=(1, 1))
    out, _ = _run(c)
    G = c["Hq"] // c["Hkv"]
    for b in range(2):
        L = int(c["L"][b])
        K = gather_slots(c["k"], c["pt"][b], L + 1, c["page"])
        V = gather_slots(c["v"], c["pt"][b], L + 1, c["page"])
        for h in range(c["Hq"]):
            ref = _sdpa(c["q"][b, :1, h], K[:, h // G], V[:, h // G], c["scale"])
            np.testing.assert_allclose(out[b, 0, h], ref[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_each_node_is_attention_over_its_own_path(seed):
    c = _case(100 + seed, T=(13, 17))
    out, lse = _run(c)
    G = c["Hq"] // c["Hkv"]
    for b in range(2):
        L, T = int(c["L"][b]), int(c["T"][b])
        K = gather_slots(c["k"], c["pt"][b], L + T, c["page"])
        V = gather_slots(c["v"], c["pt"][b], L + T, c["page"])
        for i in range(T):
            path = []
            j = i
            while True:
                path.append(j)
                if j == 0:
                    break
                j = int(c["parents"][b, j])
            slots = list(range(L)) + [L + j for j in reversed(path)]
            for h in range(c["Hq"]):
                Kp, Vp = K[slots, h // G], V[slots, h // G]
                ref = _sdpa(c["q"][b, i : i + 1, h], Kp, Vp, c["scale"])
                np.testing.assert_allclose(out[b, i, h], ref[0], rtol=0, atol=1e-12)
                s = torch.from_numpy(c["scale"] * (Kp @ c["q"][b, i, h]))
                assert abs(float(torch.logsumexp(s, 0)) - lse[b, i, h]) < 1e-12


def test_page_permutation_invariance():
    a = _case(7, shuffle=False)
    b = _case(7, shuffle=True)
    # same logical content: re-lay b's pool so each logical slot matches a's
    P = a["k"].shape[0]
    k2 = np.empty_like(a["k"])
    v2 = np.empty_like(a["v"])
    for bb in range(2):
        for lp in range(a["pt"].shape[1]):
            pa, pb = a["pt"][bb, lp], b["pt"][bb, lp]
            if pa >= 0:
                k2[pb] = a["k"][pa]
                v2[pb] = a["v"][pa]
    assert P == b["k"].shape[0]
    b["k"], b["v"], b["q"], b["parents"] = k2, v2, a["q"], a["parents"]
    oa, la = _run(a)
    ob, lb = _run(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_gqa_equals_mha_with_repeated_kv():
    c = _case(21, Hq=8, Hkv=2)
    out_gqa, lse_gqa = _run(c)
    G = 4
    m = dict(c)
    m["k"] = np.repeat(c["k"], G, axis=2)
    m["v"] = np.repeat(c["v"], G, axis=2)
    m["Hkv"] = 8
    out_mha, lse_mha = _run(m)
    np.testing.assert_array_equal(np.isnan(out_gqa), np.isnan(out_mha))
    np.testing.assert_allclose(out_gqa, out_mha, rtol=0, atol=1e-13, equal_nan=True)
    np.testing.assert_allclose(lse_gqa, lse_mha, rtol=0, atol=1e-13, equal_nan=True)


def test_padding_nodes_are_not_written():
    c = _case(3, T=(3, 9))
    out, lse = _run(c)
    assert np.isnan(out[0, 3:]).all() and np.isnan(lse[0, 3:]).all()
    assert np.isfinite(out[1]).all()
