"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from oracle.kvcompact import kv_prune as oracle_kv_prune
from oracle.tree import build_tree
from oracle.verify import verify_sequence
from workloads.synth import bf16_bits_to_f32

ATTN_MAX_ABS = 1e-2  # bf16 inputs, fp32 accumulation
ATTN_REL_L2 = 5e-3
LSE_ABS = 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    import torch

    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy()


def run_pipeline(w, compact=False):
    import torch

    from tree_attention_verification_03_amd.pipeline import DeviceWorkload, SpecTreeStep

    dw = DeviceWorkload(w)
    step = SpecTreeStep(dw)
    o = step.run(compact=compact)
    torch.cuda.synchronize()
    host = {k: to_np(getattr(o, k)) for k in o.__dataclass_fields__}
    return dw, step, host


def oracle_trees(w):
    return [build_tree(w.draft_logprobs[b], int(w.root_tokens[b]), int(w.topk[b]), int(w.depth[b]),
                       int(w.num_draft[b]), w.max_topk, token_map=w.token_map) for b in range(w.B)]


def check_build(w, host, trees):
    for b, t in enumerate(trees):
        T = len(t.tokens)
        assert host["tokens"][b, :T].tolist() == t.tokens.tolist(), f"tokens b={b}"
        assert host["parents"][b, :T].tolist() == t.parents.tolist(), f"parents b={b}"
        assert host["depth"][b, :T].tolist() == t.depth.tolist(), f"depth b={b}"
        assert [int(x) & 0xFFFFFFFFFFFFFFFF for x in host["anc"][b, :T]] == [int(x) for x in t.anc], f"anc b={b}"
        assert host["q_row"][b, :T].tolist() == t.q_row.tolist(), f"q_row b={b}"
        assert (host["tokens"][b, T:] == -1).all() and (host["parents"][b, T:] == -1).all()
        D = int(w.depth[b])
        k = int(w.topk[b])
        want = t.frontier_tokens[D - 1] + [-1] * (w.max_topk - k)
        assert host["frontier"][b].tolist() == want, f"frontier b={b}"


def parents_array(w, trees):
    par = np.full((w.B, w.max_T), -1, dtype=np.int32)
    for b, t in enumerate(trees):
        par[b, : len(t.parents)] = t.parents
    return par


def compare_attention(w, out_gpu, lse_gpu, parents, pairs=None):
    """Oracle on (b, h) pairs; returns (max_abs, rel_l2, max_lse_err)."""
    kf = bf16_bits_to_f32(w.k_pages)
    vf = bf16_bits_to_f32(w.v_pages)
    qf = bf16_bits_to_f32(w.q).astype(np.float64)
    ref, lref = oracle.attention.tree_attention(qf, kf, vf, w.page_table, w.prefix_lens, parents, w.T_b, w.sm_scale,
                                                batch_heads=pairs)
    mask = ~np.isnan(ref)
    diff = out_gpu[mask] - ref[mask]
    max_abs = float(np.abs(diff).max())
    rel = float(np.linalg.norm(diff) / np.linalg.norm(ref[mask]))
    lm = ~np.isnan(lref)
    lse_err = float(np.abs(lse_gpu[lm].astype(np.float64) - lref[lm]).max())
    return max_abs, rel, lse_err


def check_verify(w, host, trees, seqs=None, tokens=None, parents=None, q_row=None, target=None):
    seqs = range(w.B) if seqs is None else seqs
    target = w.target if target is None else target
    for b in seqs:
        T = int(w.T_b[b])
        tok = trees[b].tokens if tokens is None else tokens[b]
        par = trees[b].parents if parents is None else parents[b]
        qr = trees[b].q_row if q_row is None else q_row[b]
        n, nodes, out, st = verify_sequence(target[b], w.draft_probs[b], qr, tok, par, T, int(w.modes[b]),
                                            w.philox_key, w.philox_offset, b)
        assert int(host["accept_len"][b]) == n, f"accept_len b={b}: gpu {host['accept_len'][b]} oracle {n}"
        assert host["accept_nodes"][b, : n + 1].tolist() == nodes, f"accept_nodes b={b}"
        assert host["out_tokens"][b, : n + 1].tolist() == out, f"out_tokens b={b}"
        assert (host["accept_nodes"][b, n + 1 :] == -1).all() and (host["out_tokens"][b, n + 1 :] == -1).all()
        assert int(host["status"][b]) == st, f"status b={b}: gpu {host['status'][b]} oracle {st}"


def gpu_kv_prune(pt, L, T, nodes, alen, page, num_pages, mode, in_place=False):
    """spec_kv_prune on device copies (outputs pre-filled with junk); returns host arrays."""
    import torch

    from tree_attention_verification_03_amd import ops

    dev = torch.device("cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    B, max_T = nodes.shape
    tpt, tl = i32(pt), i32(L)
    junk = lambda *s: torch.full(s, 7, dtype=torch.int32, device=dev)
    freed, cnt, st = junk(B, max_T), junk(B), junk(B)
    newl = tl if in_place else junk(B)
    ops.spec_kv_prune(tpt, tl, i32(T), i32(nodes), i32(alen), page, num_pages, mode, freed, cnt, newl, st)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in (tpt, freed, cnt, newl, st))


def check_kv_prune(pt, L, T, nodes, alen, page, num_pages, mode, in_place=False):
    got = gpu_kv_prune(pt, L, T, nodes, alen, page, num_pages, mode, in_place)
    ref = oracle_kv_prune(pt, L, T, nodes, alen, page, num_pages, mode)
    for name, g, r in zip(("page_table", "freed", "freed_count", "new_prefix_lens", "status"), got, ref):
        assert np.array_equal(g.astype(np.int64), np.asarray(r, dtype=np.int64)), name
    return ref


# FP8-KV attention: the kernel rounds each softmax weight p to E4M3 before P V and sums the rounded weights, so with
# u_i = exp(s_i - max s) (p_i = u_i 2^D for some 0 <= D <= 8) a weight with u_i >= 2^-6 is a normal E4M3 value
# (relative error <= 2^-4) and any other is off by at most 2^-10 2^D, and
#   |O' - O| <= [2^-4 sum_{u >= 2^-6} u_i |v_i - O| + 2^-10 sum_{u < 2^-6} |v_i - O|] / ((1 - 2^-4) sum_{u >= 2^-6} u_i)
# per output column; plus 1e-3 relative on the scores (fp32 dot products and exp2), 2^-8 |O| for bf16 output and
# fp16 partials, and 1e-5 absolute. The lse bound is log(1 + the same relative error of the row sum).
def fp8_attention_bound(w, k8, v8, ks, vs, parents, b, h):
    """(out bound [T, d], lse bound [T]) for sequence b, query head h, from the oracle's fp64 scores."""
    from oracle.attention import gather_slots
    from oracle.fp8 import e4m3_decode, quantize_q_rows
    from oracle.tree import tree_mask

    L, T = int(w.prefix_lens[b]), int(w.T_b[b])
    g = h // (w.Hq // w.Hkv)
    K = e4m3_decode(gather_slots(k8, w.page_table[b], L + T, w.page)[:, g]) * float(ks[g])
    Vv = e4m3_decode(gather_slots(v8, w.page_table[b], L + T, w.page)[:, g]) * float(vs[g])
    q = quantize_q_rows(bf16_bits_to_f32(w.q[b, :T, h]))
    anc, _, _ = tree_mask(parents[b], T)
    ob, lb = np.zeros((T, w.d)), np.zeros(T)
    for i in range(T):
        vis = np.ones(L + T, dtype=bool)
        vis[L:] = False
        vis[L] = vis[L + i] = True
        for j in range(1, T):
            if (int(anc[i]) >> (j - 1)) & 1:
                vis[L + j] = True
        s = w.sm_scale * (K[vis] @ q[i])
        u = np.exp(s - s.max())
        O = u @ Vv[vis] / u.sum()
        dv = np.abs(Vv[vis] - O)
        nrm = u >= 2.0**-6
        den = (1 - 2.0**-4) * u[nrm].sum()
        ob[i] = ((2.0**-4 + 1e-3) * (u[nrm] @ dv[nrm]) + 2.0**-10 * dv[~nrm].sum(axis=0)) / den + 2.0**-8 * np.abs(O) + 1e-5
        lb[i] = np.log1p(((2.0**-4 + 1e-3) * u[nrm].sum() + 2.0**-10 * (~nrm).sum()) / den) + 1e-4
    return ob, lb


def check_fp8_attention(w, k8, v8, ks, vs, parents, out_gpu, lse_gpu, pairs):
    """GPU FP8-KV attention against oracle.attention.tree_attention_fp8 within fp8_attention_bound, element by
    element, on the (b, h) pairs given; returns (worst error / bound, rel L2 of the outputs)."""
    from oracle.attention import tree_attention_fp8

    q = bf16_bits_to_f32(w.q)
    ref, ref_lse = tree_attention_fp8(q, k8, v8, ks, vs, w.page_table, w.prefix_lens, parents, w.T_b, w.sm_scale,
                                      batch_heads=pairs)
    worst, num, den = 0.0, 0.0, 0.0
    for b, h in pairs:
        T = int(w.T_b[b])
        ob, lb = fp8_attention_bound(w, k8, v8, ks, vs, parents, b, h)
        err = np.abs(out_gpu[b, :T, h] - ref[b, :T, h])
        lerr = np.abs(lse_gpu[b, :T, h] - ref_lse[b, :T, h])
        worst = max(worst, float((err / ob).max()), float((lerr / lb).max()))
        num += float((err**2).sum())
        den += float((ref[b, :T, h] ** 2).sum())
        assert (err <= ob).all(), f"fp8 attention b={b} h={h}: max err {err.max():.3e}, worst ratio {(err / ob).max():.2f}"
        assert (lerr <= lb).all(), f"fp8 lse b={b} h={h}: max err {lerr.max():.3e}"
    return worst, (num / max(den, 1e-30)) ** 0.5


def run_attention_fp8(w, parents, k8, v8, ks, vs, T_b=True):
    """spec_tree_attention_fp8 on device copies; returns host (out, lse, status)."""
    import torch

    from tree_attention_verification_03_amd import ops
    from tree_attention_verification_03_amd.pipeline import bf16_tensor

    dev = torch.device("cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    out = torch.full((w.B, w.max_T, w.Hq, w.d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(w.B, w.max_T, w.Hq, dtype=torch.float32, device=dev)
    status = torch.zeros(w.B, dtype=torch.int32, device=dev)
    ops.spec_tree_attention_fp8(bf16_tensor(w.q, dev), torch.from_numpy(k8).to(dev), torch.from_numpy(v8).to(dev),
                                f32(ks), f32(vs), i32(w.page_table), i32(w.prefix_lens), i32(parents),
                                i32(w.T_b) if T_b else None, w.sm_scale, out, lse, status)
    torch.cuda.synchronize()
    return to_np(out), to_np(lse), to_np(status)


def plant_path(rng, w, trees, target, draft):
    """Make a random root->leaf path likely to be accepted (inputs only)."""
    for b, t in enumerate(trees):
        sampling = int(w.modes[b]) == 1
        u = 0
        while True:
            kids = [i for i in range(1, len(t.tokens)) if t.parents[i] == u]
            if not kids or rng.random() < 0.15:
                break
            c = kids[int(rng.integers(len(kids)))]
            if sampling:
                if t.q_row[u] >= 0:
                    draft[b, t.q_row[u]] = target[b, u]  # q == p: accepted with probability 1
            else:
                target[b, u, t.tokens[c]] = target[b, u].max() + 1.0
            u = c


def oracle_accepts(w, trees, target=None):
    """The oracle's accepted paths: (accept_nodes [B, max_T] padded with -1, accept_len [B])."""
    target = w.target if target is None else target
    nodes = np.full((w.B, w.max_T), -1, dtype=np.int64)
    alen = np.zeros(w.B, dtype=np.int64)
    for b, t in enumerate(trees):
        n, path, _, _ = verify_sequence(target[b], w.draft_probs[b], t.q_row, t.tokens, t.parents, int(w.T_b[b]),
                                        int(w.modes[b]), w.philox_key, w.philox_offset, b)
        nodes[b, : n + 1] = path
        alen[b] = n
    return nodes, alen
