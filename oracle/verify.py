"""Tree verification: greedy, or rejection sampling with residual resampling.

Sources: n1n.ai "Speculative Decoding in Production: EAGLE-3 Dynamic Trees",
section "Mathematical Proof of Lossless Speedup" (step 1: alpha = min(1, p/q);
step 2: draw r ~ U(0, 1), accept iff r <= alpha, else stop the branch; step 3:
on rejection draw from norm(max(0, p - q))) and section "From Linear Sequences
to Dynamic Draft Trees" (if B1 is rejected but B2 matches, B2 -> C2 is
accepted); tanhdev "Tech Radar: SGLang EAGLE-2", section 5 "Speculative
Rejection Sampling: Mathematical Invariance" (the output marginal equals the
target; the accept mass is sum_v min(M(v), D(v))); lesty.tech "EAGLE-2 &
Lookahead Decoding", "Tree Attention Masking and Target Verification" (the
longest valid path is accepted, then the next token is emitted).

Readings (the pages state the single-candidate rule only):

Greedy. a_u = argmax of node u's target row (ties -> smallest index, NaN
counts as -inf). Node i is valid iff its parent is valid and tokens[i] equals
a_parent. The end node e is the valid node of largest depth (ties -> smallest
index). Emitted: the drafts on root -> e, then the bonus a_e.

Sampling at node u (probabilities supplied by the caller, temperature already
applied). Probabilities become 2^-32 fixed point, fx(x) = 0 for NaN or x <= 0,
2^32 - 1 for x >= 1, floor(x * 2^32) otherwise, so every sum is an exact
integer: P = fx(target row of u), Q = fx(draft row q_row[u]), S_P = sum P,
S_Q = sum Q. The residual after j rejections is N_j / W_j with
N_j[v] = max(0, P[v] * S_Q - G_j * Q[v]), W_j = sum N_j, G_0 = 0,
G_{j+1} = G_j + floor(W_j / S_Q); G_0 = 0 reproduces p itself and the update is
norm(max(0, residual - q)) up to the floor, which moves G by less than one unit
in S_P. Children are tested in index order against the current residual:
child c with token t is accepted iff N_j[t] > 0 and m_c * Q[t] * W_j <=
2^24 * N_j[t] * S_Q, i.e. r <= min(1, residual(t) / q(t)) with r = m_c / 2^24.
If no child is accepted the bonus is the smallest v with
2^32 * sum_{w <= v} N[w] > K_u * W (inverse CDF at u = K_u / 2^32); W = 0
gives the smallest-index argmax of P. A node without children (or whose q row
is missing / sums to zero) resamples from P.

Probabilities from logits (tree_verify_logits): the target distribution the
rule consumes is the target model's (n1n.ai, "Mathematical Proof of Lossless
Speedup"), at the request's temperature (SGLang "Speculative Decoding": a
sampling parameter). Reading: p = softmax(l / T) per row, evaluated here in
fp64 and stored fp32 like supplied probabilities; a logit whose fp32 quotient
l / T is not finite gets a NaN probability and stays out of the normalisation;
a temperature that is not a finite positive number makes every probability of
the sequence NaN. Greedy sequences use the logits themselves.

Status bits (per sequence): INVALID_PARENT - a parent outside [0, i) (the node
is then a child of the root); INVALID_TOKEN - a draft token outside [0, V)
(never accepted, never tested); NAN_INPUT - a NaN in any target row of the tree
or in the q row of a sampling node that has children; ZERO_Q and
ZERO_RESIDUAL - raised at a node on the walked path.
"""
from __future__ import annotations

import numpy as np

from .philox import node_uniforms
from .tree import STATUS_INVALID_PARENT

STATUS_INVALID_TOKEN = 2
STATUS_NAN_INPUT = 4
STATUS_ZERO_Q = 8
STATUS_ZERO_RESIDUAL = 16

MODE_GREEDY = 0
MODE_SAMPLE = 1

TWO24 = 1 << 24
TWO32 = 1 << 32


def fx_row(row) -> np.ndarray:
    """2^-32 fixed point of an fp32 probability row (uint64 values < 2^32)."""
    r = np.asarray(row, dtype=np.float32).astype(np.float64)
    out = np.zeros(r.shape, dtype=np.uint64)
    inside = (r > 0.0) & (r < 1.0)  # NaN fails both tests
    out[inside] = np.floor(r[inside] * 4294967296.0).astype(np.uint64)
    out[r >= 1.0] = np.uint64(TWO32 - 1)
    return out


def argmax_nan_low(row) -> int:
    """Smallest index of the maximum, NaN counted as -inf."""
    r = np.asarray(row, dtype=np.float32).astype(np.float64)
    r = np.where(np.isnan(r), -np.inf, r)
    return int(np.flatnonzero(r == r.max())[0])


def effective_parents(parents, T):
    p = np.zeros(T, dtype=np.int64)
    p[0] = -1
    status = 0
    for i in range(1, T):
        pi = int(parents[i])
        if 0 <= pi < i:
            p[i] = pi
        else:
            p[i] = 0
            status |= STATUS_INVALID_PARENT
    return p, status


def sample_node_outcome(P, S_P, Q, S_Q, kid_tokens, kid_m, K, V):
    """Outcome of rejection sampling at one node.

    P, Q: uint64 fixed-point rows (Q may be None); kid_tokens / kid_m: the
    children's tokens and acceptance integers m in test order.
    Returns (index into kid list or -1, bonus token or -1, flags).
    """
    flags = 0
    tested = False
    if kid_tokens and (Q is None or S_Q == 0):
        flags |= STATUS_ZERO_Q
        kid_tokens = []
    if kid_tokens:
        Po = P.astype(object)
        Qo = Q.astype(object)
        gamma = 0
        N = Po * S_Q
        W = S_P * S_Q
        for idx, (t, m) in enumerate(zip(kid_tokens, kid_m)):
            if not (0 <= t < V):
                continue
            tested = True
            N_t = int(N[t])
            if N_t > 0 and m * int(Q[t]) * W <= TWO24 * N_t * S_Q:
                return idx, -1, flags
            gamma = gamma + W // S_Q
            N = np.maximum(Po * S_Q - gamma * Qo, 0)
            W = int(N.sum())
            if W == 0:
                flags |= STATUS_ZERO_RESIDUAL
    if not tested:
        N = P.astype(object)
        W = S_P
    if W == 0:
        return -1, int(np.argmax(P)), flags
    cdf = np.cumsum(N)
    hit = np.flatnonzero((cdf * TWO32) > K * W)
    return -1, int(hit[0]), flags


def verify_sequence(target_rows, draft_rows, q_row, tokens, parents, T, mode, key, offset, b):
    """Verify one sequence's tree.

    target_rows: [>=T, V] fp32 (logits for greedy, probabilities for sampling);
    draft_rows: [R, V] fp32 probabilities or None; q_row, tokens, parents: [>=T].
    Returns (accept_len, accept_nodes (root first), out_tokens (drafts then bonus), status).
    """
    V = target_rows.shape[-1]
    peff, status = effective_parents(parents, T)
    tok_ok = [True] + [0 <= int(tokens[i]) < V for i in range(1, T)]
    if not all(tok_ok):
        status |= STATUS_INVALID_TOKEN
    children = [[] for _ in range(T)]
    for i in range(1, T):
        children[peff[i]].append(i)
    if np.isnan(np.asarray(target_rows[:T], dtype=np.float32)).any():
        status |= STATUS_NAN_INPUT

    if mode == MODE_GREEDY:
        a = [argmax_nan_low(target_rows[u]) for u in range(T)]
        ok = [True] * T
        depth = [0] * T
        for i in range(1, T):
            p = peff[i]
            depth[i] = depth[p] + 1
            ok[i] = ok[p] and tok_ok[i] and int(tokens[i]) == a[p]
        e = max((i for i in range(T) if ok[i]), key=lambda i: (depth[i], -i))
        path = [e]
        while path[-1] != 0:
            path.append(int(peff[path[-1]]))
        path.reverse()
        out = [int(tokens[n]) for n in path[1:]] + [a[e]]
        return len(path) - 1, path, out, status

    # sampling
    R = 0 if draft_rows is None else draft_rows.shape[0]
    for u in range(T):
        qr = int(q_row[u]) if q_row is not None else -1
        if children[u] and 0 <= qr < R and np.isnan(np.asarray(draft_rows[qr], dtype=np.float32)).any():
            status |= STATUS_NAN_INPUT
    u = 0
    path = [0]
    while True:
        P = fx_row(target_rows[u])
        S_P = int(P.sum())
        kids = children[u]
        qr = int(q_row[u]) if q_row is not None else -1
        Q = None
        S_Q = 0
        if kids and 0 <= qr < R:
            Q = fx_row(draft_rows[qr])
            S_Q = int(Q.sum())
        kid_tokens = [int(tokens[c]) for c in kids]
        kid_m = [node_uniforms(key, offset, b, c)[0] for c in kids]
        _, K = node_uniforms(key, offset, b, u)
        idx, bonus, flags = sample_node_outcome(P, S_P, Q, S_Q, kid_tokens, kid_m, K, V)
        status |= flags
        if idx >= 0:
            u = kids[idx]
            path.append(u)
            continue
        out = [int(tokens[n]) for n in path[1:]] + [bonus]
        return len(path) - 1, path, out, status


def target_probs_from_logits(logits_row, temperature) -> np.ndarray:
    """softmax(logits / temperature) of one row, fp64 arithmetic, stored fp32 (readings in the header)."""
    l32 = np.asarray(logits_row, dtype=np.float32)
    T = np.float32(temperature)
    out = np.full(l32.shape, np.nan, dtype=np.float64)
    if not (np.isfinite(T) and T > 0):
        return out.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        finite = np.isfinite(l32 / T)  # the fp32 quotient decides which logits take part
    x = l32.astype(np.float64) / float(T)
    if finite.any():
        m = x[finite].max()
        e = np.exp(x[finite] - m)
        out[finite] = e / e.sum()
    return out.astype(np.float32)


def tree_verify_logits(logits, temperature, draft_probs, q_row, tokens, parents, T_b, modes, key, offset, seqs=None):
    """tree_verify with each sampling sequence's target rows formed from its logits and temperature."""
    target = np.array(logits, dtype=np.float32, copy=True)
    for b in range(target.shape[0]):
        if int(modes[b]) == MODE_SAMPLE:
            t_b = 1.0 if temperature is None else float(temperature[b])
            for u in range(target.shape[1]):
                target[b, u] = target_probs_from_logits(logits[b, u], t_b)
    return tree_verify(target, draft_probs, q_row, tokens, parents, T_b, modes, key, offset, seqs)


def tree_verify(target, draft_probs, q_row, tokens, parents, T_b, modes, key, offset, seqs=None):
    """Batch wrapper: returns lists (accept_len, accept_nodes, out_tokens, status) per sequence."""
    B = target.shape[0]
    res = []
    for b in (range(B) if seqs is None else seqs):
        dr = None if draft_probs is None else draft_probs[b]
        qr = None if q_row is None else q_row[b]
        res.append(verify_sequence(target[b], dr, qr, tokens[b], parents[b], int(T_b[b]),
                                   int(modes[b]), key, offset, b))
    return res
