"""Pins for the oracle's tree verification.

* greedy: brute-force enumeration of every root->node path on tiny trees with
  many ties, and the worked topology of the n1n.ai page
  (tests/golden/verify_p3_topology.json);
* fixed point: exact values of fx on hand-chosen inputs;
* sampling, closed forms: with p = (1/2, 1/4, 1/4, 0), q = (1/4, 1/2, 1/4, 0) a
  draft of token 1 is accepted iff r <= 1/2, the residual max(0, p - q) puts all
  mass on token 0, and so on;
* sampling, distribution: with children drawn i.i.d. from q the emitted token
  follows p (chi-square, 16-token vocabulary), a single draft is accepted with
  probability sum_v min(p_v, q_v) (tanhdev page, section 5 "Speculative
  Rejection Sampling: Mathematical Invariance"), and the second token of an
  accepted chain follows the child's target row.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle.philox import node_uniforms
from oracle.verify import (
    MODE_GREEDY,
    MODE_SAMPLE,
    STATUS_INVALID_TOKEN,
    STATUS_NAN_INPUT,
    STATUS_ZERO_Q,
    STATUS_ZERO_RESIDUAL,
    fx_row,
    sample_node_outcome,
    verify_sequence,
)
from oracle.tree import STATUS_INVALID_PARENT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEY = (1003, 0x5EED)


def test_fixed_point_values():
    x = np.array([0.5, 1.0, 2.0, np.nan, -0.25, 0.0, -0.0, 2.0**-32, 2.0**-33, 3 * 2.0**-32,
                  np.nextafter(np.float32(1), np.float32(0)), np.inf, -np.inf,
                  1.5 * 2.0**-32, 2.75 * 2.0**-32, 0.999 * 2.0**-32], dtype=np.float32)
    # floor, not round: 1.5 -> 1, 2.75 -> 2, 0.999 -> 0
    want = [2**31, 2**32 - 1, 2**32 - 1, 0, 0, 0, 0, 1, 0, 3, 2**32 - 2**8, 2**32 - 1, 0, 1, 2, 0]
    assert [int(v) for v in fx_row(x)] == want


# ---------------------------------------------------------------- greedy
def _brute_force_greedy(target, tokens, parents, T):
    def amax(row):
        best = max(row)
        return min(v for v in range(len(row)) if row[v] == best)

    a = [amax(list(target[u])) for u in range(T)]
    best = None
    for e in range(T):
        path = [e]
        while path[-1] != 0:
            path.append(int(parents[path[-1]]))
        path.reverse()
        if all(int(tokens[path[k]]) == a[path[k - 1]] for k in range(1, len(path))):
            key = (len(path), -e)
            if best is None or key > best[0]:
                best = (key, path)
    path = best[1]
    return len(path) - 1, path, [int(tokens[n]) for n in path[1:]] + [a[path[-1]]]


@pytest.mark.parametrize("seed", range(200))
def test_greedy_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 9))
    V = int(rng.integers(2, 7))
    parents = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)])
    tokens = rng.integers(0, V, size=T)
    target = rng.integers(-2, 3, size=(T, V)).astype(np.float32)  # many ties
    got = verify_sequence(target, None, None, tokens, parents, T, MODE_GREEDY, KEY, 0, 0)
    want = _brute_force_greedy(target, tokens, parents, T)
    assert got[:3] == (want[0], want[1], want[2])
    assert got[3] == 0


def test_greedy_worked_topology():
    with open(os.path.join(GOLDEN, "verify_p3_topology.json")) as f:
        g = json.load(f)
    T, V = len(g["parents"]), g["V"]
    target = np.zeros((T, V), dtype=np.float32)
    for u, t in enumerate(g["argmax_per_row"]):
        target[u, t] = 1.0
    got = verify_sequence(target, None, None, g["tokens"], g["parents"], T, MODE_GREEDY, KEY, 0, 0)
    e = g["expect"]
    assert got == (e["accept_len"], e["accept_nodes"], e["out_tokens"], e["status"])


def test_greedy_nan_is_minus_infinity_and_status_bits():
    V = 5
    target = np.array([[np.nan, -np.inf, 1.0, 1.0, np.nan], [0, 0, 0, 0, 0], [np.nan] * 5], dtype=np.float32)
    # node 1 (token 2) matches argmax(row 0) = 2 (tie with 3 -> smallest index)
    got = verify_sequence(target, None, None, [0, 2, 9], [-1, 0, 7], 3, MODE_GREEDY, KEY, 0, 0)
    acc_len, nodes, out, status = got
    assert (acc_len, nodes) == (1, [0, 1])
    assert out == [2, 0]  # argmax of an all-zero row is index 0
    assert status == STATUS_NAN_INPUT | STATUS_INVALID_TOKEN | STATUS_INVALID_PARENT


# ---------------------------------------------------------------- sampling, closed forms
P4 = np.array([0.5, 0.25, 0.25, 0.0], dtype=np.float32)
Q4 = np.array([0.25, 0.5, 0.25, 0.0], dtype=np.float32)


def _sample(p_rows, q_rows, q_row, tokens, parents, offset=0, b=0):
    T = len(tokens)
    return verify_sequence(np.asarray(p_rows, np.float32), np.asarray(q_rows, np.float32), q_row, tokens,
                           parents, T, MODE_SAMPLE, KEY, offset, b)


def test_single_draft_accept_iff_r_below_ratio():
    seen = set()
    for off in range(300):
        m, _ = node_uniforms(KEY, off, 0, 1)
        acc_len, nodes, out, st = _sample([P4, P4], [Q4], [0, -1], [0, 1], [-1, 0], offset=off)
        accept = m <= 2**23  # r = m / 2^24 <= p(1)/q(1) = 1/2
        assert (acc_len == 1) == accept
        if not accept:
            assert out == [0]  # max(0, p - q) = (1/4, 0, 0, 0)
        seen.add(accept)
        assert st == 0
    assert seen == {True, False}


def test_second_draft_tested_against_residual():
    # after token 1 is rejected the residual is all on token 0, q(0) = 1/4 -> accept surely
    for off in range(200):
        m, _ = node_uniforms(KEY, off, 0, 1)
        acc_len, nodes, out, st = _sample([P4] * 3, [Q4], [0, -1, -1], [0, 1, 0], [-1, 0, 0], offset=off)
        if m <= 2**23:
            assert nodes == [0, 1]
        else:
            assert nodes == [0, 2] and out[0] == 0


def test_zero_probability_draft_always_rejected():
    for off in range(50):
        acc_len, nodes, out, st = _sample([P4, P4], [Q4], [0, -1], [0, 3], [-1, 0], offset=off)
        assert acc_len == 0 and out == [0]


def test_zero_residual_and_zero_q_fallbacks():
    p = np.array([0.5, 0.5, 0.0, 0.0], dtype=np.float32)
    # q == p: drafting token 2 (p = 0) is rejected and leaves max(0, p - q) = 0
    acc_len, nodes, out, st = _sample([p, p], [p], [0, -1], [0, 2], [-1, 0])
    assert acc_len == 0 and out == [0] and st == STATUS_ZERO_RESIDUAL
    # an all-zero q row: no draft is tested, the bonus is drawn from p
    z = np.zeros(4, dtype=np.float32)
    for off in range(20):
        _, K = node_uniforms(KEY, off, 0, 0)
        acc_len, nodes, out, st = _sample([p, p], [z], [0, -1], [0, 0], [-1, 0], offset=off)
        assert acc_len == 0 and st == STATUS_ZERO_Q
        assert out == [0 if K < 2**31 else 1]
    # a missing q row on a node with children behaves the same
    acc_len, nodes, out, st = _sample([p, p], [z], [-1, -1], [0, 0], [-1, 0])
    assert st == STATUS_ZERO_Q


def test_leaf_resample_is_inverse_cdf():
    p = np.array([0.125, 0.375, 0.25, 0.25], dtype=np.float32)
    for off in range(100):
        _, K = node_uniforms(KEY, off, 0, 0)
        u = K / 2**32
        want = int(np.searchsorted(np.cumsum([0.125, 0.375, 0.25, 0.25]), u, side="right"))
        acc_len, nodes, out, st = _sample([p], [p], [-1], [0], [-1], offset=off)
        assert out == [want]


def test_inverse_cdf_boundary_is_strict():
    # P = (1/2, 1/2): u = K / 2^32 = 1/2 exactly lands on the boundary between tokens 0 and 1;
    # the inverse CDF picks the smallest v with CDF(v) > u, so K = 2^31 gives token 1
    P = fx_row(np.array([0.5, 0.5], dtype=np.float32))
    S_P = int(P.sum())
    for K, want in [(2**31 - 1, 0), (2**31, 1), (0, 0), (2**32 - 1, 1)]:
        assert sample_node_outcome(P, S_P, None, 0, [], [], K, 2) == (-1, want, 0)


def test_nan_in_q_row_flags():
    q = np.array([np.nan, 0.5, 0.5, 0.0], dtype=np.float32)
    *_, st = _sample([P4, P4], [q], [0, -1], [0, 1], [-1, 0])
    assert st & STATUS_NAN_INPUT


# ---------------------------------------------------------------- sampling, distributions
def _fixed(rng, V):
    p = rng.dirichlet(np.ones(V)).astype(np.float32)
    q = rng.dirichlet(np.ones(V)).astype(np.float32)
    P, Q = fx_row(p).astype(np.float64), fx_row(q).astype(np.float64)
    return p, q, P / P.sum(), Q / Q.sum()


@pytest.mark.parametrize("m", [1, 2, 3])
def test_emitted_token_follows_target(m):
    V, trials = 16, 30000
    rng = np.random.default_rng(40 + m)
    p, q, pn, qn = _fixed(rng, V)
    counts = np.zeros(V)
    accepts = 0
    parents = [-1] + [0] * m
    for t in range(trials):
        toks = [0] + list(rng.choice(V, size=m, p=qn))
        acc_len, nodes, out, _ = _sample([p] * (m + 1), [q], [0] + [-1] * m, toks, parents, offset=t)
        counts[out[0]] += 1
        accepts += acc_len
    chi2 = ((counts - trials * pn) ** 2 / (trials * pn)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-3, (chi2, counts)
    if m == 1:
        alpha = np.minimum(pn, qn).sum()
        z = (accepts - trials * alpha) / np.sqrt(trials * alpha * (1 - alpha))
        assert abs(z) < 4.5


def test_second_token_of_accepted_chain_follows_child_row():
    V, trials = 16, 30000
    rng = np.random.default_rng(77)
    p0, q0, p0n, q0n = _fixed(rng, V)
    # make the first draft likely to be accepted so the second level is exercised often
    q0 = p0.copy()
    q0n = fx_row(q0).astype(np.float64)
    q0n /= q0n.sum()
    p1, q1, p1n, q1n = _fixed(rng, V)
    counts = np.zeros(V)
    reached = 0
    for t in range(trials):
        toks = [0, int(rng.choice(V, p=q0n)), 0]
        toks[2] = int(rng.choice(V, p=q1n))
        acc_len, nodes, out, _ = _sample([p0, p1, p1], [q0, q1], [0, 1, -1], toks, [-1, 0, 1], offset=t)
        if acc_len >= 1:
            reached += 1
            counts[out[1]] += 1
    assert reached > trials * 0.9
    chi2 = ((counts - reached * p1n) ** 2 / (reached * p1n)).sum()
    assert stats.chi2.sf(chi2, V - 1) > 1e-3


# ---------------------------------------------------------------- probabilities from logits
def test_probs_from_logits_match_scipy_softmax():
    from scipy.special import softmax

    from oracle.verify import target_probs_from_logits

    rng = np.random.default_rng(11)
    for T in (1.0, 0.7, 2.5):
        l = (rng.standard_normal(1000) * 3.0).astype(np.float32)
        p = target_probs_from_logits(l, np.float32(T))
        ref = softmax(l.astype(np.float64) / float(np.float32(T)))
        assert p.dtype == np.float32
        np.testing.assert_allclose(p, ref, rtol=2e-7, atol=0)
        assert abs(float(p.astype(np.float64).sum()) - 1.0) < 1e-5


def test_probs_from_logits_shift_and_temperature():
    from oracle.verify import target_probs_from_logits

    rng = np.random.default_rng(12)
    l = (rng.standard_normal(777) * 3.0).astype(np.float32)
    base = target_probs_from_logits(l, 1.0)
    np.testing.assert_allclose(target_probs_from_logits(l + np.float32(40.0), 1.0), base, rtol=1e-5)
    # T = 1/2 on l is T = 1 on 2 l (both quotients exact in fp32)
    np.testing.assert_array_equal(target_probs_from_logits(l, 0.5), target_probs_from_logits(2 * l, 1.0))
    # a small temperature concentrates the mass on the argmax
    sharp = target_probs_from_logits(l, 0.01)
    assert int(np.argmax(sharp)) == int(np.argmax(l)) and sharp.max() > 0.99


def test_probs_from_logits_non_finite():
    from oracle.verify import target_probs_from_logits

    l = np.arange(10, dtype=np.float32)
    l[3], l[7] = np.nan, np.inf
    p = target_probs_from_logits(l, 1.0)
    assert np.isnan(p[3]) and np.isnan(p[7])
    keep = np.array([i for i in range(10) if i not in (3, 7)])
    e = np.exp(l[keep].astype(np.float64) - l[keep].max())
    np.testing.assert_allclose(p[keep], (e / e.sum()).astype(np.float32), rtol=1e-7)
    for T in (0.0, -1.0, np.nan, np.inf):
        assert np.isnan(target_probs_from_logits(np.ones(5, np.float32), T)).all()


def test_workload_sampling_rows_are_the_softmax_of_their_logits():
    from oracle.verify import target_probs_from_logits
    from workloads import make_workload

    w = make_workload(name="lg", B=4, Hq=2, Hkv=1, d=64, prefix=16, topk=2, depth=2, num_draft=3, V=500,
                      verify="alternate", temperature=0.7, seed=21)
    for b in range(w.B):
        for u in range(w.max_T):
            if int(w.modes[b]) == 1:
                # the generator divides by the temperature as the fp64 value 0.7, the logits path by the fp32
                # temperature array (0.7 rounded, 1.7e-8 relative away): quotients of ~10 move by ~2e-7
                np.testing.assert_allclose(target_probs_from_logits(w.target_logits[b, u], w.temperature[b]),
                                           w.target[b, u], rtol=1e-6)
            else:
                np.testing.assert_array_equal(w.target_logits[b, u], w.target[b, u])


def _dispatch_case(seed=31):
    """Alternate-mode trees (even sequences greedy, odd sampling) at distinct fp32-exact temperatures, with
    acceptance planted on some sampling sequences (their q rows on a path are set to the target's p there) and
    a greedy root row whose top two logits collapse to one value under an fp32 softmax."""
    from scipy.special import softmax

    from oracle.tree import build_tree
    from workloads import make_workload

    w = make_workload(name="disp", B=6, Hq=2, Hkv=1, d=64, prefix=16, topk=3, depth=3, num_draft=8, V=300,
                      verify="alternate", temperature=1.0, seed=seed)
    temps = np.array([0.0, 0.5, 0.0, 2.0, 0.0, 1.0], dtype=np.float32)
    trees = [build_tree(w.draft_logprobs[b], int(w.root_tokens[b]), int(w.topk[b]), int(w.depth[b]),
                        int(w.num_draft[b]), w.max_topk) for b in range(w.B)]
    logits = w.target_logits.copy()
    # greedy sequence 0: logits 0.01 and the fp32 value just below it at tokens 5 and 2; a softmax in fp32
    # rounds both to one probability, so only the logits themselves make token 5 the argmax
    logits[0, 0, :] = -10.0
    logits[0, 0, 5] = np.float32(0.01)
    logits[0, 0, 2] = np.nextafter(np.float32(0.01), np.float32(0))
    draft = w.draft_probs.copy()

    def probs(b, T):
        return softmax(logits[b].astype(np.float64) / float(T), axis=-1).astype(np.float32)

    for b in (1, 5):  # plant along the first-child path: the child's token leads the logits, and the
        t = trees[b]  # node's q row is the target's p there
        u, path = 0, []
        while True:
            kids = [i for i in range(1, len(t.tokens)) if t.parents[i] == u]
            if not kids or t.q_row[u] < 0:
                break
            logits[b, u, t.tokens[kids[0]]] = logits[b, u].max() + np.float32(1.0)
            path.append(u)
            u = kids[0]
        p = probs(b, temps[b])
        for u in path:
            draft[b, t.q_row[u]] = p[u]
    T = len(trees[0].tokens)
    tok = np.stack([t.tokens for t in trees])
    par = np.stack([t.parents for t in trees])
    qr = np.stack([t.q_row for t in trees])
    T_b = np.full(w.B, T, dtype=np.int32)
    return w, logits, temps, draft, qr, tok, par, T_b, probs


def test_verify_from_logits_dispatch():
    """Pins tree_verify_logits: each sampling sequence b verifies against softmax(logits / temperature[b]) formed
    independently here (scipy, fp64, stored fp32), each greedy sequence against its raw logits, and a missing
    temperature array means 1 for every sequence (the tree_verify results on those rows are the reference)."""
    from oracle.verify import tree_verify, tree_verify_logits

    w, logits, temps, draft, qr, tok, par, T_b, probs = _dispatch_case()
    key, off = w.philox_key, w.philox_offset

    def reference(tvals):
        target = logits.copy()
        for b in range(w.B):
            if int(w.modes[b]) == MODE_SAMPLE:
                target[b] = probs(b, tvals[b])
        return tree_verify(target, draft, qr, tok, par, T_b, w.modes, key, off)

    got = tree_verify_logits(logits, temps, draft, qr, tok, par, T_b, w.modes, key, off)
    want = reference(temps)
    assert got == want
    # the case is sensitive: planted sequences accept, the greedy root's bonus is token 5 (the fp32 logit
    # argmax), and the sampling outcomes change when the temperatures are swapped between sequences
    assert got[1][0] > 0 and got[5][0] > 0
    assert got[0][2][-1] == 5 or 5 in got[0][2]
    swapped = temps.copy()
    swapped[[1, 3]] = swapped[[3, 1]]
    assert reference(swapped) != want
    # no temperature array: every sampling sequence at T = 1
    got1 = tree_verify_logits(logits, None, draft, qr, tok, par, T_b, w.modes, key, off)
    assert got1 == reference(np.ones(w.B, dtype=np.float32))
    assert got1 != want
