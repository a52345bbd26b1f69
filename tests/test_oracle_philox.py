"""Pins for the oracle's Philox4x64-10 against numpy's independent implementation.

numpy.random.Philox is Philox4x64-10; it advances its 256-bit counter before
producing a block, so its first block at counter c is the textbook block at
counter c + 1 (carry into the next word on wrap).
"""
import numpy as np
import pytest

from oracle.philox import MASK64, node_uniforms, philox4x64_10


def _inc(ctr):
    c = list(ctr)
    for i in range(4):
        c[i] = (c[i] + 1) & MASK64
        if c[i] != 0:
            break
    return tuple(c)


@pytest.mark.parametrize("seed", range(12))
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    key = tuple(int(x) for x in rng.integers(0, 2**63, size=2, dtype=np.uint64))
    ctr = tuple(int(x) for x in rng.integers(0, 2**63, size=4, dtype=np.uint64))
    if seed == 0:
        ctr = (MASK64, 5, 0, 0)  # exercises the carry of numpy's pre-increment
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = [int(x) for x in g.random_raw(8)]
    assert list(philox4x64_10(_inc(ctr), key)) == raw[:4]
    assert list(philox4x64_10(_inc(_inc(ctr)), key)) == raw[4:]


def test_node_uniform_ranges_and_independence():
    key = (1003, 0x5EED)
    ms, Ks = [], []
    for i in range(2000):
        m, K = node_uniforms(key, 0, i % 7, i)
        assert 1 <= m <= 2**24 and 0 <= K < 2**32
        ms.append(m)
        Ks.append(K)
    # uniform means within 5 sigma
    ms = np.array(ms, dtype=np.float64) / 2**24
    Ks = np.array(Ks, dtype=np.float64) / 2**32
    for x in (ms, Ks):
        assert abs(x.mean() - 0.5) < 5 * np.sqrt(1 / 12 / len(x))
    # different counters give different blocks; the same counter repeats
    assert node_uniforms(key, 0, 0, 1) == node_uniforms(key, 0, 0, 1)
    assert node_uniforms(key, 0, 0, 1) != node_uniforms(key, 1, 0, 1)
    assert node_uniforms(key, 0, 0, 1) != node_uniforms(key, 0, 1, 1)


def test_node_uniforms_use_counter_offset_b_i_and_words_0_1():
    # the stream layout, checked against numpy's generator: counter (offset, b, i, 0),
    # m = top 24 bits of word 0 plus one (r = m / 2^24 in (0, 1]), K = top 32 bits of word 1
    key = (77, 0x5EED)
    for offset, b, i in [(0, 0, 0), (3, 1, 5), (2**40, 31, 64)]:
        # numpy pre-increments, so start it one below the counter we want
        g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=_dec((offset, b, i, 0)))
        w = [int(x) for x in g.random_raw(4)]
        assert node_uniforms(key, offset, b, i) == ((w[0] >> 40) + 1, w[1] >> 32)


def _dec(ctr):
    c = list(ctr)
    for k in range(4):
        borrow = c[k] == 0
        c[k] = (c[k] - 1) & MASK64
        if not borrow:
            break
    return np.array(c, dtype=np.uint64)
