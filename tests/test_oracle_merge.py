"""Pins of the oracle's triplet, merge and fan-out functions.

The kernbench2 `_attention_mesh_mlo.py` page states that merging every
shard's (m, l, o) exactly once, in any order the fan-out produces, leaves
every rank with the same final answer, and that the triplet of rank i
reaches rank j at step |i - j|. These tests check exactly those statements
against the unsplit result. CPU only.
"""
import itertools

import numpy as np
import pytest

import oracle


def unsplit(s, vr):
    """Reference: softmax(s) @ V written directly, no triplets."""
    e = np.exp(s - s.max())
    return (e / e.sum()) @ vr


def chunks_of(n, cuts):
    bounds = [0] + sorted(cuts) + [n]
    return [(bounds[i], bounds[i + 1]) for i in range(len(bounds) - 1)]


def merge_all(trips):
    acc = (oracle.NEG_INF, 0.0, np.zeros_like(trips[0][2]))
    for t in trips:
        acc = oracle.merge(acc, t)
    return acc


@pytest.mark.parametrize("S", [1, 2, 17, 1000, 65536])
def test_whole_triplet_equals_unsplit(S):
    rng = np.random.default_rng(S)
    s = rng.standard_normal(S) * 3
    vr = rng.standard_normal((S, 16))
    np.testing.assert_allclose(oracle.finalize(oracle.triplet(s, vr)), unsplit(s, vr), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,n_cuts,seed", [(10, 3, 0), (257, 8, 1), (4096, 31, 2), (65536, 63, 3)])
def test_random_chunkings_with_empty_chunks(S, n_cuts, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(S) * 4
    vr = rng.standard_normal((S, 8))
    cuts = list(rng.integers(0, S + 1, size=n_cuts))
    cuts += [cuts[0], 0, S]             # duplicates make empty chunks
    trips = [oracle.triplet(s[a:b], vr[a:b]) for a, b in chunks_of(S, cuts)]
    assert any(t[1] == 0.0 for t in trips)
    ref = unsplit(s, vr)
    np.testing.assert_allclose(oracle.finalize(merge_all(trips)), ref, rtol=0, atol=1e-12)
    rng.shuffle(trips)
    np.testing.assert_allclose(oracle.finalize(merge_all(trips)), ref, rtol=0, atol=1e-12)


def test_size_one_chunks_every_order():
    rng = np.random.default_rng(4)
    s = rng.standard_normal(5) * 10
    vr = rng.standard_normal((5, 4))
    trips = [oracle.triplet(s[i:i + 1], vr[i:i + 1]) for i in range(5)]
    ref = unsplit(s, vr)
    for perm in itertools.permutations(range(5)):
        got = oracle.finalize(merge_all([trips[i] for i in perm]))
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_tree_merge_equals_sequential():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(64) * 2
    vr = rng.standard_normal((64, 4))
    trips = [oracle.triplet(s[i:i + 8], vr[i:i + 8]) for i in range(0, 64, 8)]
    while len(trips) > 1:
        trips = [oracle.merge(trips[i], trips[i + 1]) for i in range(0, len(trips), 2)]
    np.testing.assert_allclose(oracle.finalize(trips[0]), unsplit(s, vr), rtol=0, atol=1e-12)


def test_merge_formula_on_hand_values():
    """(m, l, o) = (0, 1, [1]) and (ln 3, 1, [5]): m_c = ln 3, factors 1/3 and 1,
    l = 4/3, o = 1/3 + 5 = 16/3, o / l = 4."""
    a = (0.0, 1.0, np.array([1.0]))
    b = (np.log(3.0), 1.0, np.array([5.0]))
    m, l, o = oracle.merge(a, b)
    assert m == np.log(3.0)
    np.testing.assert_allclose([l, o[0]], [4.0 / 3.0, 16.0 / 3.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.finalize((m, l, o)), [4.0], rtol=0, atol=1e-15)


def test_empty_triplets():
    e = oracle.triplet(np.zeros(0), np.zeros((0, 3)))
    assert e[0] == oracle.NEG_INF and e[1] == 0.0 and not e[2].any()
    t = (1.5, 2.0, np.array([1.0, 2.0, 3.0]))
    for got in (oracle.merge(e, t), oracle.merge(t, e)):
        assert got[0] == 1.5 and got[1] == 2.0
        np.testing.assert_array_equal(got[2], t[2])
    both = oracle.merge(e, e)
    assert both[1] == 0.0
    np.testing.assert_array_equal(oracle.finalize(both), np.zeros(3))


def test_merge_survives_far_apart_maxima():
    """A chunk 2000 score units below the other must vanish without NaN."""
    a = oracle.triplet(np.array([0.0, 1.0]), np.array([[1.0], [2.0]]))
    b = oracle.triplet(np.array([2000.0]), np.array([[7.0]]))
    np.testing.assert_allclose(oracle.finalize(oracle.merge(a, b)), [7.0], rtol=0, atol=0)
    np.testing.assert_allclose(oracle.finalize(oracle.merge(b, a)), [7.0], rtol=0, atol=0)


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_fanout_every_rank_gets_the_unsplit_answer(n):
    rng = np.random.default_rng(100 + n)
    S = 40 * n
    s = rng.standard_normal(S) * 3
    vr = rng.standard_normal((S, 6))
    per = S // n
    trips = [oracle.triplet(s[i * per:(i + 1) * per], vr[i * per:(i + 1) * per]) for i in range(n)]
    outs, order = oracle.fanout(trips)
    ref = unsplit(s, vr)
    for i in range(n):
        np.testing.assert_allclose(outs[i], ref, rtol=0, atol=1e-12)
        assert sorted(order[i]) == list(range(n))        # every origin exactly once


@pytest.mark.parametrize("n", [2, 4, 7])
def test_fanout_arrival_step_is_rank_distance(n):
    """The page: the triplet from rank i reaches rank j at step |i - j|;
    within a step the west arrival (rank j - step) is merged before the east
    one (rank j + step)."""
    trips = [oracle.triplet(np.array([float(i)]), np.array([[float(i)]])) for i in range(n)]
    _, order = oracle.fanout(trips)
    for j in range(n):
        want = [j]
        for step in range(1, n):
            if j - step >= 0:
                want.append(j - step)
            if j + step < n:
                want.append(j + step)
        assert order[j] == want


def test_triplet_matches_definition():
    rng = np.random.default_rng(6)
    s = rng.standard_normal(50)
    vr = rng.standard_normal((50, 3))
    m, l, o = oracle.triplet(s, vr)
    assert m == s.max()
    np.testing.assert_allclose(l, sum(np.exp(x - m) for x in s), rtol=1e-14)
    np.testing.assert_allclose(o, sum(np.exp(s[t] - m) * vr[t] for t in range(50)), rtol=0, atol=1e-12)
