"""Pins of oracle.attend_multi (several causal query tokens per sequence)."""
import math

import numpy as np
import pytest

import oracle
from brute import attend_brute


def case(rng, B, S_q, h_q, h_kv, d, lens, sigma=1.5):
    T = int(sum(lens))
    q = rng.standard_normal((B, S_q, h_q, d))
    k = sigma * rng.standard_normal((T, h_kv, d))
    v = rng.standard_normal((T, h_kv, d))
    return q, k, v, np.asarray(lens, dtype=np.int32)


def test_single_query_token_is_attend():
    rng = np.random.default_rng(1)
    q, k, v, sl = case(rng, 3, 1, 8, 2, 16, [40, 1, 77])
    a = oracle.attend_multi(q, k, v, sl, np.float32(0.25), 2, dtype="f64")
    b = oracle.attend(q[:, 0], k, v, sl, np.float32(0.25), 2, dtype="f64")
    np.testing.assert_array_equal(a[:, 0], b)


@pytest.mark.parametrize("S_q", [2, 3, 5])
def test_each_token_is_brute_force_on_its_prefix(S_q):
    """Token i of sequence b equals single-token brute force over the first
    S_b - S_q + i + 1 cached rows (independent loop code)."""
    rng = np.random.default_rng(10 + S_q)
    lens = [9, 4, 12]
    B, h_q, h_kv, d = 3, 4, 2, 3
    q, k, v, sl = case(rng, B, S_q, h_q, h_kv, d, lens)
    scale = np.float32(1 / math.sqrt(d))
    got = oracle.attend_multi(q, k, v, sl, scale, h_kv, dtype="f64")
    start = 0
    for b, S in enumerate(lens):
        for i in range(S_q):
            p = S - S_q + i
            if p < 0:
                np.testing.assert_array_equal(got[b, i], 0.0)
                continue
            ref = attend_brute([q[b, i].tolist()], k[start:start + p + 1].tolist(),
                               v[start:start + p + 1].tolist(), [p + 1], float(scale), h_kv)
            np.testing.assert_allclose(got[b, i], np.array(ref[0]), rtol=0, atol=1e-13)
        start += S


def test_future_positions_do_not_matter():
    """Changing K/V after a token's position leaves that token's output alone."""
    rng = np.random.default_rng(3)
    S_q, S = 4, 30
    q, k, v, sl = case(rng, 1, S_q, 8, 4, 8, [S])
    a = oracle.attend_multi(q, k, v, sl, np.float32(0.3), 4, dtype="f64")
    k2, v2 = k.copy(), v.copy()
    k2[S - 2:] += 5.0
    v2[S - 2:] -= 7.0
    b = oracle.attend_multi(q, k2, v2, sl, np.float32(0.3), 4, dtype="f64")
    np.testing.assert_array_equal(a[0, :2], b[0, :2])      # positions S-4, S-3 see rows < S-2
    assert not np.allclose(a[0, 2:], b[0, 2:])


def test_last_token_sees_everything():
    rng = np.random.default_rng(4)
    q, k, v, sl = case(rng, 2, 3, 8, 2, 16, [25, 7])
    a = oracle.attend_multi(q, k, v, sl, np.float32(0.25), 2, dtype="f64")
    b = oracle.attend(q[:, -1], k, v, sl, np.float32(0.25), 2, dtype="f64")
    np.testing.assert_allclose(a[:, -1], b, rtol=0, atol=1e-15)


def test_more_query_tokens_than_cached_positions():
    rng = np.random.default_rng(5)
    q, k, v, sl = case(rng, 1, 4, 2, 1, 4, [2])
    a = oracle.attend_multi(q, k, v, sl, np.float32(0.5), 1, dtype="f64")
    np.testing.assert_array_equal(a[0, :2], 0.0)             # positions -2, -1
    np.testing.assert_allclose(a[0, 2], np.broadcast_to(v[0, 0], (2, 4)), rtol=0, atol=1e-15)
