"""Pins of oracle.kv_append: hand-placed rows, capacity clamping, and the
decode-step identity append(prefix) + attend == attend(full sequence)."""
import numpy as np

import oracle


def test_rows_land_where_expected():
    cap, h_kv, d = 5, 1, 2
    kc = np.zeros((3 * cap, h_kv, d))
    vc = np.zeros((3 * cap, h_kv, d))
    k_new = np.arange(3 * 2 * h_kv * d, dtype=float).reshape(3, 2, h_kv, d) + 1
    v_new = -k_new
    lens = np.array([0, 2, 4])
    k2, v2, nl = oracle.kv_append(kc, vc, k_new, v_new, lens, cap)
    np.testing.assert_array_equal(nl, [2, 4, 5])
    np.testing.assert_array_equal(k2[0], k_new[0, 0]); np.testing.assert_array_equal(k2[1], k_new[0, 1])
    np.testing.assert_array_equal(k2[cap + 2], k_new[1, 0]); np.testing.assert_array_equal(k2[cap + 3], k_new[1, 1])
    np.testing.assert_array_equal(k2[2 * cap + 4], k_new[2, 0])          # second row does not fit
    np.testing.assert_array_equal(v2[2 * cap + 4], v_new[2, 0])
    written = {0, 1, cap + 2, cap + 3, 2 * cap + 4}
    for r in range(3 * cap):
        if r not in written:
            assert not k2[r].any() and not v2[r].any()
    assert not kc.any()                                                  # input left alone


def test_explicit_offsets():
    kc = np.zeros((10, 1, 1)); vc = np.zeros((10, 1, 1))
    k_new = np.array([[[[7.0]]], [[[9.0]]]]); v_new = k_new + 1
    k2, v2, nl = oracle.kv_append(kc, vc, k_new, v_new, np.array([1, 0]), 4, kv_offsets=np.array([6, 0]))
    assert k2[7, 0, 0] == 7.0 and k2[0, 0, 0] == 9.0 and v2[7, 0, 0] == 8.0
    np.testing.assert_array_equal(nl, [2, 1])


def test_append_then_attend_equals_attend_on_full_cache():
    rng = np.random.default_rng(0)
    B, cap, h_kv, h_q, d = 3, 40, 2, 8, 16
    full = [33, 7, 20]
    kf = rng.standard_normal((B * cap, h_kv, d)); vf = rng.standard_normal((B * cap, h_kv, d))
    q = rng.standard_normal((B, h_q, d))
    prefix = np.array(full) - 1
    kc = kf.copy(); vc = vf.copy()
    k_new = np.stack([kf[b * cap + prefix[b]] for b in range(B)])[:, None]
    v_new = np.stack([vf[b * cap + prefix[b]] for b in range(B)])[:, None]
    for b in range(B):                                  # garbage where the new rows go
        kc[b * cap + prefix[b]] = 99.0; vc[b * cap + prefix[b]] = -99.0
    k2, v2, nl = oracle.kv_append(kc, vc, k_new, v_new, prefix, cap)
    np.testing.assert_array_equal(nl, full)
    for b in range(B):
        rows = slice(b * cap, b * cap + full[b])
        got = oracle.attend(q[b:b + 1], k2[rows], v2[rows], np.array([full[b]]), np.float32(0.25), h_kv, dtype="f64")
        ref = oracle.attend(q[b:b + 1], kf[rows], vf[rows], np.array([full[b]]), np.float32(0.25), h_kv, dtype="f64")
        np.testing.assert_array_equal(got, ref)
