"""Pins of the fp64 oracle against things other than itself.

Brute force (pure Python, mpmath), hand-derived closed forms, the shapes the
pages print, a library special case (torch's CPU attention on key/value heads
repeated per group) and invariants. CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from brute import attend_brute, attend_mp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B, h_q, h_kv, d, lens, sigma=1.0):
    T = int(sum(lens))
    q = rng.standard_normal((B, h_q, d))
    k = sigma * rng.standard_normal((T, h_kv, d))
    v = rng.standard_normal((T, h_kv, d))
    return q, k, v, np.asarray(lens, dtype=np.int32)


SHAPES = [
    # B, h_q, h_kv, d, lens
    (1, 1, 1, 1, [1]),
    (1, 2, 1, 3, [2]),
    (1, 4, 2, 3, [3]),
    (1, 8, 2, 8, [7]),
    (2, 4, 4, 3, [16, 5]),
    (2, 8, 1, 8, [1, 16]),
    (3, 8, 4, 1, [2, 0, 7]),
]


@pytest.mark.parametrize("B,h_q,h_kv,d,lens", SHAPES)
def test_oracle_matches_brute_force(B, h_q, h_kv, d, lens):
    rng = np.random.default_rng(1234 + B * 7 + h_q + d)
    q, k, v, sl = rand_case(rng, B, h_q, h_kv, d, lens, sigma=2.0)
    scale = np.float32(1.0 / math.sqrt(d))
    ref = np.array(attend_brute(q.tolist(), k.tolist(), v.tolist(), sl, float(scale), h_kv))
    got = oracle.attend(q, k, v, sl, scale, h_kv, dtype="f64")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("B,h_q,h_kv,d,lens", [(1, 4, 2, 3, [5]), (2, 2, 1, 2, [3, 4])])
def test_oracle_matches_mpmath(B, h_q, h_kv, d, lens):
    pytest.importorskip("mpmath")
    rng = np.random.default_rng(99)
    q, k, v, sl = rand_case(rng, B, h_q, h_kv, d, lens, sigma=3.0)
    got = oracle.attend(q, k, v, sl, np.float32(0.7), h_kv, dtype="f64")
    # the oracle widens the fp32 scale; give mpmath the same value
    ref = np.array(attend_mp(q.tolist(), k.tolist(), v.tolist(), sl, float(np.float32(0.7)), h_kv))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_oracle_on_bf16_bits_matches_brute_force():
    """bf16 storage: the oracle must use the exact widened values."""
    w = workloads.custom("pin", B=2, h_q=4, h_kv=2, d=8, seq_lens=[6, 9], seed=7)
    qf = workloads.bf16_bits_to_f32(w.q).astype(np.float64)
    kf = workloads.bf16_bits_to_f32(w.k).astype(np.float64)
    vf = workloads.bf16_bits_to_f32(w.v).astype(np.float64)
    ref = np.array(attend_brute(qf.tolist(), kf.tolist(), vf.tolist(), w.seq_lens,
                                float(w.scale), 2))
    got = oracle.attend(w.q, w.k, w.v, w.seq_lens, w.scale, 2, dtype="bf16")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_widen_bf16_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, 0.0, -0.0]
    np.testing.assert_array_equal(oracle.widen(bits, "bf16"), np.array(want))


@pytest.mark.parametrize("ex", json.load(open(os.path.join(GOLDEN, "closed_form_examples.json")))["examples"],
                         ids=lambda e: e["name"])
def test_closed_form_examples(ex):
    q = np.array(ex["q"], dtype=np.float64)
    k = np.array(ex["k"], dtype=np.float64).reshape(-1, ex["h_kv"], ex["d"])
    v = np.array(ex["v"], dtype=np.float64).reshape(-1, ex["h_kv"], ex["d"])
    got = oracle.attend(q, k, v, np.array(ex["seq_lens"]), np.float32(ex["scale"]), ex["h_kv"], dtype="f64")
    np.testing.assert_allclose(got, np.array(ex["out"]), rtol=0, atol=1e-12)


def test_single_token_gives_its_value_row():
    rng = np.random.default_rng(5)
    q, k, v, sl = rand_case(rng, 3, 8, 2, 16, [1, 1, 1], sigma=5.0)
    got = oracle.attend(q, k, v, sl, np.float32(0.25), 2, dtype="f64")
    for b in range(3):
        for h in range(8):
            np.testing.assert_array_equal(got[b, h], v[b, h // 4])


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(6)
    q, k, v, sl = rand_case(rng, 1, 4, 2, 8, [33])
    k[:] = 0.0
    got = oracle.attend(q, k, v, sl, np.float32(0.125), 2, dtype="f64")
    for h in range(4):
        np.testing.assert_allclose(got[0, h], v[:, h // 2].mean(axis=0), rtol=0, atol=1e-14)


def test_identical_value_rows_give_that_row():
    rng = np.random.default_rng(7)
    q, k, v, sl = rand_case(rng, 2, 8, 4, 16, [100, 37], sigma=3.0)
    row = rng.standard_normal((4, 16))
    v[:] = row[None, :, :]
    got = oracle.attend(q, k, v, sl, np.float32(0.25), 4, dtype="f64")
    for b in range(2):
        for h in range(8):
            np.testing.assert_allclose(got[b, h], row[h // 2], rtol=0, atol=1e-12)


def test_one_hot_dominant_score_selects_its_row():
    d, S, t_star = 16, 200, 123
    rng = np.random.default_rng(8)
    q, k, v, sl = rand_case(rng, 1, 8, 1, d, [S])
    q[0, :, 0] = 10.0 + np.abs(q[0, :, 0])   # every head positive on coordinate 0
    k[:, 0, 0] = 0.0
    k[t_star, 0, 0] = 40.0                    # gap >= 400 * scale = 100 score units
    got = oracle.attend(q, k, v, sl, np.float32(0.25), 1, dtype="f64")
    for h in range(8):
        np.testing.assert_allclose(got[0, h], v[t_star, 0], rtol=0, atol=1e-15)


def test_large_scores_stay_finite_and_exact():
    """Scores near 1000: exp without the max subtraction would overflow."""
    q = np.array([[[1.0]]])
    k = np.array([[[1000.0]], [[1000.0 + math.log(3.0)]]])
    v = np.array([[[1.0]], [[5.0]]])
    got = oracle.attend(q, k, v, np.array([2]), np.float32(1.0), 1, dtype="f64")
    np.testing.assert_allclose(got[0, 0, 0], 4.0, rtol=0, atol=1e-12)


def test_head_mapping_is_contiguous_groups():
    """V of kv head g is the constant g: out of query head h must be h // n_rep
    (tinygrad's Attention.__call__ splits q by n_rep*head_dim, k/v by head_dim)."""
    h_q, h_kv, d, S = 16, 4, 8, 9
    rng = np.random.default_rng(9)
    q, k, v, sl = rand_case(rng, 2, h_q, h_kv, d, [S, S])
    for g in range(h_kv):
        v[:, g, :] = g
    got = oracle.attend(q, k, v, sl, np.float32(0.3), h_kv, dtype="f64")
    for h in range(h_q):
        np.testing.assert_allclose(got[:, h, :], h // (h_q // h_kv), rtol=0, atol=1e-12)


def test_token_offsets_follow_packed_layout():
    np.testing.assert_array_equal(oracle.token_offsets([3, 0, 5, 1]), [0, 3, 3, 8])
    np.testing.assert_array_equal(oracle.token_offsets([7]), [0])


def test_ragged_batch_equals_independent_sequences():
    rng = np.random.default_rng(10)
    lens = [5, 0, 17, 1]
    q, k, v, sl = rand_case(rng, 4, 8, 2, 8, lens)
    got = oracle.attend(q, k, v, sl, np.float32(0.35), 2, dtype="f64")
    start = 0
    for b, S in enumerate(lens):
        one = oracle.attend(q[b:b + 1], k[start:start + S], v[start:start + S],
                            np.array([S]), np.float32(0.35), 2, dtype="f64")
        np.testing.assert_array_equal(got[b], one[0])
        start += S


def test_gqa_equals_mha_on_repeated_kv_via_torch():
    """Library special case: torch's CPU scaled_dot_product_attention in
    float64, with each kv head repeated n_rep times, is plain MHA."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    B, h_q, h_kv, d, S = 1, 8, 2, 32, 77
    q, k, v, sl = rand_case(rng, B, h_q, h_kv, d, [S], sigma=1.5)
    scale = np.float32(1 / math.sqrt(d))
    got = oracle.attend(q, k, v, sl, scale, h_kv, dtype="f64")
    n_rep = h_q // h_kv
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(n_rep, dim=0)[None]  # [1,h_q,S,d]
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(n_rep, dim=0)[None]
    qt = torch.from_numpy(q)[:, :, None, :]                                           # [1,h_q,1,d]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale))
    np.testing.assert_allclose(got, ref[:, :, 0, :].numpy(), rtol=0, atol=1e-12)


def test_shift_of_all_scores_changes_nothing():
    rng = np.random.default_rng(12)
    s = rng.standard_normal(300) * 4
    vr = rng.standard_normal((300, 8))
    a = oracle.finalize(oracle.triplet(s, vr))
    b = oracle.finalize(oracle.triplet(s + 123.25, vr))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_output_inside_value_hull():
    w = workloads.custom("hull", B=2, h_q=8, h_kv=2, d=16, seq_lens=[50, 300], seed=13, k_sigma=2.0)
    out = oracle.attend(w.q, w.k, w.v, w.seq_lens, w.scale, 2, dtype="bf16")
    vf = oracle.widen(w.v, "bf16")
    start = 0
    for b, S in enumerate(w.seq_lens):
        for h in range(8):
            rows = vf[start:start + S, h // 4]
            assert np.all(out[b, h] <= rows.max(axis=0) + 1e-12)
            assert np.all(out[b, h] >= rows.min(axis=0) - 1e-12)
        start += S


def test_workload_shapes_match_printed_llama2_configs():
    cfg = json.load(open(os.path.join(GOLDEN, "llama2_70b_config.json")))
    heads = json.load(open(os.path.join(GOLDEN, "llama2_head_counts.json")))
    d70 = cfg["hidden_size"] // cfg["num_attention_heads"]
    for name in ["llama70b_gqa_b1_s8192", "llama70b_gqa_b8_ragged", "llama70b_gqa_b1_s1m"]:
        w = workloads.WORKLOADS[name]
        assert (w.h_q, w.h_kv, w.d) == (cfg["num_attention_heads"], cfg["num_key_value_heads"], d70)
        assert w.n_rep == 8
    w7 = workloads.WORKLOADS["llama2_7b_mha_s4096"]
    assert w7.h_q == heads["heads"]["7B"] and w7.h_kv == w7.h_q   # MHA: n_rep = 1
    assert "7B" in heads["multi_head_attention"]


def test_scores_on_hand_values():
    """s_t = scale * <q, K_t>, worked by hand: q = (1, 2, -1), scale 0.5,
    K rows (1, 0, 0), (0, 1, 1), (2, -1, 3) -> 0.5 * (1, 1, -3)."""
    q = np.array([1.0, 2.0, -1.0])
    k = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 1.0], [2.0, -1.0, 3.0]])
    np.testing.assert_array_equal(oracle.scores(q, k, np.float32(0.5)), [0.5, 0.5, -1.5])
    # the scale is the float32 value the GPU receives, widened
    np.testing.assert_array_equal(oracle.scores(np.array([1.0]), np.array([[1.0]]), 0.1),
                                  [float(np.float32(0.1))])


def test_scores_triplet_finalize_is_brute_force():
    """The chunk pieces composed by hand (scores of one head, its triplet,
    o / l) give the brute-force attention of that head, with a scale that is
    neither 1 nor 1/sqrt(d) and a negative one."""
    rng = np.random.default_rng(14)
    q, k, v, sl = rand_case(rng, 1, 2, 1, 5, [23], sigma=2.0)
    for scale in (np.float32(0.37), np.float32(-1.3)):
        ref = np.array(attend_brute(q.tolist(), k.tolist(), v.tolist(), sl, float(scale), 1))
        for h in range(2):
            s = oracle.scores(q[0, h], k[:, 0, :], scale)
            got = oracle.finalize(oracle.triplet(s, v[:, 0, :]))
            np.testing.assert_allclose(got, ref[0, h], rtol=0, atol=1e-13)
