"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Bar: max abs error <= 5e-3 with fp32 output, <= 1.6e-2 with bf16 output, on
the same seeded inputs. Each case prints its name, shape and error first, so
a failing run names its case.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err, oracle_all_heads, run_gpu, to_device

pytestmark = pytest.mark.gpu


def ref_of(inp, heads=None):
    return oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv,
                         dtype=inp.w.dtype, heads=heads)


def report(name, err, ns, tol):
    print(f"[parity] {name}: n_splits={ns} max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol, f"{name}: max abs error {err} > {tol}"


@pytest.mark.parametrize("name", ["tiny_gqa_f32", "llama2_7b_mha_s4096", "llama70b_gqa_b1_s8192",
                                  "llama70b_gqa_b8_ragged"])
def test_workload_parity(name):
    inp = workloads.make_inputs(name)
    print(f"[case] {name} B={inp.w.B} lens={inp.seq_lens.tolist()}", flush=True)
    got, ns = run_gpu(inp, n_splits=inp.w.n_splits)
    report(name, max_err(got, ref_of(inp)), ns, TOL_F32)


@pytest.mark.parametrize("name", ["llama2_7b_mha_s4096", "llama70b_gqa_b1_s8192"])
def test_workload_parity_bf16_out(name):
    inp = workloads.make_inputs(name)
    got, ns = run_gpu(inp, out_dtype="bf16")
    report(name + "/bf16-out", max_err(got, ref_of(inp)), ns, TOL_BF16)


def test_bf16_output_is_rounded_fp32_output():
    inp = workloads.make_inputs("llama70b_gqa_b1_s8192")
    dev = to_device(inp)
    f32, _ = run_gpu(inp, dev=dev)
    b16, _ = run_gpu(inp, out_dtype="bf16", dev=dev)
    rounded = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(f32.astype(np.float32)))
    np.testing.assert_array_equal(b16, rounded.astype(np.float64))


def test_long_context_1m_every_head():
    """Full-size 1M-token case (4 GiB KV, K ~ N(0, 4), so the running max
    grows many times along the sequence): every one of the 64 heads, in all 8
    kv groups, against the fp64 oracle (computed one kv group at a time), with
    the split count the length hint gives (256 chunks of 4096 tokens)."""
    inp = workloads.make_inputs("llama70b_gqa_b1_s1m")
    print(f"[case] 1M B=1 S={int(inp.seq_lens[0])}", flush=True)
    got, ns = run_gpu(inp)
    ref = oracle_all_heads("llama70b_gqa_b1_s1m")
    assert not np.isnan(ref).any()
    report("llama70b_gqa_b1_s1m/all heads", max_err(got, ref), ns, TOL_F32)
    vmin = workloads.bf16_bits_to_f32(inp.v).min(axis=0)  # [h_kv, d]
    vmax = workloads.bf16_bits_to_f32(inp.v).max(axis=0)
    g = np.arange(64) // 8
    assert np.all(got[0] <= vmax[g] + 1e-6) and np.all(got[0] >= vmin[g] - 1e-6)


def test_long_context_1m_base_entry_point():
    """The base entry point (no length hint: it plans without knowing S) at
    1M tokens, every head against the oracle."""
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b1_s1m")
    q, k, v, lens = to_device(inp)
    out = gqa.gqa_decode_attn(q, k, v, lens, scale=float(inp.scale))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    report("llama70b_gqa_b1_s1m/base entry", max_err(got, oracle_all_heads("llama70b_gqa_b1_s1m")), 0, TOL_F32)


@pytest.mark.parametrize("valu", [False, True], ids=["mfma", "valu"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16])
def test_shapes_ragged_tail(n_rep, d, valu):
    """Several 32/64-token blocks per chunk plus ragged tails, 3 sequences."""
    inp = workloads.custom(f"grid_r{n_rep}_d{d}", B=3, h_q=2 * n_rep, h_kv=2, d=d,
                           seq_lens=[1000, 37, 2049], seed=20 + n_rep + d)
    ref = ref_of(inp)
    for ns in (0, 7):
        got, used = run_gpu(inp, n_splits=ns, valu=valu)
        report(f"grid n_rep={n_rep} d={d} {'valu' if valu else 'mfma'} ns={ns}", max_err(got, ref), used, TOL_F32)


@pytest.mark.parametrize("n_rep,d", [(4, 64), (8, 128), (1, 128)])
def test_fp32_inputs(n_rep, d):
    inp = workloads.custom("f32", B=2, h_q=2 * n_rep, h_kv=2, d=d, seq_lens=[333, 1200],
                           dtype="f32", seed=40 + d)
    got, ns = run_gpu(inp, n_splits=5)
    report(f"fp32 n_rep={n_rep} d={d}", max_err(got, ref_of(inp)), ns, TOL_F32)


# The merge takes up to 32 * U chunks per load round, U = 1, 2, 4, 8 by split
# count: 1..32, 33..64, 65..128, 129..256; 300 and 600 take 2 and 3 rounds
# (600 chunks of 14 tokens over 8192: only 586 are non-empty).
@pytest.mark.parametrize("ns", [1, 2, 7, 64, 100, 200, 300, 600, 0])
def test_split_counts_agree(ns):
    inp = workloads.make_inputs("llama70b_gqa_b1_s8192")
    got, used = run_gpu(inp, n_splits=ns)
    report(f"70B S=8192 ns={ns}", max_err(got, ref_of(inp)), used, TOL_F32)


_RAGGED = {}


@pytest.mark.parametrize("hint", [0, 100, 5000, 1 << 20])
def test_wrong_length_hints_only_change_the_split_count(hint):
    """s_kv_hint is a performance hint: below the real lengths (100, 5000 for
    lengths up to 32739), unknown (0) or far above them, the chunking on the
    device still covers every token with at most n_splits chunks."""
    if not _RAGGED:
        _RAGGED["inp"] = inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
        _RAGGED["ref"] = ref_of(inp)
    inp, ref = _RAGGED["inp"], _RAGGED["ref"]
    got, used = run_gpu(inp, hint=hint)
    report(f"ragged hint={hint}", max_err(got, ref), used, TOL_F32)


@pytest.mark.parametrize("ns", [33, 129, 300])
def test_split_counts_d64(ns):
    """d = 64: two 32-column slices per merged row; several load rounds."""
    inp = workloads.custom("d64", B=2, h_q=16, h_kv=4, d=64, seq_lens=[5000, 2100], seed=61)
    got, used = run_gpu(inp, n_splits=ns)
    report(f"d=64 ns={ns}", max_err(got, ref_of(inp)), used, TOL_F32)


def test_empty_short_and_block_edge_sequences():
    """S_b = 0, 1 and values around the 32-token block; more chunks than
    tokens, so some chunks are empty."""
    lens = [0, 1, 3, 31, 32, 33, 0, 64, 65]
    inp = workloads.custom("edges", B=len(lens), h_q=16, h_kv=2, d=128, seq_lens=lens, seed=50)
    ref = ref_of(inp)
    for ns in (8, 40, 1, 0):
        for valu in (False, True):
            got, used = run_gpu(inp, n_splits=ns, valu=valu)
            report(f"edges ns={ns} valu={valu}", max_err(got, ref), used, TOL_F32)
            assert np.all(got[0] == 0) and np.all(got[6] == 0)


def test_identical_value_rows():
    inp = workloads.custom("idv", B=2, h_q=64, h_kv=8, d=128, seq_lens=[3000, 517], seed=51)
    inp.v[:] = inp.v[:1]                               # every row equal to row 0
    got, ns = run_gpu(inp)
    want = workloads.bf16_bits_to_f32(inp.v[0]).astype(np.float64)   # [h_kv, d]
    for h in range(64):
        np.testing.assert_allclose(got[:, h, :], np.broadcast_to(want[h // 8], (2, 128)), rtol=0, atol=1e-5)
    report("identical V rows", max_err(got, ref_of(inp)), ns, TOL_F32)


def test_one_hot_dominant_score():
    S, t_star = 5000, 4321
    inp = workloads.custom("onehot", B=1, h_q=64, h_kv=8, d=128, seq_lens=[S], seed=52)
    one = workloads.f32_to_bf16_bits(np.float32([1.0]))[0]
    big = workloads.f32_to_bf16_bits(np.float32([60.0]))[0]
    inp.q[0, :, :] = 0
    inp.q[0, :, 0] = one                              # q = e_0 for every head
    inp.k[:, :, 0] = 0
    inp.k[t_star, :, 0] = big                         # score gap 60/sqrt(128) ~ 5.3 -> weight ~0.96 ...
    inp.k[t_star, :, 1:] = 0
    inp.q[0, :, 1] = one
    inp.k[t_star, :, 1] = workloads.f32_to_bf16_bits(np.float32([600.0]))[0]   # ... plus 53: one-hot
    got, ns = run_gpu(inp)
    want = workloads.bf16_bits_to_f32(inp.v[t_star]).astype(np.float64)
    for h in range(64):
        np.testing.assert_allclose(got[0, h], want[h // 8], rtol=0, atol=1e-6)


def test_bitwise_deterministic():
    inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
    dev = to_device(inp)
    a, _ = run_gpu(inp, dev=dev)
    b, _ = run_gpu(inp, dev=dev, poison=False)
    np.testing.assert_array_equal(a, b)


def test_padded_layout_with_token_offsets():
    import torch

    import decode_attention_gqa_amd as gqa
    lens = np.array([700, 64, 1500], dtype=np.int32)
    S_max = 1536
    inp = workloads.custom("padded", B=3, h_q=32, h_kv=4, d=128, seq_lens=lens, seed=53)
    ref = ref_of(inp)
    q, k, v, dl = to_device(inp)
    kp = torch.full((3 * S_max, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    off = np.concatenate([[0], np.cumsum(lens[:-1])])
    for b in range(3):
        kp[b * S_max:b * S_max + lens[b]] = k[off[b]:off[b] + lens[b]]
        vp[b * S_max:b * S_max + lens[b]] = v[off[b]:off[b] + lens[b]]
    offs = torch.arange(3, dtype=torch.int64, device="cuda") * S_max
    out = gqa.gqa_decode_attn_ex(q, kp, vp, dl, scale=float(inp.scale), kv_token_offsets=offs,
                                 s_kv_hint=S_max)
    torch.cuda.synchronize()
    report("padded layout", max_err(out.cpu().numpy().astype(np.float64), ref), 0, TOL_F32)


def test_base_entry_point_and_library_workspace():
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b1_s8192")
    q, k, v, dl = to_device(inp)
    ref = ref_of(inp)
    for ns in (0, 16, 128):                            # the library workspace grows
        out = gqa.gqa_decode_attn(q, k, v, dl, scale=float(inp.scale), n_splits=ns)
        torch.cuda.synchronize()
        report(f"base entry ns={ns}", max_err(out.cpu().numpy().astype(np.float64), ref), ns, TOL_F32)


@pytest.mark.parametrize("lens", [[1], [31], [32], [33], [256], [1000], [1024], [3000], [4096], [4097],
                                  [8192], [8193], [20000], [70000], [5, 0, 2049, 8191],
                                  [11032, 4287, 10486, 11180, 21209, 32739, 5895, 7145]])
def test_base_entry_point_without_hint_at_many_lengths(lens):
    """The base entry point plans without the lengths: one sequence gets one
    round of 8-wave workgroups (one per CU), a batch a grid of several rounds
    of 4-wave ones, and either sizes its chunks on the device from each
    sequence's length. Every length class (an empty sequence, one token, a
    block and one past it, lengths just past a multiple of the 32 chunks)
    against the oracle; the merge must agree with the split kernel on which
    chunks exist (the workspace is NaN-poisoned)."""
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.custom(f"nohint_{len(lens)}_{lens[0]}", B=len(lens), h_q=64, h_kv=8, d=128, seq_lens=lens,
                           seed=90 + len(lens) + lens[0] % 97)
    got, ns = run_gpu(inp, hint=False)
    assert ns == gqa.gqa_decode_pick_splits(len(lens), 8, 0)
    report(f"no hint lens={lens[:4]}", max_err(got, ref_of(inp)), ns, TOL_F32)
    if len(lens) == 1:                                 # the base entry: the same plan and bits
        q, k, v, dl = to_device(inp)
        out = gqa.gqa_decode_attn(q, k, v, dl, scale=float(inp.scale))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().astype(np.float64), got)


@pytest.mark.parametrize("hint", [0, 4096])
def test_single_empty_sequence_reads_nothing(hint):
    """One sequence of length 0 (its rows at an explicit offset into a cache
    of NaN rows): without a hint (the one-round 8-wave plan, chunks sized on
    the device) and with one, the output is exactly 0 and no row is read."""
    import torch

    import decode_attention_gqa_amd as gqa
    k = torch.full((64, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, float("nan"))
    q = torch.randn((1, 64, 128), device="cuda").to(torch.bfloat16)
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.tensor([16], dtype=torch.int64, device="cuda")
    out = gqa.gqa_decode_attn_ex(q, k, v, lens, kv_token_offsets=offs, scale=0.088, s_kv_hint=hint)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))


@pytest.mark.parametrize("h_kv,lens", [(32, [4096]), (32, [77]), (1, [50000]), (16, [9000])])
def test_base_entry_point_without_hint_other_head_counts(h_kv, lens):
    """The hint-less one-round plan at other kv-head counts (N_CU / h_kv
    chunks: 8 for MHA's 32 kv heads, 256 for one kv head, 16 for 16)."""
    import decode_attention_gqa_amd as gqa
    h_q = 32 if h_kv == 32 else 8 * h_kv
    inp = workloads.custom(f"nohint_h{h_kv}_{lens[0]}", B=1, h_q=h_q, h_kv=h_kv, d=128, seq_lens=lens,
                           seed=120 + h_kv + lens[0] % 89)
    got, ns = run_gpu(inp, hint=False)
    assert ns == gqa.gqa_decode_pick_splits(1, h_kv, 0)
    report(f"no hint h_kv={h_kv} lens={lens}", max_err(got, ref_of(inp)), ns, TOL_F32)


def test_runs_on_a_side_stream():
    import torch
    inp = workloads.make_inputs("llama2_7b_mha_s4096")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got, ns = run_gpu(inp, stream=s)
    report("side stream", max_err(got, ref_of(inp)), ns, TOL_F32)


@pytest.mark.parametrize("ns", [0, 1, 5])
def test_partial_then_merge_equals_full_call(ns):
    """The two halves give the same bits as the one-call path (with one chunk
    per sequence the one-call path writes out in the split kernel)."""
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
    q, k, v, dl = to_device(inp)
    w = inp.w
    hint = int(inp.seq_lens.max())
    n = ns if ns > 0 else gqa.gqa_decode_pick_splits_d(w.B, w.h_kv, w.d, hint)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B, w.h_q, w.d, n), dtype=torch.uint8, device="cuda")
    full = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), n_splits=ns, s_kv_hint=hint, workspace=ws)
    out = torch.empty_like(full)
    ws2 = torch.full_like(ws, 255)
    gqa.gqa_decode_partial(q, k, v, dl, ws2, scale=float(inp.scale), n_splits=ns, s_kv_hint=hint)
    gqa.gqa_decode_merge(dl, ws2, out, h_kv=w.h_kv, n_splits=ns, s_kv_hint=hint)
    torch.cuda.synchronize()
    assert torch.equal(full, out)
    report(f"partial+merge ns={ns}", max_err(out.cpu().numpy().astype(np.float64), ref_of(inp)), n, TOL_F32)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_one_chunk_per_sequence_writes_out_directly(out_dtype):
    """n_splits = 1: no merge kernel; empty sequences still give zeros, bf16
    output is the rounded fp32 output."""
    lens = [0, 1, 31, 33, 700, 0, 2048]
    inp = workloads.custom("direct", B=len(lens), h_q=64, h_kv=8, d=128, seq_lens=lens, seed=62)
    got, used = run_gpu(inp, n_splits=1, out_dtype=out_dtype)
    assert used == 1
    report(f"one chunk per sequence out={out_dtype}", max_err(got, ref_of(inp)), used,
           TOL_BF16 if out_dtype == "bf16" else TOL_F32)


@pytest.mark.parametrize("B", [63, 64, 65, 130])
def test_many_sequences_packed(B):
    """Sequence offsets are prefix sums over seq_lens; more than 64 sequences
    take more than one pass of the wave."""
    rng = np.random.default_rng(80 + B)
    lens = rng.integers(0, 300, size=B)
    lens[B // 2] = 0
    inp = workloads.custom(f"many{B}", B=B, h_q=16, h_kv=4, d=128, seq_lens=lens, seed=80 + B)
    ref = ref_of(inp)
    for ns in (0, 3):
        for valu in (False, True):
            got, used = run_gpu(inp, n_splits=ns, valu=valu)
            report(f"B={B} ns={ns} valu={valu}", max_err(got, ref), used, TOL_F32)


@pytest.mark.parametrize("B", [257, 9000])
def test_many_sequences_packed_scan(B):
    """More than 256 sequences in the packed layout: the token bases come from
    one scan launch (three 4096-sequence passes at B = 9000). The output
    equals, bit for bit, that of the same call given the bases as explicit
    offsets, and the oracle within tolerance."""
    import torch

    import decode_attention_gqa_amd as gqa
    rng = np.random.default_rng(90 + B)
    lens = rng.integers(0, 40 if B > 1000 else 300, size=B)
    lens[B // 3] = 0
    inp = workloads.custom(f"scan{B}", B=B, h_q=16, h_kv=4, d=128, seq_lens=lens, seed=90 + B)
    ref = ref_of(inp)
    dev = to_device(inp)
    q, k, v, dl = dev
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)).cuda()
    for ns, valu in ((0, False), (3, False), (3, True)):
        got, used = run_gpu(inp, n_splits=ns, valu=valu, dev=dev)
        report(f"B={B} packed ns={ns} valu={valu}", max_err(got, ref), used, TOL_F32)
        exp = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), n_splits=ns, valu=valu,
                                     s_kv_hint=int(lens.max()), kv_token_offsets=offs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got, exp.float().cpu().numpy().astype(np.float64))


# One-wave workgroups need, by the length hint, chunks of at most 128 tokens
# and more than two chunks (B * h_kv * n_splits) per compute unit: more than
# 512 on a 256-CU GPU. The cases below have 640 or more.
ONE_WAVE_UNITS = 512


@pytest.mark.parametrize("n_rep,d", [(1, 128), (8, 128), (4, 64), (16, 64)])
def test_short_sequences_one_wave(n_rep, d):
    """Chunks of at most 128 tokens, many of them: one-wave workgroups.
    Lengths 0..128 around the 32-token block edges, one chunk per sequence
    (written out directly) and forced splits (merged), fp32 and bf16 output."""
    lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 47, 63, 64, 65, 96, 127, 128] * 5
    h_kv = 8
    inp = workloads.custom(f"short{n_rep}_{d}", B=len(lens), h_q=h_kv * n_rep, h_kv=h_kv, d=d, seq_lens=lens,
                           seed=100 + n_rep + d)
    ref = ref_of(inp)
    for ns in (0, 1, 3):
        got, used = run_gpu(inp, n_splits=ns)
        assert len(lens) * h_kv * used > ONE_WAVE_UNITS
        report(f"short n_rep={n_rep} d={d} ns={ns}", max_err(got, ref), used, TOL_F32)
    got, used = run_gpu(inp, out_dtype="bf16")
    report(f"short n_rep={n_rep} d={d} bf16 out", max_err(got, ref), used, TOL_BF16)


@pytest.mark.parametrize("ns", [0, 4])
def test_one_wave_with_a_hint_below_the_lengths(ns):
    """A hint of 32 tokens picks one-wave workgroups; the real chunks are far
    longer (up to 3000 tokens), which that form walks block by block: slower,
    same result."""
    lens = [3000, 65, 0, 1000, 32] * 14
    inp = workloads.custom("onewave_hint", B=len(lens), h_q=64, h_kv=8, d=128, seq_lens=lens, seed=111)
    got, used = run_gpu(inp, n_splits=ns, hint=32)
    assert len(lens) * 8 * used > ONE_WAVE_UNITS
    report(f"one-wave hint 32 ns={ns}", max_err(got, ref_of(inp)), used, TOL_F32)


@pytest.mark.parametrize("S,d,n_rep", [(8192, 128, 8), (8193, 128, 8), (20000, 128, 4), (32768, 128, 16)])
def test_single_sequence_eight_wave(S, d, n_rep):
    """One sequence of 8k to 32k tokens over 8 kv heads of 128 dimensions: 32
    chunks of 256 to 1024 tokens, one 8-wave workgroup per compute unit
    (8193: a partial last block in every chunk)."""
    inp = workloads.custom(f"eight{S}", B=1, h_q=8 * n_rep, h_kv=8, d=d, seq_lens=[S], seed=130 + d + n_rep)
    ref = ref_of(inp)
    got, used = run_gpu(inp)
    assert used == 32
    report(f"8-wave S={S} d={d} n_rep={n_rep}", max_err(got, ref), used, TOL_F32)
    got, used = run_gpu(inp, out_dtype="bf16")
    report(f"8-wave S={S} d={d} n_rep={n_rep} bf16 out", max_err(got, ref), used, TOL_BF16)


@pytest.mark.parametrize("scale", [-0.088, 0.0, 0.6])
def test_negative_zero_and_large_scale(scale):
    """The matrix-core kernels take the scale's sign with Q and its size
    inside the exponent; a zero scale (every attended position weighs the
    same) and a large one (a peaky softmax) too. The 8-wave, 4-wave and
    one-wave forms and the vector-ALU kernel, against the oracle."""
    import torch

    import decode_attention_gqa_amd as gqa
    cases = [("8-wave", dict(B=1, h_q=64, h_kv=8, d=128, seq_lens=[8192])),
             ("4-wave", dict(B=3, h_q=16, h_kv=2, d=128, seq_lens=[700, 37, 1500])),
             ("one-wave", dict(B=200, h_q=8, h_kv=2, d=64, seq_lens=[40 + (i * 7) % 90 for i in range(200)]))]
    for name, kw in cases:
        inp = workloads.custom(f"scale_{name}", seed=61, **kw)
        ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, np.float32(scale), kw["h_kv"], dtype="bf16")
        q, k, v, dl = to_device(inp)
        for valu in (False, True):
            out = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=scale, s_kv_hint=int(max(kw["seq_lens"])), valu=valu)
            torch.cuda.synchronize()
            report(f"scale={scale} {name} valu={valu}", max_err(out.cpu().numpy().astype(np.float64), ref), 0, TOL_F32)
