"""GPU checks of gqa_decode_step (append one token per sequence + attend, with
the append folded into the split kernel): the cache bytes and new lengths
equal oracle.kv_append's, the output equals the oracle's attention over the
grown cache within tolerance, and equals - bit for bit - the two separate
calls (gqa_kv_append, then gqa_decode_attn_ex) on a copy of the cache.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err

pytestmark = pytest.mark.gpu


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_case(lens, cap, h_q, h_kv, d, explicit, out_dtype="f32", n_splits=0, seed=0):
    import torch

    import decode_attention_gqa_amd as gqa
    B = len(lens)
    lens = np.asarray(lens, dtype=np.int32)
    T = B * cap + (7 if explicit else 0)
    k0 = workloads.normals(90 + seed, 1, T * h_kv * d).reshape(T, h_kv, d)
    v0 = workloads.normals(90 + seed, 2, T * h_kv * d).reshape(T, h_kv, d)
    kn = workloads.normals(90 + seed, 3, B * h_kv * d).reshape(B, 1, h_kv, d)
    vn = workloads.normals(90 + seed, 4, B * h_kv * d).reshape(B, 1, h_kv, d)
    q = workloads.normals(90 + seed, 5, B * h_q * d).reshape(B, h_q, d)
    # explicit offsets: sequences in reverse order, shifted by 7 rows
    offs = (np.arange(B)[::-1] * cap + 7).astype(np.int64) if explicit else None
    print(f"[case] step lens={lens.tolist()} cap={cap} h_q={h_q} h_kv={h_kv} d={d} explicit={explicit} "
          f"out={out_dtype} ns={n_splits}", flush=True)

    kc_ref, vc_ref, lens_ref = oracle.kv_append(k0, v0, kn, vn, lens, cap, offs)
    ref = np.zeros((B, h_q, d))
    for b in range(B):
        off = int(offs[b]) if explicit else b * cap
        rows = slice(off, off + int(lens_ref[b]))
        ref[b] = oracle.attend(q[b:b + 1], kc_ref[rows], vc_ref[rows], lens_ref[b:b + 1], np.float32(d ** -0.5),
                               h_kv, dtype="bf16")[0]

    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    offs_d = torch.from_numpy(offs).cuda() if explicit else None
    kc, vc = bf16_dev(k0), bf16_dev(v0)
    lens_in = torch.from_numpy(lens).cuda()
    lens_out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    out = gqa.gqa_decode_step(bf16_dev(q), bf16_dev(kn), bf16_dev(vn), kc, vc, lens_in, lens_out, capacity=cap,
                              kv_token_offsets=offs_d, out_dtype=odt, n_splits=n_splits)
    # the same step as two calls, on a second copy of the cache
    kc2, vc2 = bf16_dev(k0), bf16_dev(v0)
    lens_out2 = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    offs2 = offs_d if explicit else torch.arange(B, dtype=torch.int64, device="cuda") * cap
    gqa.gqa_kv_append(bf16_dev(kn), bf16_dev(vn), kc2, vc2, lens_in, capacity=cap, seq_lens_out=lens_out2,
                      kv_token_offsets=offs2)
    out2 = gqa.gqa_decode_attn_ex(bf16_dev(q), kc2, vc2, lens_out2, kv_token_offsets=offs2, s_kv_hint=cap,
                                  out_dtype=odt, n_splits=n_splits)
    torch.cuda.synchronize()

    np.testing.assert_array_equal(lens_out.cpu().numpy(), lens_ref)
    np.testing.assert_array_equal(bits(kc), kc_ref)
    np.testing.assert_array_equal(bits(vc), vc_ref)
    np.testing.assert_array_equal(lens_in.cpu().numpy(), lens)           # input lengths untouched
    got = out.float().cpu().numpy().astype(np.float64)
    err = max_err(got, ref)
    tol = TOL_BF16 if out_dtype == "bf16" else TOL_F32
    print(f"[step] max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol
    assert torch.equal(out, out2), "folded step differs from append + attend"


@pytest.mark.parametrize("explicit", [False, True])
def test_step_edge_lengths(explicit):
    """Empty sequence (the new token alone), block and chunk edges, one row
    below capacity, and a full sequence (the new token is dropped)."""
    cap = 1024
    run_case([0, 1, 31, 32, 127, 128, 1000, cap - 1, cap], cap, 64, 8, 128, explicit, seed=1)


@pytest.mark.parametrize("n_rep,d", [(1, 128), (2, 64), (4, 128), (16, 64)])
def test_step_head_shapes(n_rep, d):
    run_case([700, 2047, 64, 1], 2048, 2 * n_rep, 2, d, True, seed=2 + n_rep)


@pytest.mark.parametrize("ns", [1, 7, 100])
def test_step_forced_split_counts(ns):
    run_case([5000, 129, 3333], 8192, 64, 8, 128, False, n_splits=ns, seed=3)


def test_step_bf16_out():
    run_case([4095, 17], 4096, 64, 8, 128, True, out_dtype="bf16", seed=4)


def test_step_graph_loop():
    """A decode loop of gqa_decode_step captured in two graphs (lengths
    alternate between two buffers) and replayed: every replay equals the
    oracle on the grown cache."""
    import torch

    import decode_attention_gqa_amd as gqa
    B, h_q, h_kv, d, cap = 3, 64, 8, 128, 1024
    lens0 = np.array([100, 1000, 31], dtype=np.int32)
    steps = 6
    k0 = workloads.normals(95, 1, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    v0 = workloads.normals(95, 2, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    kc, vc = bf16_dev(k0), bf16_dev(v0)
    lens = [torch.from_numpy(lens0).cuda(), torch.zeros(B, dtype=torch.int32, device="cuda")]
    kn_d = torch.empty((B, h_kv, d), dtype=torch.bfloat16, device="cuda")
    vn_d = torch.empty_like(kn_d)
    q_d = torch.empty((B, h_q, d), dtype=torch.bfloat16, device="cuda")
    out_d = torch.empty((B, h_q, d), dtype=torch.float32, device="cuda")
    ns = gqa.gqa_decode_pick_splits_d(B, h_kv, d, cap)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, h_q, d, ns), dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    graphs = []
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            gqa.gqa_decode_step(q_d, kn_d, vn_d, kc, vc, lens[i], lens[1 - i], out_d, capacity=cap, workspace=ws)
        graphs.append(g)
    torch.cuda.synchronize()

    kc_ref, vc_ref, lens_ref = k0, v0, lens0
    for t in range(steps):
        kn = workloads.normals(96, t, B * h_kv * d).reshape(B, 1, h_kv, d)
        vn = workloads.normals(97, t, B * h_kv * d).reshape(B, 1, h_kv, d)
        q = workloads.normals(98, t, B * h_q * d).reshape(B, h_q, d)
        kn_d.copy_(bf16_dev(kn).view(B, h_kv, d))
        vn_d.copy_(bf16_dev(vn).view(B, h_kv, d))
        q_d.copy_(bf16_dev(q))
        out_d.fill_(float("nan"))
        torch.cuda.synchronize()
        graphs[t % 2].replay()
        torch.cuda.synchronize()
        kc_ref, vc_ref, lens_ref = oracle.kv_append(kc_ref, vc_ref, kn, vn, lens_ref, cap)
        np.testing.assert_array_equal(lens[(t + 1) % 2].cpu().numpy(), lens_ref)
        ref = np.zeros((B, h_q, d))
        for b in range(B):
            rows = slice(b * cap, b * cap + int(lens_ref[b]))
            ref[b] = oracle.attend(q[b:b + 1], kc_ref[rows], vc_ref[rows], lens_ref[b:b + 1],
                                   np.float32(d ** -0.5), h_kv, dtype="bf16")[0]
        err = max_err(out_d.cpu().numpy().astype(np.float64), ref)
        print(f"[step-graph] step {t}: lens={lens_ref.tolist()} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32
    np.testing.assert_array_equal(bits(kc), kc_ref)
    np.testing.assert_array_equal(bits(vc), vc_ref)


@pytest.mark.parametrize("explicit,ns", [(False, 0), (True, 0), (False, 2)])
def test_step_short_capacity_one_wave(explicit, ns):
    """A capacity of 100 tokens puts every chunk at 128 tokens or fewer, and 70
    sequences x 8 kv heads give more than two chunks per compute unit: the
    step and the two-call path both take one-wave workgroups (same bits)."""
    run_case([0, 1, 31, 32, 63, 99, 100] * 10, 100, 64, 8, 128, explicit, n_splits=ns, seed=6)


@pytest.mark.parametrize("explicit", [False, True])
def test_step_single_sequence_eight_wave(explicit):
    """One sequence in a 16384-token cache: 32 chunks of 512 tokens, 8-wave
    workgroups in the step and in the two-call path alike (same bits)."""
    run_case([12000], 16384, 64, 8, 128, explicit, seed=7)
