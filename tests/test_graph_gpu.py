"""A decode loop captured once in HIP graphs and replayed step after step.

The kernels take the sequence lengths from device memory, so a graph holding
one decode step (append the new token's K/V, then attend) stays valid while
the lengths grow: with the lengths alternating between two buffers, two
graphs (buffer 0 -> 1 and 1 -> 0) serve every step. Each replay is checked
against the oracle on the cache as it stands after that step, with eager
work and synchronisations between replays.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_F32, max_err

pytestmark = pytest.mark.gpu


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def test_graph_decode_loop_append_attend():
    import torch

    import decode_attention_gqa_amd as gqa
    B, h_q, h_kv, d, cap = 4, 64, 8, 128, 2048
    lens0 = np.array([1000, 1, 2000, 517], dtype=np.int32)
    steps = 6                                            # 2000 + 6 <= cap
    full = workloads.normals(7, 1, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    fullv = workloads.normals(7, 2, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    k_d, v_d = bf16_dev(full), bf16_dev(fullv)
    for b in range(B):                                   # rows after each prefix: junk until appended
        k_d[b * cap + lens0[b]:(b + 1) * cap] = 3.0
        v_d[b * cap + lens0[b]:(b + 1) * cap] = -3.0
    lens = [torch.from_numpy(lens0).cuda(), torch.zeros(B, dtype=torch.int32, device="cuda")]
    offs = torch.arange(B, dtype=torch.int64, device="cuda") * cap
    # Fixed buffers the graphs read and write.
    kn_d = torch.empty((B, 1, h_kv, d), dtype=torch.bfloat16, device="cuda")
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
            gqa.gqa_kv_append(kn_d, vn_d, k_d, v_d, lens[i], capacity=cap, seq_lens_out=lens[1 - i],
                              kv_token_offsets=offs)
            gqa.gqa_decode_attn_ex(q_d, k_d, v_d, lens[1 - i], out_d, kv_token_offsets=offs, s_kv_hint=cap,
                                   workspace=ws)
        graphs.append(g)
    torch.cuda.synchronize()
    assert torch.equal(lens[0].cpu(), torch.from_numpy(lens0)), "capture must not run the kernels"

    for t in range(steps):
        kn = np.stack([full[b * cap + lens0[b] + t] for b in range(B)])[:, None]
        vn = np.stack([fullv[b * cap + lens0[b] + t] for b in range(B)])[:, None]
        q = workloads.normals(8, t, B * h_q * d).reshape(B, h_q, d)
        kn_d.copy_(bf16_dev(kn))
        vn_d.copy_(bf16_dev(vn))
        q_d.copy_(bf16_dev(q))
        out_d.fill_(float("nan"))
        torch.cuda.synchronize()
        graphs[t % 2].replay()
        torch.cuda.synchronize()
        new_lens = lens0 + t + 1
        np.testing.assert_array_equal(lens[(t + 1) % 2].cpu().numpy(), new_lens)
        ref = np.zeros((B, h_q, d))
        for b in range(B):
            rows = slice(b * cap, b * cap + new_lens[b])
            ref[b] = oracle.attend(q[b:b + 1], full[rows], fullv[rows], new_lens[b:b + 1], np.float32(d ** -0.5),
                                   h_kv, dtype="bf16")[0]
        err = max_err(out_d.cpu().numpy().astype(np.float64), ref)
        print(f"[graph] step {t}: lens={new_lens.tolist()} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32
        # eager work between replays: the same step on copies must agree bit for bit
        lens_e = lens[(t + 1) % 2].clone()
        e = gqa.gqa_decode_attn_ex(q_d, k_d, v_d, lens_e, kv_token_offsets=offs, s_kv_hint=cap)
        torch.cuda.synchronize()
        assert torch.equal(e, out_d), f"step {t}: graph replay differs from the eager call"


def test_one_graph_serves_every_length_without_a_hint():
    """A call without a length hint (one sequence: one round of 8-wave
    workgroups whose chunks are sized on the device) captured once and
    replayed while the length in device memory changes from a few tokens to
    the whole cache: every replay matches the oracle, with eager work and
    synchronisations between replays."""
    import torch

    import decode_attention_gqa_amd as gqa
    h_q, h_kv, d, cap = 64, 8, 128, 20000
    k = workloads.normals(9, 1, cap * h_kv * d).reshape(cap, h_kv, d)
    v = workloads.normals(9, 2, cap * h_kv * d).reshape(cap, h_kv, d)
    q = workloads.normals(9, 3, h_q * d).reshape(1, h_q, d)
    k_d, v_d, q_d = bf16_dev(k), bf16_dev(v), bf16_dev(q)
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_d = torch.empty((1, h_q, d), dtype=torch.float32, device="cuda")
    ns = gqa.gqa_decode_pick_splits_d(1, h_kv, d, 0)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(1, h_q, d, ns), dtype=torch.uint8, device="cuda")
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        gqa.gqa_decode_attn_ex(q_d, k_d, v_d, lens, out_d, s_kv_hint=0, workspace=ws)
    torch.cuda.synchronize()
    scale = np.float32(d ** -0.5)
    for S in (3, 700, 8192, 8193, 20000, 31):
        lens.fill_(S)
        out_d.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.attend(q, k[:S], v[:S], np.array([S], dtype=np.int32), scale, h_kv, dtype="bf16")
        err = max_err(out_d.cpu().numpy().astype(np.float64), ref)
        print(f"[graph, no hint] S={S} n_splits={ns} max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32
