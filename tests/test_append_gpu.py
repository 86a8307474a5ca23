"""GPU checks of the KV-cache append: byte-exact against oracle.kv_append,
and an append + attend decode step against the oracle on the full cache."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_F32, max_err

pytestmark = pytest.mark.gpu


def bf16_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def back(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n_new", [1, 3, 130])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("explicit", [False, True])
def test_append_is_byte_exact(n_new, d, explicit):
    import torch

    import decode_attention_gqa_amd as gqa
    B, h_kv, cap = 5, 4, 300
    rng = np.random.default_rng(n_new + d)
    lens = np.array([0, 17, 299, 300 - n_new, 150], dtype=np.int32)
    rows = B * cap + (7 if explicit else 0)
    kc = workloads.normals(1, 1, rows * h_kv * d).reshape(rows, h_kv, d)
    vc = workloads.normals(1, 2, rows * h_kv * d).reshape(rows, h_kv, d)
    kn = workloads.normals(1, 3, B * n_new * h_kv * d).reshape(B, n_new, h_kv, d)
    vn = workloads.normals(1, 4, B * n_new * h_kv * d).reshape(B, n_new, h_kv, d)
    offs = (np.arange(B) * cap + 7)[::-1].copy() if explicit else None    # sequences in reverse order
    ref_k, ref_v, ref_l = oracle.kv_append(kc, vc, kn, vn, lens, cap, kv_offsets=offs)
    k_d, v_d = bf16_dev(kc), bf16_dev(vc)
    lens_d = torch.from_numpy(lens).cuda()
    lens_out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    gqa.gqa_kv_append(bf16_dev(kn), bf16_dev(vn), k_d, v_d, lens_d, capacity=cap, seq_lens_out=lens_out,
                      kv_token_offsets=torch.from_numpy(offs).cuda() if explicit else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(back(k_d), ref_k)
    np.testing.assert_array_equal(back(v_d), ref_v)
    np.testing.assert_array_equal(lens_out.cpu().numpy(), ref_l)
    np.testing.assert_array_equal(lens_d.cpu().numpy(), lens)               # input lengths untouched


def test_fp32_append_and_no_length_output():
    import torch

    import decode_attention_gqa_amd as gqa
    B, h_kv, d, cap = 2, 2, 64, 10
    kc = np.zeros((B * cap, h_kv, d), dtype=np.float32)
    kn = np.arange(B * 2 * h_kv * d, dtype=np.float32).reshape(B, 2, h_kv, d)
    lens = np.array([3, 9], dtype=np.int32)
    ref_k, ref_v, _ = oracle.kv_append(kc, kc, kn, -kn, lens, cap)
    k_d = torch.from_numpy(kc.copy()).cuda(); v_d = torch.from_numpy(kc.copy()).cuda()
    gqa.gqa_kv_append(torch.from_numpy(kn).cuda(), torch.from_numpy(-kn).cuda(), k_d, v_d,
                      torch.from_numpy(lens).cuda(), capacity=cap)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(k_d.cpu().numpy(), ref_k)
    np.testing.assert_array_equal(v_d.cpu().numpy(), ref_v)


def test_decode_steps_append_then_attend():
    """Three decode steps on a padded cache: append the new token's K/V, then
    attend with the new lengths (lengths ping-pong between two buffers)."""
    import torch

    import decode_attention_gqa_amd as gqa
    B, h_q, h_kv, d, cap = 4, 64, 8, 128, 2048
    lens0 = np.array([1000, 1, 2000, 517], dtype=np.int32)
    steps = 3
    full = workloads.normals(5, 1, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    fullv = workloads.normals(5, 2, B * cap * h_kv * d).reshape(B * cap, h_kv, d)
    k_d, v_d = bf16_dev(full), bf16_dev(fullv)
    for b in range(B):                                   # rows at and after the prefix: junk
        k_d[b * cap + lens0[b]:(b + 1) * cap] = 3.0
        v_d[b * cap + lens0[b]:(b + 1) * cap] = -3.0
    lens = [torch.from_numpy(lens0).cuda(), torch.empty(B, dtype=torch.int32, device="cuda")]
    offs = torch.arange(B, dtype=torch.int64, device="cuda") * cap
    for t in range(steps):
        kn = np.stack([full[b * cap + lens0[b] + t] for b in range(B)])[:, None]
        vn = np.stack([fullv[b * cap + lens0[b] + t] for b in range(B)])[:, None]
        gqa.gqa_kv_append(bf16_dev(kn), bf16_dev(vn), k_d, v_d, lens[t % 2], capacity=cap,
                          seq_lens_out=lens[(t + 1) % 2], kv_token_offsets=offs)
        q = workloads.normals(6, t, B * h_q * d).reshape(B, h_q, d)
        out = gqa.gqa_decode_attn_ex(bf16_dev(q), k_d, v_d, lens[(t + 1) % 2], kv_token_offsets=offs,
                                     s_kv_hint=cap)
        torch.cuda.synchronize()
        new_lens = lens0 + t + 1
        ref = np.zeros((B, h_q, d))
        for b in range(B):
            rows = slice(b * cap, b * cap + new_lens[b])
            ref[b] = oracle.attend(q[b:b + 1], full[rows], fullv[rows], new_lens[b:b + 1], np.float32(d ** -0.5),
                                   h_kv, dtype="bf16")[0]
        err = max_err(out.cpu().numpy().astype(np.float64), ref)
        print(f"[append] step {t}: max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32
        np.testing.assert_array_equal(lens[(t + 1) % 2].cpu().numpy(), new_lens)
