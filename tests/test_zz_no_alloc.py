"""The no-allocation entry point (gqa_decode_attn_noalloc) against the
existing one it varies (gqa_decode_attn_ex with a caller workspace), through
the C ABI: two calls in a row, the second with a smaller input, so the
second runs on the scratch the first left behind. Both use the same kernels
and plan, so the results are compared bit for bit, and each against the fp64
oracle within the fp32 / bf16 tolerances."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err, to_device

pytestmark = pytest.mark.gpu


def _pair(inp, out_dtype, hint, n_splits=0, fused=False):
    import torch

    import decode_attention_gqa_amd as gqa
    w = inp.w
    q, k, v, lens = to_device(inp)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    s_max = int(inp.seq_lens.max())
    h = s_max if hint else 0
    ns = n_splits if n_splits > 0 else gqa.gqa_decode_pick_splits_d(w.B, w.h_kv, w.d, h)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B, w.h_q, w.d, ns), dtype=torch.uint8, device=q.device)
    ws.view(torch.float32).fill_(float("nan"))
    ref = gqa.gqa_decode_attn_ex(q, k, v, lens, scale=float(inp.scale), n_splits=n_splits, out_dtype=odt,
                                 s_kv_hint=h, workspace=ws, fused=fused)
    out = torch.full((w.B, w.h_q, w.d), float("nan"), dtype=odt, device=q.device)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    gqa.gqa_decode_attn_noalloc(q, k, v, lens, out, scale=float(inp.scale), n_splits=n_splits, s_kv_hint=h,
                                fused=fused)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0          # nothing allocated on the device
    return ref, out


@pytest.mark.parametrize("out_dtype,hint,fused", [("f32", True, False), ("bf16", False, False),
                                                  ("f32", True, True)])
def test_noalloc_equals_ex_on_two_calls(out_dtype, hint, fused):
    big = workloads.custom("noalloc_big", B=3, h_q=64, h_kv=8, d=128, seq_lens=[5000, 1234, 77], seed=31)
    small = workloads.custom("noalloc_small", B=1, h_q=64, h_kv=8, d=128, seq_lens=[999], seed=32)
    tol = TOL_BF16 if out_dtype == "bf16" else TOL_F32
    for inp in (big, small):                  # the second call is smaller
        ref, out = _pair(inp, out_dtype, hint, fused=fused)
        assert bool((out.view(-1) == ref.view(-1)).all()), f"{inp.w.name}: differs from gqa_decode_attn_ex"
        want = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv, dtype=inp.w.dtype)
        err = max_err(out.float().cpu().numpy().astype(np.float64), want)
        assert err <= tol, f"{inp.w.name}: max abs error {err}"


def test_noalloc_forced_splits_and_70b_shape():
    """The bench workload's shapes (B = 1, 8192 tokens, 8-wave form) with the
    heuristic's split count, then a forced count on a shorter sequence."""
    big = workloads.custom("noalloc_8k", B=1, h_q=64, h_kv=8, d=128, seq_lens=[8192], seed=33)
    small = workloads.custom("noalloc_short", B=2, h_q=64, h_kv=8, d=128, seq_lens=[700, 0], seed=34)
    for inp, ns in ((big, 0), (small, 5)):
        ref, out = _pair(inp, "f32", True, n_splits=ns)
        assert bool((out == ref).all())
        want = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv, dtype=inp.w.dtype)
        assert max_err(out.double().cpu().numpy(), want) <= TOL_F32


def test_noalloc_rejects_oversized_plan_without_launching():
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.custom("noalloc_reject", B=1, h_q=64, h_kv=8, d=128, seq_lens=[4096], seed=35)
    q, k, v, lens = to_device(inp)
    out = torch.zeros((1, 64, 128), dtype=torch.float32, device=q.device)
    with pytest.raises(gqa.GQAError) as e:
        gqa.gqa_decode_attn_noalloc(q, k, v, lens, out, n_splits=1024)
    assert e.value.status == gqa.GQA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not out.any()                       # nothing was written
