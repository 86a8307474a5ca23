"""GPU parity of the single-launch form (GQA_FLAG_FUSED): the last split
workgroup of each (sequence, kv head) merges the group's triplets."""
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
    print(f"[fused] {name}: n_splits={ns} max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol, f"{name}: max abs error {err} > {tol}"


@pytest.mark.parametrize("name", ["tiny_gqa_f32", "llama2_7b_mha_s4096", "llama70b_gqa_b1_s8192",
                                  "llama70b_gqa_b8_ragged"])
def test_fused_workload_parity(name):
    inp = workloads.make_inputs(name)
    got, ns = run_gpu(inp, n_splits=inp.w.n_splits, fused=True)
    report(name, max_err(got, ref_of(inp)), ns, TOL_F32)


def test_fused_bf16_out():
    inp = workloads.make_inputs("llama70b_gqa_b1_s8192")
    got, ns = run_gpu(inp, out_dtype="bf16", fused=True)
    report("70B S=8192 bf16-out", max_err(got, ref_of(inp)), ns, TOL_BF16)


def test_fused_long_context_1m_every_head():
    """1M tokens, K ~ N(0, 4): every head of all 8 kv groups against the fp64
    oracle (shared with the two-launch parity test when both run)."""
    inp = workloads.make_inputs("llama70b_gqa_b1_s1m")
    got, ns = run_gpu(inp, fused=True)
    report("1M all heads", max_err(got, oracle_all_heads("llama70b_gqa_b1_s1m")), ns, TOL_F32)


@pytest.mark.parametrize("valu", [False, True], ids=["mfma", "valu"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rep", [1, 2, 4, 8, 16])
def test_fused_shapes_ragged_tail(n_rep, d, valu):
    inp = workloads.custom(f"fgrid_r{n_rep}_d{d}", B=3, h_q=2 * n_rep, h_kv=2, d=d,
                           seq_lens=[1000, 37, 2049], seed=60 + n_rep + d)
    ref = ref_of(inp)
    for ns in (0, 7, 40):
        got, used = run_gpu(inp, n_splits=ns, valu=valu, fused=True)
        report(f"grid n_rep={n_rep} d={d} {'valu' if valu else 'mfma'} ns={ns}", max_err(got, ref), used, TOL_F32)


def test_fused_empty_and_short_sequences():
    lens = [0, 1, 3, 31, 32, 33, 0, 64, 65]
    inp = workloads.custom("fedges", B=len(lens), h_q=16, h_kv=2, d=128, seq_lens=lens, seed=70)
    ref = ref_of(inp)
    for ns in (8, 40, 1, 0):
        for valu in (False, True):
            got, used = run_gpu(inp, n_splits=ns, valu=valu, fused=True)
            report(f"edges ns={ns} valu={valu}", max_err(got, ref), used, TOL_F32)
            assert np.all(got[0] == 0) and np.all(got[6] == 0)


def test_fused_counters_reset_between_calls():
    """Repeated calls on one workspace, with changing lengths and shapes: each
    call must leave the arrival counters at zero for the next."""
    import torch

    import decode_attention_gqa_amd as gqa
    ws = torch.full((64 << 20,), 0x5A, dtype=torch.uint8, device="cuda")   # arbitrary initial bytes
    for rep, lens in enumerate([[3000, 17, 900], [3001, 18, 901], [5, 0, 2500], [3000, 17, 900]]):
        inp = workloads.custom("freset", B=3, h_q=32, h_kv=4, d=128, seq_lens=lens, seed=71)
        q, k, v, dl = to_device(inp)
        ref = ref_of(inp)
        for ns in (0, 9):
            out = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), n_splits=ns,
                                         s_kv_hint=max(lens), workspace=ws, fused=True)
            torch.cuda.synchronize()
            report(f"reset rep={rep} ns={ns}", max_err(out.cpu().numpy().astype(np.float64), ref), ns, TOL_F32)
    used = 3 * 4                                        # B * h_kv counters, cleared by each call
    assert int(ws[:8 * used].view(torch.int64).abs().sum()) == 0


def test_fused_graph_replays_match_eager():
    """A HIP graph of fused calls, replayed several times with eager work and
    synchronisations in between; every replay must equal the eager result."""
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
    q, k, v, dl = to_device(inp)
    hint = int(inp.seq_lens.max())
    n = gqa.gqa_decode_pick_splits(8, 8, hint)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(8, 64, 128, n), dtype=torch.uint8, device="cuda")
    eager = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), s_kv_hint=hint, workspace=ws, fused=True)
    torch.cuda.synchronize()
    eager = eager.clone()
    out = torch.empty_like(eager)
    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for _ in range(3):
            gqa.gqa_decode_attn_ex(q, k, v, dl, out, scale=float(inp.scale), s_kv_hint=hint, workspace=ws,
                                   fused=True)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager call"
        e = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), s_kv_hint=hint, workspace=ws, fused=True)
        torch.cuda.synchronize()
        assert torch.equal(e, eager)
    report("graph replays", max_err(eager.cpu().numpy().astype(np.float64), ref_of(inp)), n, TOL_F32)
