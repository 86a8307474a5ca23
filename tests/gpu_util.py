"""Helpers shared by the GPU tests: upload seeded inputs and run the library."""
from __future__ import annotations

import functools

import numpy as np

import workloads

TOL_F32 = 5e-3      # max abs error vs the fp64 oracle, fp32 output
TOL_BF16 = 1.6e-2   # max abs error vs the fp64 oracle, bf16-rounded output


def to_device(inp: workloads.Inputs, device="cuda"):
    import torch

    def conv(a):
        if inp.w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return conv(inp.q), conv(inp.k), conv(inp.v), torch.from_numpy(inp.seq_lens).to(device)


def run_gpu(inp: workloads.Inputs, n_splits=0, out_dtype="f32", valu=False, poison=True,
            hint=True, dev=None, stream=None, fused=False):
    """Run the library on `inp`; returns (out as float64 numpy, split count used).

    The workspace is filled with NaN first, so a chunk the merge reads but no
    split workgroup wrote shows up as NaN in the output.
    """
    import torch

    import decode_attention_gqa_amd as gqa
    q, k, v, lens = dev if dev is not None else to_device(inp)
    w = inp.w
    s_max = int(inp.seq_lens.max()) if len(inp.seq_lens) else 0
    hint_v = (s_max if hint else 0) if isinstance(hint, bool) else int(hint)   # an int: that hint
    ns = n_splits if n_splits > 0 else gqa.gqa_decode_pick_splits_d(w.B, w.h_kv, w.d, hint_v)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(w.B, w.h_q, w.d, ns), dtype=torch.uint8, device=q.device)
    if poison:   # every byte, the arrival counters included
        ws.view(torch.float32).fill_(float("nan"))
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = gqa.gqa_decode_attn_ex(q, k, v, lens, scale=float(inp.scale), n_splits=n_splits,
                                 out_dtype=odt, s_kv_hint=hint_v, workspace=ws, valu=valu,
                                 stream=stream, fused=fused)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), ns


def max_err(got, ref) -> float:
    ok = ~np.isnan(ref)
    if not np.all(np.isfinite(got[ok])):
        return float("inf")
    return float(np.max(np.abs(got[ok] - ref[ok]))) if ok.any() else 0.0


@functools.lru_cache(maxsize=2)
def oracle_all_heads(name: str) -> np.ndarray:
    """The fp64 oracle on every head of a named workload, one kv group at a
    time (for the 1M-token workload a group's K and V in fp64 are 2 GiB, so
    host memory stays bounded). Cached per process: the parity and the
    single-launch tests share it."""
    import oracle
    inp = workloads.make_inputs(name)
    w = inp.w
    out = np.full((w.B, w.h_q, w.d), np.nan)
    for g in range(w.h_kv):
        heads = [(b, h) for b in range(w.B) for h in range(g * w.n_rep, (g + 1) * w.n_rep)]
        part = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, w.h_kv, dtype=w.dtype, heads=heads)
        for b, h in heads:
            out[b, h] = part[b, h]
        print(f"[oracle] {name}: kv group {g} done", flush=True)
    return out
