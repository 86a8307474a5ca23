"""Randomised GPU parity: seeded draws over the whole argument space of
gqa_decode_attn_ex (batch, head grouping, head size, lengths with empty
sequences and block edges, packed or offset layout with unused gaps between
sequences, split count, length hint below / at / above the lengths or none,
input and output dtypes, the vector-ALU kernel, the single-launch form),
each case checked against the fp64 oracle. The gaps of the offset layout
hold NaN, so a read outside a sequence's rows would show in the output.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err, to_device

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw(i):
    r = np.random.default_rng(5000 + i)
    B = int(r.integers(1, 13))
    h_kv = int(r.choice([1, 2, 4, 8]))
    n_rep = int(r.choice([1, 2, 4, 8, 16]))
    while h_kv * n_rep > 64:
        h_kv //= 2
    d = int(r.choice([64, 128]))
    s_top = int(r.choice([40, 300, 3000, 9000]))
    lens = r.integers(0, s_top + 1, size=B)
    edges = [0, 1, 31, 32, 33, 127, 128, 129]
    for b in range(B):
        if r.random() < 0.3:
            lens[b] = min(s_top, int(r.choice(edges)))
    case = dict(B=B, h_kv=h_kv, h_q=h_kv * n_rep, d=d, lens=lens.astype(np.int32),
                dtype="f32" if r.random() < 0.15 else "bf16",
                offsets=bool(r.random() < 0.4),
                ns=int(r.choice([0, 0, 0, 1, 2, 5, 17, 64, 200])),
                hint=str(r.choice(["exact", "exact", "none", "below", "above"])),
                out="bf16" if r.random() < 0.25 else "f32",
                valu=bool(r.random() < 0.2), fused=bool(r.random() < 0.15), seed=5000 + i)
    return case


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    import torch

    import decode_attention_gqa_amd as gqa
    c = draw(i)
    lens = c["lens"]
    s_max = int(lens.max())
    hint = {"exact": s_max, "none": 0, "below": s_max // 3, "above": 4 * s_max + 1}[c["hint"]]
    print(f"[case {i}] B={c['B']} h_q={c['h_q']} h_kv={c['h_kv']} d={c['d']} lens={lens.tolist()} "
          f"dtype={c['dtype']} offsets={c['offsets']} ns={c['ns']} hint={hint} out={c['out']} "
          f"valu={c['valu']} fused={c['fused']}", flush=True)
    inp = workloads.custom(f"random{i}", B=c["B"], h_q=c["h_q"], h_kv=c["h_kv"], d=c["d"], seq_lens=lens,
                           dtype=c["dtype"], seed=c["seed"])
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, c["h_kv"], dtype=c["dtype"])
    q, k, v, dl = to_device(inp)
    offs = None
    if c["offsets"]:
        # sequences in reverse order, each followed by a gap of NaN rows
        r = np.random.default_rng(c["seed"] + 1)
        gaps = r.integers(0, 50, size=c["B"])
        packed = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
        order = list(range(c["B"]))[::-1]
        start, pos = np.zeros(c["B"], dtype=np.int64), 0
        for b in order:
            start[b] = pos
            pos += int(lens[b]) + int(gaps[b])
        kp = torch.full((max(pos, 1), c["h_kv"], c["d"]), float("nan"), dtype=k.dtype, device="cuda")
        vp = torch.full_like(kp, float("nan"))
        for b in range(c["B"]):
            n = int(lens[b])
            kp[start[b]:start[b] + n] = k[packed[b]:packed[b] + n]
            vp[start[b]:start[b] + n] = v[packed[b]:packed[b] + n]
        k, v = kp, vp
        offs = torch.from_numpy(start).cuda()
    odt = torch.bfloat16 if c["out"] == "bf16" else torch.float32
    out = gqa.gqa_decode_attn_ex(q, k, v, dl, scale=float(inp.scale), n_splits=c["ns"], out_dtype=odt,
                                 s_kv_hint=hint, kv_token_offsets=offs, valu=c["valu"], fused=c["fused"])
    torch.cuda.synchronize()
    err = max_err(out.float().cpu().numpy().astype(np.float64), ref)
    tol = TOL_BF16 if c["out"] == "bf16" else TOL_F32
    print(f"[case {i}] max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("i", range(16))
def test_random_multi_token_case(i):
    """gqa_decode_attn_multi on seeded draws: S_q in [1, 64] (one or two
    column tiles per workgroup), lengths shorter than S_q included, split
    count and hint varied; against oracle.attend_multi."""
    multi_case(i, 7000, long_hint=False)


@pytest.mark.parametrize("i", range(12))
def test_random_multi_token_tile_waves_case(i):
    """The same draws with S_q >= 8 and a hint of 65536 tokens or more over
    the batch, which sends every call with at least 4 query tiles per
    sequence to the kernel with one tile per wave."""
    multi_case(i, 7500, long_hint=True)


def multi_case(i, seed0, long_hint):
    import torch

    import decode_attention_gqa_amd as gqa
    r = np.random.default_rng(seed0 + i)
    B = int(r.integers(1, 6))
    h_kv = int(r.choice([1, 2, 8]))
    n_rep = int(r.choice([1, 4, 8, 16]))
    while h_kv * n_rep > 64:
        h_kv //= 2
    h_q, d = h_kv * n_rep, int(r.choice([64, 128]))
    S_q = int(r.choice([8, 13, 16, 33, 64] if long_hint else [1, 2, 3, 5, 8, 16, 33, 64]))
    lens = r.integers(0, int(r.choice([50, 600, 4000])) + 1, size=B).astype(np.int32)
    ns = int(r.choice([0, 0, 1, 3, 40]))
    if long_hint:
        hint = max(int(lens.max()), 65536 // B + 1)
    else:
        hint = int(lens.max()) if r.random() < 0.7 else 0
    out_bf16 = bool(r.random() < 0.25)
    print(f"[multi case {seed0 + i}] B={B} S_q={S_q} h_q={h_q} h_kv={h_kv} d={d} lens={lens.tolist()} ns={ns} "
          f"hint={hint} out={'bf16' if out_bf16 else 'f32'}", flush=True)
    inp = workloads.custom(f"rmulti{seed0 + i}", B=B, h_q=h_q, h_kv=h_kv, d=d, seq_lens=lens, seed=seed0 + i)
    qm = workloads.normals(seed0 + i, 9, B * S_q * h_q * d).reshape(B, S_q, h_q, d)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, h_kv, dtype="bf16")
    _, k, v, dl = to_device(inp)
    q = torch.from_numpy(np.ascontiguousarray(qm).view(np.int16)).cuda().view(torch.bfloat16)
    out = gqa.gqa_decode_attn_multi(q, k, v, dl, scale=float(inp.scale), n_splits=ns, s_kv_hint=hint,
                                    out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    err = max_err(out.float().cpu().numpy().astype(np.float64), ref)
    tol = TOL_BF16 if out_bf16 else TOL_F32
    print(f"[multi case {seed0 + i}] max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("i", range(12))
def test_random_decode_step_case(i):
    """gqa_decode_step on seeded draws (lengths from empty to full capacity,
    padded or explicit offsets, split counts): the cache and new lengths equal
    oracle.kv_append's bit for bit, the output the oracle's attention over the
    grown cache within tolerance."""
    import torch

    import decode_attention_gqa_amd as gqa
    r = np.random.default_rng(8000 + i)
    B = int(r.integers(1, 9))
    h_kv = int(r.choice([1, 2, 8]))
    n_rep = int(r.choice([1, 2, 8, 16]))
    while h_kv * n_rep > 64:
        h_kv //= 2
    h_q, d = h_kv * n_rep, int(r.choice([64, 128]))
    cap = int(r.choice([40, 200, 2048]))
    lens = r.integers(0, cap + 1, size=B).astype(np.int32)
    lens[r.integers(0, B)] = cap if r.random() < 0.3 else lens[0]
    explicit = bool(r.random() < 0.5)
    ns = int(r.choice([0, 0, 1, 7]))
    print(f"[step case {i}] B={B} h_q={h_q} h_kv={h_kv} d={d} cap={cap} lens={lens.tolist()} "
          f"explicit={explicit} ns={ns}", flush=True)
    T = B * cap + (5 if explicit else 0)
    k0 = workloads.normals(8000 + i, 1, T * h_kv * d).reshape(T, h_kv, d)
    v0 = workloads.normals(8000 + i, 2, T * h_kv * d).reshape(T, h_kv, d)
    kn = workloads.normals(8000 + i, 3, B * h_kv * d).reshape(B, 1, h_kv, d)
    vn = workloads.normals(8000 + i, 4, B * h_kv * d).reshape(B, 1, h_kv, d)
    q = workloads.normals(8000 + i, 5, B * h_q * d).reshape(B, h_q, d)
    offs = (np.arange(B)[::-1] * cap + 5).astype(np.int64) if explicit else None
    kc_ref, vc_ref, lens_ref = oracle.kv_append(k0, v0, kn, vn, lens, cap, offs)
    ref = np.zeros((B, h_q, d))
    scale = np.float32(d ** -0.5)
    for b in range(B):
        o = int(offs[b]) if explicit else b * cap
        rows = slice(o, o + int(lens_ref[b]))
        ref[b] = oracle.attend(q[b:b + 1], kc_ref[rows], vc_ref[rows], lens_ref[b:b + 1], scale, h_kv,
                               dtype="bf16")[0]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(k0), dev(v0)
    lens_out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    out = gqa.gqa_decode_step(dev(q), dev(kn), dev(vn), kc, vc, torch.from_numpy(lens).cuda(), lens_out,
                              capacity=cap, kv_token_offsets=torch.from_numpy(offs).cuda() if explicit else None,
                              n_splits=ns, scale=float(scale))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lens_out.cpu().numpy(), lens_ref)
    np.testing.assert_array_equal(kc.view(torch.int16).cpu().numpy().view(np.uint16), kc_ref)
    np.testing.assert_array_equal(vc.view(torch.int16).cpu().numpy().view(np.uint16), vc_ref)
    err = max_err(out.float().cpu().numpy().astype(np.float64), ref)
    print(f"[step case {i}] max_abs_err={err:.3e}", flush=True)
    assert err <= TOL_F32
