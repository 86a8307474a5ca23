"""Batch order. Over more than one round of workgroups, the split kernels
start the longest sequence's chunks first for batches of 2 to 8 sequences,
and for batches of up to 64 whose longest chunk holds 1024 or more tokens:
batch slot z of the grid runs the sequence of rank z by length (ties in
batch order). Which workgroup computes which chunk changes no arithmetic,
so permuting a batch must permute the output rows bit for bit, and every
order must match the fp64 oracle. Both the packed layout (token bases summed
from the lengths) and explicit token offsets are covered, with ties and an
empty sequence, ranked batches of 8, 2 (a forced split count gives the pair
more than one round) and 12, and batches that keep the batch order (9 and
65 short sequences)."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_F32, max_err, to_device

pytestmark = pytest.mark.gpu


def report(name, err, tol):
    print(f"[order] {name}: max_abs_err={err:.3e} tol={tol:.1e}", flush=True)
    assert err <= tol, f"{name}: max abs error {err} > {tol}"


def orders(B, seed):
    rng = np.random.default_rng(seed)
    return {"reversed": np.arange(B)[::-1].copy(), "shuffled": rng.permutation(B)}


def call(q, k, v, lens, scale, hint, s_q=1, offs=None, n_splits=0):
    import torch

    import decode_attention_gqa_amd as gqa
    if s_q == 1:
        out = gqa.gqa_decode_attn_ex(q, k, v, lens, scale=scale, s_kv_hint=hint, kv_token_offsets=offs,
                                     n_splits=n_splits)
    else:
        out = gqa.gqa_decode_attn_multi(q, k, v, lens, scale=scale, s_kv_hint=hint, kv_token_offsets=offs)
    torch.cuda.synchronize()
    return out.cpu()


def packed(t, lens, perm):
    """The packed K or V rows of the sequences in the order `perm`."""
    import torch
    off = np.concatenate([[0], np.cumsum(lens)[:-1]])
    return torch.cat([t[off[i]:off[i] + lens[i]] for i in perm])


@pytest.mark.parametrize("lens,ns", [
    ([700, 3000, 0, 3000, 64, 1, 1500, 33], 0),       # ranked: ties, an empty sequence, short ones
    ([5000, 17], 100),                                # ranked: B = 2 (800 workgroups)
    ([(37 * i) % 2048 for i in range(9)], 0),         # B = 9: batch order
    ([(53 * i) % 1024 + 1 for i in range(65)], 0),    # B = 65: batch order, prefix sums over two passes
], ids=["b8_ties", "b2", "b9", "b65"])
def test_permuted_batch_permutes_output(lens, ns):
    import torch
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    inp = workloads.custom(f"order{B}", B=B, h_q=32, h_kv=4, d=128, seq_lens=lens, seed=300 + B)
    q, k, v, dl = to_device(inp)
    hint, scale = int(lens.max()), float(inp.scale)
    base = call(q, k, v, dl, scale, hint, n_splits=ns)
    report(f"B={B} batch order", max_err(base.numpy().astype(np.float64), oracle.attend(
        inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv, dtype="bf16")), TOL_F32)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)).cuda()
    for name, perm in orders(B, 310 + B).items():
        pt = torch.from_numpy(perm).cuda()
        got = call(q[pt].contiguous(), packed(k, lens, perm), packed(v, lens, perm), dl[pt].contiguous(),
                   scale, hint, n_splits=ns)
        assert torch.equal(got, base[perm]), f"B={B} {name}: packed layout, rows differ from the batch order's"
        got = call(q[pt].contiguous(), k, v, dl[pt].contiguous(), scale, hint, offs=off[pt].contiguous(),
                   n_splits=ns)
        assert torch.equal(got, base[perm]), f"B={B} {name}: explicit offsets, rows differ from the batch order's"
        print(f"[order] B={B} {name}: packed and offset calls equal the batch order's rows", flush=True)


def test_permuted_large_ranked_batch():
    """Twelve sequences of 2k-24k tokens at 70B shapes: 22 chunks of up to
    1118 tokens, so the batch is ranked; the oracle checks every kv group on
    one query head each (0, 9, ..., 63)."""
    import torch
    lens = np.random.default_rng(360).integers(2048, 24577, 12).astype(np.int32)
    B = len(lens)
    inp = workloads.custom("order12", B=B, h_q=64, h_kv=8, d=128, seq_lens=lens, seed=360)
    q, k, v, dl = to_device(inp)
    hint, scale = int(lens.max()), float(inp.scale)
    base = call(q, k, v, dl, scale, hint)
    heads = list(range(0, 64, 9))                      # rows left out stay NaN, which max_err skips
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv, dtype="bf16",
                        heads=[(b, h) for b in range(B) for h in heads])
    report(f"B={B} batch order, heads {heads}", max_err(base.numpy().astype(np.float64), ref), TOL_F32)
    for name, perm in orders(B, 370).items():
        pt = torch.from_numpy(perm).cuda()
        got = call(q[pt].contiguous(), packed(k, lens, perm), packed(v, lens, perm), dl[pt].contiguous(),
                   scale, hint)
        assert torch.equal(got, base[perm]), f"B={B} {name}: rows differ from the batch order's"
        print(f"[order] B={B} {name}: rows equal the batch order's", flush=True)


@pytest.mark.parametrize("S_q", [4, 64])
def test_permuted_multi_token_batch(S_q):
    """The multi-token kernels (two tiles per workgroup at S_q = 4, two tiles
    per wave at S_q = 64 over these lengths) rank the batch the same way."""
    import torch
    lens = np.array([3000, 800, 9000, 64, 5000, 3000], dtype=np.int32)
    B, h_q, h_kv, d = len(lens), 64, 8, 128
    inp = workloads.custom(f"order_multi{S_q}", B=B, h_q=h_q, h_kv=h_kv, d=d, seq_lens=lens, seed=320 + S_q)
    qm = workloads.normals(320 + S_q, 9, B * S_q * h_q * d).reshape(B, S_q, h_q, d)
    _, k, v, dl = to_device(inp)
    q = torch.from_numpy(qm.view(np.int16)).cuda().view(torch.bfloat16)
    hint, scale = int(lens.max()), float(inp.scale)
    base = call(q, k, v, dl, scale, hint, s_q=S_q)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, h_kv, dtype="bf16")
    report(f"S_q={S_q} B={B} batch order", max_err(base.numpy().astype(np.float64), ref), TOL_F32)
    for name, perm in orders(B, 330 + S_q).items():
        pt = torch.from_numpy(perm).cuda()
        got = call(q[pt].contiguous(), packed(k, lens, perm), packed(v, lens, perm), dl[pt].contiguous(),
                   scale, hint, s_q=S_q)
        assert torch.equal(got, base[perm]), f"S_q={S_q} {name}: rows differ from the batch order's"
        print(f"[order] S_q={S_q} B={B} {name}: rows equal the batch order's", flush=True)


def test_permuted_decode_step():
    """The decode step with the append folded in (gqa_decode_step) ranks the
    batch by its lengths before the append. A permuted batch, addressed
    through permuted token offsets into the same padded cache, gives the
    permuted output rows and lengths bit for bit, and writes the same cache
    rows (each new row to its own sequence's slot)."""
    import torch

    import decode_attention_gqa_amd as gqa
    lens = np.array([11032, 4287, 10486, 0, 21209, 32739, 5895, 7145], dtype=np.int32)
    B, h_q, h_kv, d, cap = len(lens), 64, 8, 128, 32768
    g = torch.Generator(device="cpu").manual_seed(340)
    rnd = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()   # noqa: E731
    q, kn, vn = rnd(B, h_q, d), rnd(B, h_kv, d), rnd(B, h_kv, d)
    kc, vc = rnd(B * cap, h_kv, d), rnd(B * cap, h_kv, d)
    dl = torch.from_numpy(lens).cuda()
    off = torch.arange(B, dtype=torch.int64, device="cuda") * cap

    def step(perm, kc, vc):
        pt = torch.from_numpy(perm).cuda()
        lo = torch.empty(B, dtype=torch.int32, device="cuda")
        out = gqa.gqa_decode_step(q[pt].contiguous(), kn[pt].contiguous(), vn[pt].contiguous(), kc, vc,
                                  dl[pt].contiguous(), lo, capacity=cap, kv_token_offsets=off[pt].contiguous())
        torch.cuda.synchronize()
        return out.cpu(), lo.cpu()

    kc0, vc0 = kc.clone(), vc.clone()
    base, lo0 = step(np.arange(B), kc0, vc0)
    for name, perm in orders(B, 350).items():
        kc1, vc1 = kc.clone(), vc.clone()
        got, lo1 = step(perm, kc1, vc1)
        assert torch.equal(got, base[perm]), f"decode step {name}: rows differ from the batch order's"
        assert torch.equal(lo1, lo0[perm]), f"decode step {name}: lengths differ"
        assert torch.equal(kc1, kc0) and torch.equal(vc1, vc0), f"decode step {name}: cache rows differ"
        print(f"[order] decode step B={B} {name}: rows, lengths and cache equal the batch order's", flush=True)
