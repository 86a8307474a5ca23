"""Sequence-sharded attention on one GPU: every shard holds a contiguous slice
of each sequence's KV (as one GPU of a sequence-parallel group would), emits
one (m, l, o) triplet per (b, h), and the gathered triplets are merged. The
result must match the oracle on the whole sequence, whether the merge runs on
the GPU or in the oracle's simulation of the pages' bidirectional fan-out."""
import math

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err

pytestmark = pytest.mark.gpu


def shard(inp, P):
    """Split each sequence into P contiguous slices; return per-shard packed
    (k, v, seq_lens)."""
    off = oracle.token_offsets(inp.seq_lens)
    shards = []
    for p in range(P):
        ks, vs, lens = [], [], []
        for b, S in enumerate(inp.seq_lens):
            lo, hi = (S * p) // P, (S * (p + 1)) // P
            ks.append(inp.k[off[b] + lo:off[b] + hi])
            vs.append(inp.v[off[b] + lo:off[b] + hi])
            lens.append(hi - lo)
        shards.append((np.concatenate(ks), np.concatenate(vs), np.array(lens, dtype=np.int32)))
    return shards


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("P", [1, 2, 4, 7])
def test_sharded_matches_whole_sequence(P):
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
    q = dev(inp.q)
    mls, os_ = [], []
    for k, v, lens in shard(inp, P):
        ml, o = gqa.gqa_decode_attn_triplet(q, dev(k), dev(v), torch.from_numpy(lens).cuda(),
                                            scale=float(inp.scale), s_kv_hint=int(lens.max()))
        mls.append(ml)
        os_.append(o)
    ml = torch.stack(mls)              # the all-gather of a multi-GPU run
    o = torch.stack(os_)
    out = gqa.gqa_merge_triplets(ml, o)
    out16 = gqa.gqa_merge_triplets(ml, o, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, 8, dtype="bf16")
    err = max_err(out.cpu().numpy().astype(np.float64), ref)
    print(f"[sharded] P={P}: max_abs_err={err:.3e}", flush=True)
    assert err <= TOL_F32
    assert max_err(out16.float().cpu().numpy().astype(np.float64), ref) <= TOL_BF16


def test_gpu_triplets_through_the_pages_fanout():
    """Feed the shards' GPU triplets (converted to natural-log units) to the
    oracle's simulation of the open-chain bidirectional fan-out: every rank
    must end with the whole-sequence result."""
    import torch

    import decode_attention_gqa_amd as gqa
    P = 5
    inp = workloads.custom("fan", B=2, h_q=16, h_kv=2, d=128, seq_lens=[3001, 4], seed=123)
    q = dev(inp.q)
    trips = []
    for k, v, lens in shard(inp, P):
        ml, o = gqa.gqa_decode_attn_triplet(q, dev(k), dev(v), torch.from_numpy(lens).cuda(),
                                            scale=float(inp.scale), s_kv_hint=int(max(lens.max(), 1)))
        torch.cuda.synchronize()
        trips.append((ml.cpu().numpy().astype(np.float64), o.cpu().numpy().astype(np.float64)))
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, 2, dtype="bf16")
    ln2 = math.log(2.0)
    for b, h in [(0, 0), (0, 9), (1, 3), (1, 15)]:
        ranks = [(t[0][b, h, 0] * ln2, t[0][b, h, 1], t[1][b, h]) for t in trips]
        outs, order = oracle.fanout(ranks)
        for r in range(P):
            assert sorted(order[r]) == list(range(P))
            err = float(np.max(np.abs(outs[r] - ref[b, h])))
            assert err <= TOL_F32, (b, h, r, err)


def test_empty_shards_give_neutral_triplets():
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.custom("empty_shard", B=3, h_q=8, h_kv=2, d=64, seq_lens=[0, 2, 40], seed=124)
    q = dev(inp.q)
    mls, os_ = [], []
    for k, v, lens in shard(inp, 4):
        if k.shape[0] == 0:                 # a shard holding no token of any sequence still needs a buffer
            k = v = np.zeros((1, 2, 64), dtype=np.uint16)
        ml, o = gqa.gqa_decode_attn_triplet(q, dev(k), dev(v), torch.from_numpy(lens).cuda(),
                                            scale=float(inp.scale))
        mls.append(ml)
        os_.append(o)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(mls[0][0, :, 0])) and torch.all(mls[0][0, :, 1] == 0)
    out = gqa.gqa_merge_triplets(torch.stack(mls), torch.stack(os_))
    torch.cuda.synchronize()
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, 2, dtype="bf16")
    assert max_err(out.cpu().numpy().astype(np.float64), ref) <= TOL_F32
    assert torch.all(out[0] == 0)


@pytest.mark.parametrize("ns", [1, 3, 20, 100])
def test_shard_triplets_through_every_merge_kernel(ns):
    """The shard's own merge writes merged triplets instead of o / l; forced
    split counts take it through each merge kernel (up to 8 chunks: several
    rows per workgroup; 9 to 32: a wave per slice; more: a workgroup per
    slice)."""
    import torch

    import decode_attention_gqa_amd as gqa
    inp = workloads.make_inputs("llama70b_gqa_b8_ragged")
    q = dev(inp.q)
    mls, os_ = [], []
    for k, v, lens in shard(inp, 2):
        ml, o = gqa.gqa_decode_attn_triplet(q, dev(k), dev(v), torch.from_numpy(lens).cuda(),
                                            scale=float(inp.scale), n_splits=ns, s_kv_hint=int(lens.max()))
        mls.append(ml)
        os_.append(o)
    out = gqa.gqa_merge_triplets(torch.stack(mls), torch.stack(os_))
    torch.cuda.synchronize()
    ref = oracle.attend(inp.q, inp.k, inp.v, inp.seq_lens, inp.scale, 8, dtype="bf16")
    err = max_err(out.cpu().numpy().astype(np.float64), ref)
    print(f"[sharded] ns={ns}: max_abs_err={err:.3e}", flush=True)
    assert err <= TOL_F32
