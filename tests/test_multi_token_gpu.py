"""GPU parity of multi-token decode (S_q query tokens per sequence, causal
among themselves) against oracle.attend_multi."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import TOL_BF16, TOL_F32, max_err, to_device

pytestmark = pytest.mark.gpu


def make(name, B, S_q, h_q, h_kv, d, lens, seed):
    inp = workloads.custom(name, B=B, h_q=h_q, h_kv=h_kv, d=d, seq_lens=lens, seed=seed)
    qm = workloads.normals(seed, 9, B * S_q * h_q * d).reshape(B, S_q, h_q, d)
    return inp, qm


def run(inp, qm, n_splits=0, out_dtype="f32", poison=True, hint=True):
    import torch

    import decode_attention_gqa_amd as gqa
    _, k, v, dl = to_device(inp)
    q = torch.from_numpy(qm.view(np.int16)).cuda().view(torch.bfloat16)
    w = inp.w
    B, S_q = qm.shape[0], qm.shape[1]
    if hint is True:
        s_max = int(inp.seq_lens.max())
    else:
        s_max = int(hint) if hint else 0               # False / 0: no hint; an int: that hint
    ns = gqa.multi_splits(B, S_q, w.h_q, w.h_kv, s_max, n_splits, w.d)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B * S_q, w.h_q, w.d, ns), dtype=torch.uint8, device="cuda")
    if poison:
        ws.view(torch.float32).fill_(float("nan"))
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = gqa.gqa_decode_attn_multi(q, k, v, dl, scale=float(inp.scale), n_splits=n_splits,
                                    out_dtype=odt, s_kv_hint=s_max, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), ns


def check(name, inp, qm, **kw):
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, inp.w.h_kv, dtype="bf16")
    got, ns = run(inp, qm, **kw)
    tol = TOL_BF16 if kw.get("out_dtype") == "bf16" else TOL_F32
    err = max_err(got, ref)
    print(f"[multi] {name}: n_splits={ns} max_abs_err={err:.3e}", flush=True)
    assert err <= tol, f"{name}: {err} > {tol}"
    return got, ref


@pytest.mark.parametrize("n_rep,S_q", [(8, 2), (8, 3), (8, 4), (8, 7), (4, 4), (4, 9), (2, 8), (1, 16), (1, 5), (1, 32),
                                      (16, 3), (8, 64)])
@pytest.mark.parametrize("d", [64, 128])
def test_multi_parity(n_rep, S_q, d):
    h_kv = 2
    lens = [700, 37, 1500]
    inp, qm = make(f"multi_r{n_rep}_q{S_q}_d{d}", 3, S_q, n_rep * h_kv, h_kv, d, lens, 90 + n_rep + S_q + d)
    for ns in (0, 1, 5, 64):
        check(f"n_rep={n_rep} S_q={S_q} d={d} ns={ns}", inp, qm, n_splits=ns)


def test_multi_70b_shape_and_bf16_out():
    inp, qm = make("multi70b", 2, 2, 64, 8, 128, [8192, 3000], 95)
    check("70B S_q=2", inp, qm)
    check("70B S_q=2 bf16-out", inp, qm, out_dtype="bf16")


def test_multi_short_sequences():
    """Sequences shorter than S_q (early tokens attend nothing: zeros) and
    chunks that lie entirely after some tokens' causal limit."""
    lens = [0, 1, 2, 3, 5, 33, 64]
    S_q = 4
    inp, qm = make("multi_short", len(lens), S_q, 16, 2, 128, lens, 96)
    for ns in (0, 1, 8, 40):
        got, ref = check(f"short ns={ns}", inp, qm, n_splits=ns)
        assert np.all(got[0] == 0)                           # S_b = 0
        assert np.all(got[1, :3] == 0) and np.all(got[2, :2] == 0)


def test_single_query_token_equals_one_token_path():
    import torch

    import decode_attention_gqa_amd as gqa
    inp, qm = make("multi_one", 3, 1, 64, 8, 128, [4000, 77, 1234], 97)
    got, _ = run(inp, qm)
    q, k, v, dl = to_device(inp)
    q1 = torch.from_numpy(qm[:, 0].copy().view(np.int16)).cuda().view(torch.bfloat16)
    one = gqa.gqa_decode_attn_ex(q1, k, v, dl, scale=float(inp.scale), s_kv_hint=4000)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[:, 0], one.cpu().numpy().astype(np.float64))


# A hint of LONG tokens over the batch sends calls with at least 4 query tiles
# per sequence to the kernel with one tile per wave (8 per workgroup, K/V
# blocks shared through LDS); no hint keeps them on the two-tile kernel.
LONG = 65536


@pytest.mark.parametrize("n_rep,S_q,d", [(8, 16, 128), (8, 16, 64), (8, 13, 128), (8, 64, 128), (4, 32, 128),
                                         (2, 64, 64), (1, 64, 128), (16, 8, 128), (16, 5, 64), (8, 40, 64),
                                         (8, 40, 128)])
def test_tile_waves_parity(n_rep, S_q, d):
    """One or two tiles per wave (16 or more tiles: two): ragged lengths (a
    partial last block, a sequence shorter than one block), several passes
    (S_q = 64, n_rep = 8: 32 tiles; S_q = 40: 20, a second pass of 4),
    a last tile with fewer tokens than it holds (S_q = 13, 5), split counts
    from one chunk (written out directly) to more chunks than blocks; against
    the oracle, and against the two-tile kernel (the same sums in another
    chunking: 1e-3)."""
    h_kv = 2
    lens = [700, 37, 1500]
    inp, qm = make(f"tiles_r{n_rep}_q{S_q}_d{d}", 3, S_q, n_rep * h_kv, h_kv, d, lens, 190 + n_rep + S_q + d)
    for ns in (0, 1, 5, 64):
        got, ref = check(f"tiles n_rep={n_rep} S_q={S_q} d={d} ns={ns}", inp, qm, n_splits=ns, hint=LONG)
        two, _ = run(inp, qm, n_splits=ns, hint=False)
        assert max_err(got, two) <= 1e-3


def test_tile_waves_short_sequences_and_bf16_out():
    """Sequences shorter than S_q (their early tokens attend nothing: zeros)
    and chunks past some tokens' causal limit, on the one-tile-per-wave
    kernel; bf16 output."""
    lens = [0, 1, 2, 3, 5, 33, 64]
    S_q = 16
    inp, qm = make("tiles_short", len(lens), S_q, 16, 2, 128, lens, 197)
    for ns in (0, 1, 8, 40):
        got, ref = check(f"tiles short ns={ns}", inp, qm, n_splits=ns, hint=LONG)
        assert np.all(got[0] == 0)                           # S_b = 0
        assert np.all(got[1, :15] == 0) and np.all(got[2, :14] == 0)
    check("tiles short bf16-out", inp, qm, out_dtype="bf16", hint=LONG)


@pytest.mark.parametrize("n_rep,S_q,d,S", [(8, 16, 128, 4096), (8, 16, 128, 6001), (8, 15, 128, 12000),
                                           (8, 16, 128, 24000), (16, 8, 128, 5000), (8, 16, 64, 4096)])
def test_tile_waves_one_sequence(n_rep, S_q, d, S):
    """One sequence of 8 query tiles over 8 kv heads from 4096 tokens: the
    default plan takes one tile per wave in one workgroup per CU (32 chunks
    of 128 to 750 tokens, the last one partial at 6001; S_q = 15 leaves the
    last tile half full; 16 query heads per kv head make a tile of one
    token; d = 64). Against the oracle, and against the two-tile kernel (no
    hint) within 1e-3."""
    inp, qm = make(f"tiles_one_r{n_rep}_q{S_q}_d{d}_{S}", 1, S_q, 8 * n_rep, 8, d, [S], 210 + S_q + S % 97 + d)
    got, _ = check(f"tiles one sequence n_rep={n_rep} S_q={S_q} d={d} S={S}", inp, qm)
    assert run(inp, qm)[1] == 32
    two, _ = run(inp, qm, hint=False)
    assert max_err(got, two) <= 1e-3


def test_tile_waves_70b_shape():
    """70B heads, 16 query tokens, the kernel taken by the default rule (the
    true longest length as hint, 2 x 20000 tokens)."""
    inp, qm = make("tiles70b", 2, 16, 64, 8, 128, [20000, 3000], 198)
    check("70B S_q=16", inp, qm)
    check("70B S_q=16 bf16-out", inp, qm, out_dtype="bf16")


@pytest.mark.parametrize("S_q", [16, 40])
@pytest.mark.parametrize("hint", [False, LONG])
def test_multi_offset_layout_with_nan_gaps(hint, S_q):
    """Explicit token offsets, sequences stored in reverse order with rows of
    NaN between them: a read outside a sequence's rows would show as NaN in
    the output. Both multi-token kernels (no hint: two tiles; a long hint:
    one tile per wave at S_q = 16 (8 tiles), two per wave at S_q = 40)."""
    import torch

    import decode_attention_gqa_amd as gqa
    lens = np.array([300, 0, 77, 1025, 33], dtype=np.int32)
    B, h_kv, n_rep, d = len(lens), 2, 8, 128
    inp, qm = make(f"multi_offsets_q{S_q}", B, S_q, n_rep * h_kv, h_kv, d, lens, 199 + S_q)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, h_kv, dtype="bf16")
    _, k, v, dl = to_device(inp)
    packed = np.concatenate([[0], np.cumsum(lens[:-1])]).astype(np.int64)
    gaps = [5, 40, 0, 17, 3]
    start, pos = np.zeros(B, dtype=np.int64), 0
    for b in reversed(range(B)):
        start[b] = pos
        pos += int(lens[b]) + gaps[b]
    kp = torch.full((pos, h_kv, d), float("nan"), dtype=k.dtype, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    for b in range(B):
        n = int(lens[b])
        kp[start[b]:start[b] + n] = k[packed[b]:packed[b] + n]
        vp[start[b]:start[b] + n] = v[packed[b]:packed[b] + n]
    offs = torch.from_numpy(start).cuda()
    q = torch.from_numpy(np.ascontiguousarray(qm).view(np.int16)).cuda().view(torch.bfloat16)
    for ns in (0, 1, 7):
        out = gqa.gqa_decode_attn_multi(q, kp, vp, dl, scale=float(inp.scale), n_splits=ns,
                                        s_kv_hint=int(hint) if hint else 0, kv_token_offsets=offs)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = max_err(got, ref)
        print(f"[multi] offsets S_q={S_q} hint={hint} ns={ns}: max_abs_err={err:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err <= TOL_F32


@pytest.mark.parametrize("scale", [-0.088, 0.0])
@pytest.mark.parametrize("hint", [False, LONG])
@pytest.mark.parametrize("S_q", [16, 40])
def test_multi_negative_and_zero_scale(scale, hint, S_q):
    """Both multi-token kernels with a negative and a zero scale (a long hint:
    one tile per wave at S_q = 16, two per wave at S_q = 40)."""
    import torch

    import decode_attention_gqa_amd as gqa
    lens = [700, 37, 1500]
    inp, qm = make(f"multi_scale_q{S_q}", 3, S_q, 16, 2, 128, lens, 200 + S_q)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, np.float32(scale), 2, dtype="bf16")
    _, k, v, dl = to_device(inp)
    q = torch.from_numpy(np.ascontiguousarray(qm).view(np.int16)).cuda().view(torch.bfloat16)
    out = gqa.gqa_decode_attn_multi(q, k, v, dl, scale=scale, s_kv_hint=int(hint) if hint else 0)
    torch.cuda.synchronize()
    err = max_err(out.cpu().numpy().astype(np.float64), ref)
    print(f"[multi] scale={scale} hint={hint} S_q={S_q}: max_abs_err={err:.3e}", flush=True)
    assert err <= TOL_F32


@pytest.mark.parametrize("n_rep,S_q,d", [(8, 4, 128), (8, 3, 64), (4, 8, 128), (1, 32, 128), (2, 16, 64)])
def test_two_tiles_eight_waves(n_rep, S_q, d):
    """Two tiles per workgroup on eight waves (one block each): taken with a
    length hint when chunks hold 5 to 8 blocks and the grid fits one round;
    a partial last block, a sequence shorter than S_q's causal span. Against
    the oracle, and against the four-wave form (no hint) within 1e-3. (The
    batches keep a hint above 2048 tokens: with grouped heads, two tiles over
    shorter KV run one tile per pass instead.)"""
    h_kv = 2
    for lens, ns in (([2100, 37, 1500], 12), ([4000, 1200], 16)):
        inp, qm = make(f"t2w8_r{n_rep}_q{S_q}_d{d}", len(lens), S_q, n_rep * h_kv, h_kv, d, lens,
                       210 + n_rep + S_q + d + len(lens))
        got, ref = check(f"two tiles, 8 waves n_rep={n_rep} S_q={S_q} d={d} lens={lens} ns={ns}", inp, qm,
                         n_splits=ns, hint=True)
        four, _ = run(inp, qm, n_splits=ns, hint=False)
        assert max_err(got, four) <= 1e-3


@pytest.mark.parametrize("n_rep,S_q,S", [(8, 2, 8192), (8, 2, 20000), (4, 4, 9000), (16, 1, 8192), (8, 2, 40000),
                                         (8, 2, 70000)])
def test_one_tile_eight_waves(n_rep, S_q, S):
    """One tile of several query tokens (S_q <= 16 / n_rep) over a single
    sequence with 128-dimension heads takes the single-token 8-wave round
    when its chunks hold 256 to 2048 tokens (8k to 64k at 8 kv heads; 70000:
    past it, four waves); S_q = 1 through this entry point keeps its own
    plan. Against the oracle, and against a forced split count."""
    h_kv = 8
    inp, qm = make(f"t1w8_r{n_rep}_q{S_q}_s{S}", 1, S_q, n_rep * h_kv, h_kv, 128, [S], 250 + n_rep + S_q + S % 97)
    got, ref = check(f"one tile, 8 waves n_rep={n_rep} S_q={S_q} S={S}", inp, qm, hint=True)
    forced, _ = run(inp, qm, n_splits=7, hint=True)
    assert max_err(forced, ref) <= TOL_F32


def test_two_tiles_eight_waves_with_a_hint_below_the_lengths():
    """A hint below the true lengths picks the eight-wave two-tile form for
    chunks that turn out longer than 8 blocks: its waves then take two blocks
    each, one after the other (no second register buffer)."""
    inp, qm = make("t2w8_lowhint", 2, 4, 16, 2, 128, [4000, 3100], 230)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, 2, dtype="bf16")
    for ns in (10, 12):
        got, _ = run(inp, qm, n_splits=ns, hint=2100)   # 2100 / ns tokens per chunk by the hint
        err = max_err(got, ref)
        print(f"[multi] eight-wave two tiles, hint 2100 < 4000, ns={ns}: max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32


@pytest.mark.parametrize("lens", [[1024], [4096], [8192], [6000], [2048, 2048, 2048, 2048], [512, 700, 1500, 2000],
                                  [8192, 8192]])
@pytest.mark.parametrize("S_q", [3, 4])
def test_two_tiles_one_per_pass(lens, S_q):
    """Exactly two query tiles (70B shapes, S_q = 3 or 4) over short KV (one
    sequence up to 8k tokens, or sequences up to 2048 tokens and 8k in all)
    run one tile per pass, each tile a single-tile round of its own (the
    8-wave round for one sequence); two 8k sequences keep two tiles per
    workgroup. Against the oracle, against the two-tiles-per-workgroup plan
    (no hint) within 1e-3, and with the workspace poisoned."""
    inp, qm = make(f"t2pp_q{S_q}_{len(lens)}_{lens[0]}", len(lens), S_q, 64, 8, 128, lens, 260 + S_q + len(lens) + lens[0] % 89)
    got, ref = check(f"two tiles one per pass S_q={S_q} lens={lens}", inp, qm, hint=True)
    two, _ = run(inp, qm, hint=False)
    assert max_err(got, two) <= 1e-3


@pytest.mark.parametrize("ns", [2, 5, 8, 9, 16, 17, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_merges_of_many_rows(ns, d):
    """Calls of 1024 or more (token, head) rows merge with wider lanes (a
    chunk's whole row per lane up to 8 chunks, two 32-column slices per wave
    from 9 to 32): forced split counts that pick each merge kernel and its
    chunk-count variants, against the oracle (B = 2, S_q = 48, 16 query heads:
    1536 rows; a sequence shorter than the chunk count leaves chunks empty)."""
    lens = [1500, 40]
    inp, qm = make(f"wide_merge_ns{ns}_d{d}", 2, 48, 16, 2, d, lens, 300 + ns + d)
    check(f"wide merge ns={ns} d={d}", inp, qm, n_splits=ns)
    check(f"wide merge ns={ns} d={d} bf16", inp, qm, n_splits=ns, out_dtype="bf16")


@pytest.mark.parametrize("n_rep,S_q,d", [(8, 96, 128), (8, 256, 128), (1, 128, 128), (4, 200, 64), (16, 130, 128),
                                         (8, 90, 128), (8, 90, 64), (2, 160, 64), (1, 272, 128)])
def test_many_query_tokens(n_rep, S_q, d):
    """Chunked-prefill sizes (past 64 query tokens): many passes of tiles over
    the KV, causal among the new tokens; sequences longer than S_q, one
    exactly S_q long and one shorter (its first tokens attend nothing), on
    both kernels (the length hint picks one; the long hint gives 32 or more
    tiles two per wave, with a last pass whose waves hold two tiles, one
    tile (S_q = 90: 45 tiles, 13 in the last pass) or none (130 tiles, 2))."""
    h_kv = 2
    lens = [S_q + 600, S_q, max(1, S_q // 3)]
    inp, qm = make(f"manyq_r{n_rep}_q{S_q}_d{d}", 3, S_q, n_rep * h_kv, h_kv, d, lens, 300 + n_rep + S_q + d)
    for ns, hint in ((0, True), (3, True), (0, LONG), (1, LONG)):
        got, ref = check(f"S_q={S_q} n_rep={n_rep} d={d} ns={ns} hint={hint}", inp, qm, n_splits=ns, hint=hint)
        assert np.all(got[2, :S_q - lens[2]] == 0)          # positions before the cache's start


def test_many_query_tokens_70b_bf16_out():
    """70B heads, 512 new tokens over 2048 cached ones (a prefill chunk), bf16 out."""
    inp, qm = make("manyq70b", 1, 512, 64, 8, 128, [2560], 310)
    check("70B S_q=512", inp, qm)
    check("70B S_q=512 bf16-out", inp, qm, out_dtype="bf16")


@pytest.mark.parametrize("n_rep,S_q,d,lens", [(4, 2048, 64, [2348, 2048, 900]), (8, 1536, 128, [1536])])
def test_prefill_sized(n_rep, S_q, d, lens):
    """Prefill-sized calls: thousands of new tokens, the whole prompt when
    S_b = S_q (its causal upper triangle is half the score matrix, and the
    waves skip the blocks past all of their tokens' limits), with sequences
    shorter than S_q; both kernels (the length hint picks one) and a forced
    split count."""
    h_kv = 2 if n_rep == 4 else 1
    inp, qm = make(f"prefill_r{n_rep}_q{S_q}_d{d}", len(lens), S_q, n_rep * h_kv, h_kv, d, lens,
                   400 + n_rep + S_q + d)
    ref = oracle.attend_multi(qm, inp.k, inp.v, inp.seq_lens, inp.scale, h_kv, dtype="bf16")
    for ns, hint in ((0, True), (0, LONG), (3, LONG)):
        got, used = run(inp, qm, n_splits=ns, hint=hint)
        err = max_err(got, ref)
        print(f"[multi] prefill S_q={S_q} n_rep={n_rep} d={d} lens={lens} hint={hint}: n_splits={used} "
              f"max_abs_err={err:.3e}", flush=True)
        assert err <= TOL_F32
        for b, S in enumerate(lens):
            if S < S_q:
                assert np.all(got[b, :S_q - S] == 0)     # positions before the cache's start
