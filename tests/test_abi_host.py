"""C-ABI checks that need no GPU: the library loads, exports every function
include/gqa_decode.h declares, rejects bad arguments on the host before any
HIP call, and its split heuristic and workspace size follow their contract.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")


@pytest.fixture(scope="module")
def gqa():
    import decode_attention_gqa_amd as m
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(gqa_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["gqa_decode_attn", "gqa_decode_attn_ex", "gqa_decode_attn_noalloc",
                            "gqa_decode_attn_multi", "gqa_decode_partial",
                            "gqa_decode_merge", "gqa_kv_append", "gqa_decode_step", "gqa_decode_attn_triplet",
                            "gqa_merge_triplets", "gqa_decode_pick_splits", "gqa_decode_pick_splits_d",
                            "gqa_decode_multi_splits", "gqa_decode_multi_splits_d",
                            "gqa_decode_workspace_bytes", "gqa_status_string", "gqa_last_error",
                            "gqa_decode_set_split_events"])


def test_library_exports_every_declared_symbol(gqa):
    lib = ctypes.CDLL(gqa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_constants_match_header(gqa):
    src = open(HEADER).read()
    for name in ["GQA_OK", "GQA_ERR_INVALID_ARG", "GQA_ERR_UNSUPPORTED", "GQA_ERR_WORKSPACE",
                 "GQA_ERR_HIP", "GQA_DTYPE_F32", "GQA_DTYPE_BF16", "GQA_FLAG_VALU", "GQA_FLAG_FUSED"]:
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", src)
        assert m and int(m.group(1)) == getattr(gqa, name), name
    assert int(re.search(r"#define GQA_MAX_SPLITS (\d+)", src).group(1)) == gqa.GQA_MAX_SPLITS
    assert int(re.search(r"#define GQA_MAX_QUERY_TOKENS (\d+)", src).group(1)) == gqa.GQA_MAX_QUERY_TOKENS
    assert int(re.search(r"#define GQA_SCRATCH_BYTES \((\d+)u << (\d+)\)", src).group(1)) << \
        int(re.search(r"#define GQA_SCRATCH_BYTES \((\d+)u << (\d+)\)", src).group(2)) == gqa.GQA_SCRATCH_BYTES


def test_status_strings(gqa):
    assert gqa.gqa_status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert gqa.gqa_status_string(s) not in ("ok", "unknown status")
    assert gqa.gqa_status_string(-99) == "unknown status"


# Fake, 256-byte aligned addresses: every call below must fail in the host
# checks, before any HIP call, so nothing ever dereferences them.
P = 0x10000
Q, K, V, L, O, W = (P * i for i in range(1, 7))


def call(gqa, **kw):
    a = dict(q=Q, k=K, v=V, lens=L, offs=None, out=O, B=1, h_q=64, h_kv=8, d=128, scale=0.088,
             n_splits=0, in_dt=1, out_dt=0, hint=0, ws=None, ws_bytes=0, stream=None, flags=0)
    a.update(kw)
    return gqa.lib.gqa_decode_attn_ex(a["q"], a["k"], a["v"], a["lens"], a["offs"], a["out"], a["B"],
                                      a["h_q"], a["h_kv"], a["d"], a["scale"], a["n_splits"], a["in_dt"],
                                      a["out_dt"], a["hint"], a["ws"], a["ws_bytes"], a["stream"], a["flags"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(lens=None), -1), (dict(out=None), -1),
    (dict(B=0), -1), (dict(B=-3), -1), (dict(h_q=0), -1), (dict(h_kv=0), -1), (dict(B=70000), -1),
    (dict(h_q=60, h_kv=8), -1),                       # not a multiple
    (dict(B=65535, h_q=65535 * 16, h_kv=65535), -1),  # B * h_q rows past 2^31
    (dict(h_q=24, h_kv=8), -2),                       # n_rep = 3
    (dict(h_q=256, h_kv=8), -2),                      # n_rep = 32
    (dict(d=96), -2), (dict(d=256), -2),
    (dict(scale=math.inf), -1), (dict(scale=math.nan), -1),
    (dict(in_dt=2), -2), (dict(out_dt=7), -2),
    (dict(flags=4), -1),
    (dict(n_splits=4097), -1),
    (dict(hint=-1), -1),
    (dict(q=Q + 8), -1),                              # misaligned
    (dict(out=Q), -1),                                # out aliases q
    (dict(out=K), -1),                                # out aliases k
    (dict(ws=W + 64, ws_bytes=1 << 20), -1),          # workspace not 256-byte aligned
])
def test_host_checks_reject_bad_arguments(gqa, kw, status):
    assert call(gqa, **kw) == status
    assert gqa.lib.gqa_last_error().decode() != ""


def test_base_entry_point_checks_too(gqa):
    r = gqa.lib.gqa_decode_attn(None, K, V, L, O, 1, 64, 8, 128, 0.088, 0)
    assert r == gqa.GQA_ERR_INVALID_ARG
    r = gqa.lib.gqa_decode_attn(Q, K, V, L, O, 1, 64, 8, 80, 0.088, 0)
    assert r == gqa.GQA_ERR_UNSUPPORTED


def test_no_device_is_reported_not_crashed(gqa):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(gqa) == gqa.GQA_ERR_HIP
    assert gqa.lib.gqa_decode_pick_splits(1, 8, 8192, 0) == gqa.GQA_ERR_HIP


def test_workspace_bytes(gqa):
    r = lambda x: (x + 255) // 256 * 256
    for B, h_q, d, n in [(1, 64, 128, 64), (8, 64, 128, 37), (1, 8, 64, 4), (3, 5, 64, 1)]:
        want = r(B * h_q * 8) + r(B * h_q * n * d * 4) + r(B * h_q * n * 8) + r(B * 8)
        assert gqa.gqa_decode_workspace_bytes(B, h_q, d, n) == want
        assert gqa.workspace_layout(B, h_q, d, n)["total"] == want
    assert gqa.gqa_decode_workspace_bytes(0, 64, 128, 4) == 0
    assert gqa.gqa_decode_workspace_bytes(1, 64, 128, 0) == 0


@pytest.mark.parametrize("B,h_kv,S", [(1, 8, 8192), (1, 32, 4096), (8, 8, 32768), (1, 8, 1 << 20),
                                      (1, 2, 256), (1, 8, 0), (64, 8, 100), (1, 1, 1 << 31)])
def test_split_heuristic_contract(gqa, B, h_kv, S):
    cus = 256
    n = gqa.gqa_decode_pick_splits(B, h_kv, S, cus)
    assert 1 <= n <= gqa.GQA_MAX_SPLITS
    fill = math.ceil(2 * cus / (B * h_kv))
    if S == 0 and B == 1 and cus // h_kv >= 1:
        # no length known, one sequence: one round of 8-wave workgroups, one
        # per CU (each sizes its chunk on the device)
        assert n == cus // h_kv
    elif S == 0:
        # no length known: four rounds of the resident slots (the chunk floor
        # then grows with each length on the device)
        assert n == min(4 * fill, gqa.GQA_MAX_SPLITS)
    else:
        # never more chunks than the longest sequence fills with 128 tokens
        # each (32 for a single sequence)
        assert n <= max(1, math.ceil(S / (32 if B <= 4 else 128)))
        # every CU gets work whenever the sequence is long enough: two 4-wave
        # workgroups per CU, or, for one sequence of 256 to 2048 tokens per
        # chunk, one 8-wave workgroup per CU
        eight_wave = B == 1 and n * h_kv == cus and 256 * n <= S <= 2048 * n
        if S >= 128 * fill:
            assert n * B * h_kv >= 2 * cus or eight_wave


def test_split_heuristic_values(gqa):
    # 70B GQA at B = 1, 8k to 64k tokens: one 8-wave workgroup per CU, 8 kv
    # heads x 32 chunks of 256 to 2048 tokens
    assert gqa.gqa_decode_pick_splits(1, 8, 8192, 256) == 32
    assert gqa.gqa_decode_pick_splits(1, 8, 32768, 256) == 32
    assert gqa.gqa_decode_pick_splits(1, 8, 65536, 256) == 32
    # below: 512 workgroups of 4 waves, chunks of 128 tokens
    assert gqa.gqa_decode_pick_splits(1, 8, 8191, 256) == 64
    assert gqa.gqa_decode_pick_splits(1, 8, 4096, 256) == 32
    # short: up to one workgroup per CU (32 chunks) with chunks down to 32 tokens
    assert gqa.gqa_decode_pick_splits(1, 8, 2048, 256) == 32
    assert gqa.gqa_decode_pick_splits(1, 8, 1024, 256) == 32
    assert gqa.gqa_decode_pick_splits(1, 8, 256, 256) == 8
    assert gqa.gqa_decode_pick_splits(1, 8, 40, 256) == 2
    assert gqa.gqa_decode_pick_splits(1, 32, 1024, 256) == 8
    assert gqa.gqa_decode_pick_splits_d(1, 8, 64, 512, 256) == 16
    assert gqa.gqa_decode_pick_splits(2, 8, 256, 256) == 8      # B <= 4: the same
    assert gqa.gqa_decode_pick_splits(8, 8, 256, 256) == 2      # larger batches: 128-token chunks
    # above: two rounds of the 512 resident slots
    assert gqa.gqa_decode_pick_splits(1, 8, 65537, 256) == 128
    assert gqa.gqa_decode_pick_splits(1, 8, 131072, 256) == 128
    # the 7B MHA shape (32 kv heads): 8 chunks from 2048 to 8192 tokens
    assert gqa.gqa_decode_pick_splits(1, 32, 4096, 256) == 8
    # gqa_decode_pick_splits is the 128-dimension case; 64-dimension heads
    # never take the 8-wave count
    assert gqa.gqa_decode_pick_splits_d(1, 8, 128, 8192, 256) == 32
    assert gqa.gqa_decode_pick_splits_d(1, 8, 64, 8192, 256) == 64
    assert gqa.gqa_decode_pick_splits_d(1, 8, 64, 32768, 256) == 128
    assert gqa.gqa_decode_pick_splits_d(8, 8, 64, 32768, 256) == gqa.gqa_decode_pick_splits(8, 8, 32768, 256)
    assert gqa.lib.gqa_decode_pick_splits_d(1, 8, 96, 8192, 256) == gqa.GQA_ERR_UNSUPPORTED
    # chunks of at most 4096 tokens
    assert gqa.gqa_decode_pick_splits(1, 8, 1 << 20, 256) == 256
    assert gqa.gqa_decode_pick_splits(1, 8, 1 << 22, 256) == 1024
    # several sequences: the longest over four rounds
    assert gqa.gqa_decode_pick_splits(8, 8, 32768, 256) == 32
    # no length hint: one sequence with 128-dimension heads, one round of
    # 8-wave workgroups (chunks sized on the device); otherwise four rounds
    # of the resident slots
    assert gqa.gqa_decode_pick_splits(1, 8, 0, 256) == 32
    assert gqa.gqa_decode_pick_splits(1, 32, 0, 256) == 8
    assert gqa.gqa_decode_pick_splits(1, 512, 0, 256) == 4       # more kv heads than CUs
    assert gqa.gqa_decode_pick_splits(8, 8, 0, 256) == 32
    assert gqa.gqa_decode_pick_splits_d(1, 8, 64, 0, 256) == 256


def test_multi_split_heuristic_values(gqa):
    f = lambda B, S_q, S, h_q=64, h_kv=8: gqa.lib.gqa_decode_multi_splits(B, S_q, h_q, h_kv, S, 256)
    # one query token: the single-token rule without the 8-wave count; several
    # in a single 16-column tile with 128-dimension heads: with it (d = 64:
    # without it)
    fd = lambda B, S_q, S, d: gqa.lib.gqa_decode_multi_splits_d(B, S_q, 64, 8, d, S, 256)
    assert f(1, 1, 8192) == gqa.gqa_decode_pick_splits_d(1, 8, 64, 8192, 256) == 64
    assert f(1, 2, 8192) == fd(1, 2, 8192, 128) == gqa.gqa_decode_pick_splits_d(1, 8, 128, 8192, 256) == 32
    assert f(1, 2, 32768) == 32                  # the 8-wave round up to 2048 tokens per chunk
    assert f(1, 2, 65536) == 32
    assert f(1, 2, 65537) == 128
    assert fd(1, 2, 8192, 64) == 64
    assert fd(1, 2, 8192, 96) == -2              # GQA_ERR_UNSUPPORTED
    # two tiles per workgroup, one workgroup per CU: one round for one sequence
    assert f(1, 4, 8192) == 16                   # two tiles, one per pass, 8-wave round
    assert f(1, 4, 16384) == 32                  # longer: both tiles in one pass
    assert f(1, 8, 8192) == 16                   # two passes of two tiles
    assert f(1, 4, 1 << 20) == 64                # chunks of up to 16384 tokens
    assert f(8, 4, 32768) == 16                  # a batch: the longest over four rounds
    assert f(1, 32, 4096, 32, 32) == 8           # MHA: 16 tokens per tile
    # one tile per wave (8 tiles or more over 16384 tokens, one sequence from
    # 4096; 4 or more over 65536), two workgroups per CU: one round for one
    # sequence, two for a batch
    assert f(1, 16, 4095) == 8                   # 8 tiles, too short: two tiles per workgroup
    assert f(1, 16, 4096) == 32                  # one sequence from 4096 tokens: one workgroup per CU
    assert f(1, 16, 8192) == 32
    assert f(2, 16, 4096) == 4                   # a batch below 16384 tokens: two tiles per workgroup
    assert f(1, 8, 5000, 128, 8) == 32           # 16 query heads per kv head: 8 one-token tiles
    assert fd(1, 16, 4096, 64) == 32             # d = 64
    assert f(1, 16, 16384) == 32                 # 8 tiles, one pass, up to 768 tokens a chunk: one workgroup per CU
    assert f(1, 16, 24576) == 32
    assert f(1, 16, 24577) == 64                 # longer: two workgroups per CU
    assert f(2, 16, 8192) == 32                  # B times the longest length counts
    assert f(1, 8, 65535) == 16                  # 4 tiles: two per workgroup below 65536 tokens
    assert f(1, 8, 65536) == 64
    assert f(1, 64, 65536) == 16                 # 32 tiles: two per wave, two passes, one workgroup per CU
    assert f(1, 64, 8192) == 16                  # 32 tiles x 8192 tokens = 2^18: the same
    assert f(1, 64, 8191) == 2                   # below: two tiles per workgroup, 16 passes
    assert f(1, 128, 4096) == 8                  # 64 tiles x 4096: two per wave, four passes
    assert f(1, 12, 8192) == 10                  # 6 tiles, two per workgroup, 24 units: 10 (240 workgroups), not 11
    assert f(1, 20, 2048) == 6                   # 40 units: 6 (240 workgroups), not 7 (280 > 256 slots)
    assert f(1, 20, 8192) == 32                  # 10 tiles from 4096 tokens: one per wave
    assert f(1, 24, 8192) == 32                  # 12 tiles from 8192 tokens: one per wave, two passes
    assert f(1, 24, 4096) == 32                  # 9 to 15 tiles from 4096 tokens: one per wave, two passes
    assert f(1, 24, 2048) == 5                   # below: two tiles per workgroup, 48 units
    assert f(1, 18, 8192) == 32                  # 9 tiles: one per wave
    assert f(1, 32, 4096) == 4                   # 16 tiles below 8192 tokens and 2^18: two tiles per workgroup
    assert f(1, 48, 8192) == 16                  # 24 tiles: two per wave, two passes
    assert f(1, 10, 32768) == 64                 # 5 tiles from 32768 tokens: one per wave, one pass
    assert f(1, 10, 16384) == 10                 # below: two tiles per workgroup, 24 units
    assert f(1, 8, 32768) == 16                  # 4 tiles stay on two tiles below 65536 tokens
    assert f(1, 128, 2048) == 1                  # below: 32 passes of two tiles fill the GPU
    assert f(1, 32, 16384) == 32                 # 16 tiles from 16384 tokens: one pass of two per wave
    assert f(1, 1024, 8192) == 1                 # chunked prefill: 32 passes of 16 tiles fill the GPU
    assert f(8, 16, 32768) == 16                 # a batch: the longest over two rounds
    assert f(1, 4, 8192, 64, 0) == -1
    assert f(1, 0, 8192) == -1


def test_binding_rejects_cpu_tensors(gqa):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    kv = torch.zeros(16, 2, 64, dtype=torch.bfloat16)
    lens = torch.tensor([16], dtype=torch.int32)
    with pytest.raises(ValueError):
        gqa.gqa_decode_attn_ex(q, kv, kv, lens)


def test_split_events_need_both_or_neither(gqa):
    assert gqa.lib.gqa_decode_set_split_events(0x1000, None) == gqa.GQA_ERR_INVALID_ARG
    assert gqa.lib.gqa_decode_set_split_events(None, None) == gqa.GQA_OK


def test_partial_and_merge_check_on_the_host(gqa):
    L_ = gqa.lib
    # partial needs a workspace, and the usual shape checks apply
    assert L_.gqa_decode_partial(Q, K, V, L, None, 1, 64, 8, 128, 0.088, 0, 1, 0, None, 0, None, 0) == -1
    assert L_.gqa_decode_partial(Q, K, V, L, None, 1, 64, 8, 96, 0.088, 0, 1, 0, W, 1 << 20, None, 0) == -2
    assert L_.gqa_decode_partial(Q, K, V, L, None, 1, 64, 8, 128, 0.088, 8, 1, 0, W, 16, None, 0) == -3
    assert L_.gqa_decode_partial(Q, K, V, L, None, 1, 64, 8, 128, 0.088, 8, 1, 0, W, 1 << 20, None, 2) == -1
    assert L_.gqa_decode_merge(L, None, 0, O, 1, 64, 8, 128, 0, 0, 0, None) == -1
    assert L_.gqa_decode_merge(L, W, 1 << 20, O, 1, 60, 8, 128, 8, 0, 0, None) == -1
    assert L_.gqa_decode_merge(L, W, 1 << 20, O, 1, 64, 8, 128, 8, 0, 5, None) == -2
    assert L_.gqa_decode_merge(L, W, 16, O, 1, 64, 8, 128, 8, 0, 0, None) == -3
    assert L_.gqa_decode_merge(L, W, 1 << 20, W + 256, 1, 64, 8, 128, 8, 0, 0, None) == -1   # out in workspace


def test_multi_token_checks_on_the_host(gqa):
    L_ = gqa.lib
    f = lambda **kw: L_.gqa_decode_attn_multi(
        kw.get("q", Q), K, V, L, None, kw.get("out", O), kw.get("B", 2), kw.get("S_q", 4), kw.get("h_q", 64),
        8, kw.get("d", 128), 0.088, 0, 0, 0, None, 0, None)
    assert f(S_q=0) == -1
    assert f(S_q=16385) == -1
    # B * S_q * h_q rows past 2^31 (each factor and B * passes within its own limit)
    assert L_.gqa_decode_attn_multi(Q, K, V, L, None, O, 2047, 64, 16 * 2048, 2048, 128, 0.088, 0, 0, 0,
                                    None, 0, None) == -1
    assert f(q=None) == -1
    assert f(d=80) == -2
    assert f(h_q=48) == -2
    assert f(out=Q) == -1
    assert f(B=40000, S_q=64) == -1          # B * query tiles > 65535


def test_kv_append_checks_on_the_host(gqa):
    f = lambda **kw: gqa.lib.gqa_kv_append(kw.get("kn", Q), V, K, O, None, L, kw.get("lo", None), kw.get("B", 2),
                                           kw.get("n", 1), 8, kw.get("d", 128), kw.get("dt", 1), kw.get("cap", 100), None)
    assert f(kn=None) == -1
    assert f(n=0) == -1
    assert f(cap=0) == -1
    assert f(d=96) == -2
    assert f(dt=5) == -2
    assert f(lo=L) == -1                       # lengths out overlaps lengths in
    assert f(kn=Q + 4) == -1


def test_decode_step_checks_on_the_host(gqa):
    # k_new, v_new at W and W + 0x4000 (B * h_kv * d * 2 = 4 KiB each); lengths out at W + 0x8000
    f = lambda **kw: gqa.lib.gqa_decode_step(
        Q, kw.get("kn", W), W + 0x4000, K, V, L, kw.get("lo", W + 0x8000), None, kw.get("out", O), 2, 64, 8,
        kw.get("d", 128), 0.088, 0, kw.get("dt", 1), 0, kw.get("cap", 100), None, 0, None)
    assert f(kn=None) == -1
    assert f(lo=None) == -1                    # the new lengths are required
    assert f(lo=L) == -1                       # and must not overlap the old ones
    assert f(dt=0) == -2                       # bf16 only
    assert f(cap=0) == -1
    assert f(cap=1 << 31) == -1
    assert f(d=96) == -2
    assert f(kn=W + 4) == -1                   # misaligned
    assert f(out=W) == -1                      # out overlaps k_new
    assert f(out=Q) == -1                      # out overlaps q


def test_sharded_entry_points_check_on_the_host(gqa):
    L_ = gqa.lib
    t = lambda **kw: L_.gqa_decode_attn_triplet(Q, K, V, L, None, kw.get("ml", W), kw.get("o", W + 4096), 1, 64, 8,
                                                kw.get("d", 128), 0.088, 0, 1, 0, None, 0, None, kw.get("fl", 0))
    assert t(ml=None) == -1
    assert t(d=96) == -2
    assert t(fl=2) == -1
    assert t(o=W + 8) == -1                  # misaligned
    assert t(o=W) == -1                      # ml and o overlap
    m = lambda **kw: L_.gqa_merge_triplets(kw.get("ml", W), kw.get("o", W + (1 << 16)), kw.get("p", 4),
                                           kw.get("r", 64), kw.get("d", 128), kw.get("out", O), kw.get("dt", 0), None)
    assert m(ml=None) == -1
    assert m(p=0) == -1
    assert m(d=80) == -2
    assert m(dt=3) == -2
    assert m(out=W + (1 << 16)) == -1        # out overlaps o


def test_noalloc_checks_on_the_host(gqa):
    """The no-allocation entry point runs the same argument checks as
    gqa_decode_attn_ex, and rejects a split count whose workspace would not
    fit its static scratch before any HIP call (the split count is given, so
    no device is queried)."""
    f = lambda **kw: gqa.lib.gqa_decode_attn_noalloc(
        kw.get("q", Q), K, V, L, None, kw.get("out", O), kw.get("B", 1), 64, 8, kw.get("d", 128), 0.088,
        kw.get("n", 4), 1, 0, 0, None, kw.get("fl", 0))
    assert f(q=None) == -1
    assert f(d=96) == -2
    assert f(out=Q) == -1
    assert f(fl=4) == -1
    need = lambda B, n: gqa.gqa_decode_workspace_bytes(B, 64, 128, n)
    assert need(1, 512) > gqa.GQA_SCRATCH_BYTES >= need(1, 256)
    assert f(n=512) == gqa.GQA_ERR_WORKSPACE
    assert "GQA_SCRATCH_BYTES" in gqa.lib.gqa_last_error().decode()
    assert f(n=gqa.GQA_MAX_SPLITS) == gqa.GQA_ERR_WORKSPACE
