"""Single-token grouped-query decode attention for MI355X (gfx950).

Thin Python binding of the C library `libgqa_decode.so` (C ABI declared in
include/gqa_decode.h). This module only marshals arguments: it checks torch
tensors, takes their device pointers and the current HIP stream, allocates
the output and the split workspace with torch, and calls the library. Every
step of the attention runs in the library's HIP kernels.

If the library is not built, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "gqa_decode_attn", "gqa_decode_attn_ex", "gqa_decode_attn_noalloc", "gqa_decode_attn_multi", "gqa_decode_partial",
    "gqa_decode_merge", "gqa_kv_append", "gqa_decode_step", "gqa_decode_attn_triplet", "gqa_merge_triplets",
    "GQA_MAX_QUERY_TOKENS",
    "gqa_decode_pick_splits", "gqa_decode_pick_splits_d",
    "gqa_decode_workspace_bytes", "gqa_status_string", "GQAError", "lib", "LIB_PATH",
    "GQA_OK", "GQA_ERR_INVALID_ARG", "GQA_ERR_UNSUPPORTED", "GQA_ERR_WORKSPACE", "GQA_ERR_HIP",
    "GQA_DTYPE_F32", "GQA_DTYPE_BF16", "GQA_FLAG_VALU", "GQA_FLAG_FUSED", "GQA_MAX_SPLITS",
    "workspace_layout", "multi_splits", "GQA_SCRATCH_BYTES",
]

GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_UNSUPPORTED = -2
GQA_ERR_WORKSPACE = -3
GQA_ERR_HIP = -4
GQA_DTYPE_F32 = 0
GQA_DTYPE_BF16 = 1
GQA_FLAG_VALU = 1
GQA_FLAG_FUSED = 2
GQA_MAX_SPLITS = 4096
GQA_MAX_QUERY_TOKENS = 16384
GQA_SCRATCH_BYTES = 16 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_decode.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python decode_attention_gqa_amd/build.py` "
        "(or __graft_entry__.build()). There is no non-HIP fallback.")

# torch ships its own HIP runtime (torch/lib/libamdhip64.so, soname
# libamdhip64.so.7). Import it first so the library's libamdhip64.so.7
# dependency resolves to that already-loaded copy: loading the library first
# would bring in the system runtime, torch would then load its copy too, and
# two HIP runtimes in one process do not share devices or streams.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
lib.gqa_decode_attn.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32]
lib.gqa_decode_attn.restype = _i32
lib.gqa_decode_attn_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32,
                                   _i32, _i32, _i64, _vp, _sz, _vp, _i32]
lib.gqa_decode_attn_ex.restype = _i32
lib.gqa_decode_attn_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32,
                                        _i32, _i32, _i64, _vp, _i32]
lib.gqa_decode_attn_noalloc.restype = _i32
lib.gqa_decode_attn_multi.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                      _i32, _i64, _vp, _sz, _vp]
lib.gqa_decode_attn_multi.restype = _i32
lib.gqa_decode_attn_triplet.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32,
                                        _i32, _i64, _vp, _sz, _vp, _i32]
lib.gqa_decode_attn_triplet.restype = _i32
lib.gqa_merge_triplets.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp]
lib.gqa_merge_triplets.restype = _i32
lib.gqa_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _vp]
lib.gqa_kv_append.restype = _i32
lib.gqa_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32,
                                _i32, _i32, _i64, _vp, _sz, _vp]
lib.gqa_decode_step.restype = _i32
lib.gqa_decode_partial.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i64,
                                   _vp, _sz, _vp, _i32]
lib.gqa_decode_partial.restype = _i32
lib.gqa_decode_merge.argtypes = [_vp, _vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _vp]
lib.gqa_decode_merge.restype = _i32
lib.gqa_decode_pick_splits.argtypes = [_i32, _i32, _i64, _i32]
lib.gqa_decode_pick_splits.restype = _i32
lib.gqa_decode_pick_splits_d.argtypes = [_i32, _i32, _i32, _i64, _i32]
lib.gqa_decode_pick_splits_d.restype = _i32
lib.gqa_decode_multi_splits.argtypes = [_i32, _i32, _i32, _i32, _i64, _i32]
lib.gqa_decode_multi_splits.restype = _i32
lib.gqa_decode_multi_splits_d.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _i32]
lib.gqa_decode_multi_splits_d.restype = _i32
lib.gqa_decode_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
lib.gqa_decode_workspace_bytes.restype = _sz
lib.gqa_status_string.argtypes = [_i32]
lib.gqa_status_string.restype = ctypes.c_char_p
lib.gqa_decode_set_split_events.argtypes = [_vp, _vp]
lib.gqa_decode_set_split_events.restype = _i32
lib.gqa_last_error.argtypes = []
lib.gqa_last_error.restype = ctypes.c_char_p


class GQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.gqa_last_error().decode(errors="replace")
        super().__init__(f"{where}: {gqa_status_string(status)} ({status}): {msg}")


def gqa_status_string(status: int) -> str:
    return lib.gqa_status_string(status).decode()


def gqa_decode_pick_splits(B: int, h_kv: int, s_kv_max: int = 0, num_cus: int = 0) -> int:
    """Split count the library picks for d_head = 128 (num_cus <= 0: the
    current device's)."""
    r = lib.gqa_decode_pick_splits(B, h_kv, s_kv_max, num_cus)
    if r < 0:
        raise GQAError(r, "gqa_decode_pick_splits")
    return r


def gqa_decode_pick_splits_d(B: int, h_kv: int, d_head: int, s_kv_max: int = 0, num_cus: int = 0) -> int:
    """Split count the library picks for a head size (num_cus <= 0: the
    current device's)."""
    r = lib.gqa_decode_pick_splits_d(B, h_kv, d_head, s_kv_max, num_cus)
    if r < 0:
        raise GQAError(r, "gqa_decode_pick_splits_d")
    return r


def gqa_decode_workspace_bytes(B: int, h_q: int, d_head: int, n_splits: int) -> int:
    return int(lib.gqa_decode_workspace_bytes(B, h_q, d_head, n_splits))


def workspace_layout(B: int, h_q: int, d_head: int, n_splits: int) -> dict:
    """Byte offsets of the workspace parts, as include/gqa_decode.h documents
    them: arrival counters at 0, partial outputs at `o`, (m, l) pairs at `ml`,
    packed-layout token bases at `tok`; `total` equals
    gqa_decode_workspace_bytes."""
    r = lambda x: (x + 255) // 256 * 256
    rows = B * h_q * n_splits
    o = r(B * h_q * 8)
    ml = o + r(rows * d_head * 4)
    tok = ml + r(rows * 8)
    return {"counters": 0, "o": o, "ml": ml, "tok": tok, "total": tok + r(B * 8)}


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return GQA_DTYPE_BF16
    if dt == torch.float32:
        return GQA_DTYPE_F32
    raise TypeError(f"unsupported dtype {dt}")


def gqa_decode_attn_ex(q, k_cache, v_cache, seq_lens, out=None, *, scale=None, n_splits=0,
                       out_dtype=None, s_kv_hint=0, kv_token_offsets=None, workspace=None,
                       stream=None, valu=False, fused=False):
    """Decode attention for one query token per sequence.

    q [B, h_q, d], k_cache / v_cache [T, h_kv, d] (packed by default), seq_lens [B]
    int32; all on the same GPU, contiguous, q/k/v of one dtype (bf16 or fp32).
    Returns out [B, h_q, d] (fp32 unless out_dtype=torch.bfloat16).
    The work is enqueued on `stream` (default: torch's current stream).
    """
    torch = _torch()
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, h_q, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, h_q, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, h_q, d_head] tensor of out_dtype")
    with torch.cuda.device(q.device):
        ns = n_splits if n_splits > 0 else gqa_decode_pick_splits_d(B, h_kv, d, int(s_kv_hint), 0)
        need = gqa_decode_workspace_bytes(B, h_q, d, ns) if ns <= GQA_MAX_SPLITS else 0
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_attn_ex(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            out.data_ptr(), B, h_q, h_kv, d, float(scale), int(n_splits),
            _dtype_code(q.dtype), _dtype_code(out_dtype), int(s_kv_hint),
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            ctypes.c_void_p(st.cuda_stream),
            (GQA_FLAG_VALU if valu else 0) | (GQA_FLAG_FUSED if fused else 0))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_attn_ex")
    return out


def gqa_decode_attn_noalloc(q, k_cache, v_cache, seq_lens, out, *, scale=None, n_splits=0, s_kv_hint=0,
                            kv_token_offsets=None, stream=None, valu=False, fused=False):
    """gqa_decode_attn_ex with the library's static scratch as its workspace:
    neither this function nor the library allocates (the caller gives `out`,
    [B, h_q, d] fp32 or bf16). Calls that overlap in time on one GPU race on
    the scratch."""
    torch = _torch()
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    if out.shape != (B, h_q, d) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous [B, h_q, d_head] GPU tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_attn_noalloc(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            out.data_ptr(), B, h_q, h_kv, d, float(scale), int(n_splits),
            _dtype_code(q.dtype), _dtype_code(out.dtype), int(s_kv_hint), ctypes.c_void_p(st.cuda_stream),
            (GQA_FLAG_VALU if valu else 0) | (GQA_FLAG_FUSED if fused else 0))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_attn_noalloc")
    return out


def _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets):
    """q is [B, h_q, d] or [B, S_q, h_q, d]."""
    torch = _torch()
    B, d = q.shape[0], q.shape[-1]
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if k_cache.dim() != 3 or k_cache.shape != v_cache.shape or k_cache.shape[2] != d:
        raise ValueError("k_cache and v_cache must be [T, h_kv, d_head]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if kv_token_offsets is not None and (kv_token_offsets.dtype != torch.int64
                                         or kv_token_offsets.shape != (B,) or not kv_token_offsets.is_cuda):
        raise ValueError("kv_token_offsets must be an int64 [B] GPU tensor")


def multi_splits(B: int, S_q: int, h_q: int, h_kv: int, s_kv_hint: int = 0, n_splits: int = 0,
                 d_head: int = 128) -> int:
    """Split count gqa_decode_attn_multi uses (for sizing its workspace)."""
    if n_splits > 0:
        return n_splits
    r = lib.gqa_decode_multi_splits_d(B, S_q, h_q, h_kv, d_head, int(s_kv_hint), 0)
    if r < 1:
        raise GQAError(r, "gqa_decode_multi_splits_d")
    return r


def gqa_decode_attn_multi(q, k_cache, v_cache, seq_lens, out=None, *, scale=None, n_splits=0,
                          out_dtype=None, s_kv_hint=0, kv_token_offsets=None, workspace=None,
                          stream=None):
    """S_q new query tokens per sequence, causal among themselves.

    q [B, S_q, h_q, d] bf16; k_cache / v_cache [T, h_kv, d] bf16 holding the
    new tokens' K/V already; seq_lens [B] int32 counts them. Token i of
    sequence b attends positions [0, S_b - S_q + i]. Returns [B, S_q, h_q, d].
    """
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, S_q, h_q, d_head]")
    B, S_q, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    if q.dtype != torch.bfloat16:
        raise TypeError("gqa_decode_attn_multi takes bf16 q/k/v")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, S_q, h_q, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, S_q, h_q, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, S_q, h_q, d_head] tensor of out_dtype")
    with torch.cuda.device(q.device):
        if workspace is None:
            ns = multi_splits(B, S_q, h_q, h_kv, int(s_kv_hint), n_splits, d)
            workspace = torch.empty(gqa_decode_workspace_bytes(B * S_q, h_q, d, ns), dtype=torch.uint8,
                                    device=q.device)
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_attn_multi(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            out.data_ptr(), B, S_q, h_q, h_kv, d, float(scale), int(n_splits), _dtype_code(out_dtype),
            int(s_kv_hint), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(st.cuda_stream))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_attn_multi")
    return out


def gqa_decode_attn_triplet(q, k_cache, v_cache, seq_lens, *, scale=None, n_splits=0, s_kv_hint=0,
                            kv_token_offsets=None, workspace=None, stream=None):
    """This shard's (m, l, o) per (b, h) over its own KV: returns
    (ml [B, h_q, 2] fp32, o [B, h_q, d] fp32), m and the exponentials in log2
    units (see include/gqa_decode.h)."""
    torch = _torch()
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ml = torch.empty((B, h_q, 2), dtype=torch.float32, device=q.device)
    o = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        ns = n_splits if n_splits > 0 else gqa_decode_pick_splits_d(B, h_kv, d, int(s_kv_hint), 0)
        if workspace is None:
            workspace = torch.empty(gqa_decode_workspace_bytes(B, h_q, d, ns), dtype=torch.uint8, device=q.device)
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_attn_triplet(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            ml.data_ptr(), o.data_ptr(), B, h_q, h_kv, d, float(scale), int(n_splits),
            _dtype_code(q.dtype), int(s_kv_hint), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), ctypes.c_void_p(st.cuda_stream), 0)
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_attn_triplet")
    return ml, o


def gqa_merge_triplets(ml, o, out_dtype=None, stream=None):
    """Merge triplet sets stacked part-major: ml [P, ..., 2], o [P, ..., d]
    (the leading dims after P are the rows). Returns out [..., d]."""
    torch = _torch()
    P, d = ml.shape[0], o.shape[-1]
    rows = ml[0].numel() // 2
    if o.shape[0] != P or o[0].numel() != rows * d or ml.dtype != torch.float32 or o.dtype != torch.float32:
        raise ValueError("ml must be [P, rows..., 2] and o [P, rows..., d], fp32")
    if not ml.is_contiguous() or not o.is_contiguous():
        raise ValueError("ml and o must be contiguous")
    out_dtype = out_dtype or torch.float32
    out = torch.empty(o.shape[1:], dtype=out_dtype, device=o.device)
    with torch.cuda.device(o.device):
        st = stream if stream is not None else torch.cuda.current_stream(o.device)
        r = lib.gqa_merge_triplets(ml.data_ptr(), o.data_ptr(), P, rows, d, out.data_ptr(),
                                   _dtype_code(out_dtype), ctypes.c_void_p(st.cuda_stream))
    if r != GQA_OK:
        raise GQAError(r, "gqa_merge_triplets")
    return out


def gqa_kv_append(k_new, v_new, k_cache, v_cache, seq_lens, *, capacity, seq_lens_out=None,
                  kv_token_offsets=None, stream=None):
    """Write new tokens' K/V rows ([B, n_new, h_kv, d]) into a padded cache at
    positions seq_lens[b] + i; optionally write the new lengths to
    seq_lens_out (a different int32 [B] tensor)."""
    torch = _torch()
    B, n_new, h_kv, d = k_new.shape
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if v_new.shape != k_new.shape or k_cache.dtype != k_new.dtype or v_cache.dtype != k_new.dtype:
        raise ValueError("k_new/v_new shapes or dtypes do not match the cache")
    if k_cache.shape[1:] != (h_kv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [T, h_kv, d_head]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    with torch.cuda.device(k_new.device):
        st = stream if stream is not None else torch.cuda.current_stream(k_new.device)
        r = lib.gqa_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                              kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
                              seq_lens.data_ptr(),
                              seq_lens_out.data_ptr() if seq_lens_out is not None else None,
                              B, n_new, h_kv, d, _dtype_code(k_new.dtype), int(capacity),
                              ctypes.c_void_p(st.cuda_stream))
    if r != GQA_OK:
        raise GQAError(r, "gqa_kv_append")


def gqa_decode_step(q, k_new, v_new, k_cache, v_cache, seq_lens, seq_lens_out, out=None, *, capacity,
                    scale=None, n_splits=0, out_dtype=None, kv_token_offsets=None, workspace=None, stream=None):
    """One decode step: append each sequence's new token (k_new / v_new
    [B, h_kv, d] or [B, 1, h_kv, d] bf16) to the padded cache at position
    seq_lens[b] (dropped at capacity), write min(seq_lens + 1, capacity) to
    seq_lens_out, and attend q [B, h_q, d] over the grown sequences.
    Returns out [B, h_q, d] (fp32 unless out_dtype=torch.bfloat16)."""
    torch = _torch()
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("seq_lens_out", seq_lens_out)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if k_new.numel() != B * h_kv * d or v_new.shape != k_new.shape or k_new.dtype != q.dtype \
            or v_new.dtype != q.dtype:
        raise ValueError("k_new / v_new must be [B, h_kv, d_head] (or [B, 1, h_kv, d_head]) of q's dtype")
    if seq_lens_out.dtype != torch.int32 or seq_lens_out.shape != (B,):
        raise ValueError("seq_lens_out must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty((B, h_q, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, h_q, d) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, h_q, d_head] tensor of out_dtype")
    with torch.cuda.device(q.device):
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_step(
            q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            seq_lens.data_ptr(), seq_lens_out.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            out.data_ptr(), B, h_q, h_kv, d, float(scale), int(n_splits),
            _dtype_code(q.dtype), _dtype_code(out_dtype), int(capacity),
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() * workspace.element_size() if workspace is not None else 0,
            ctypes.c_void_p(st.cuda_stream))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_step")
    return out


def gqa_decode_partial(q, k_cache, v_cache, seq_lens, workspace, *, scale=None, n_splits=0,
                       s_kv_hint=0, kv_token_offsets=None, stream=None, valu=False):
    """Split kernel only: writes the per-chunk (m, l, o) triplets into
    `workspace` (a uint8 GPU tensor, see gqa_decode_workspace_bytes)."""
    torch = _torch()
    _check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        r = lib.gqa_decode_partial(
            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(),
            kv_token_offsets.data_ptr() if kv_token_offsets is not None else None,
            B, h_q, h_kv, d, float(scale), int(n_splits), _dtype_code(q.dtype), int(s_kv_hint),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(st.cuda_stream), GQA_FLAG_VALU if valu else 0)
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_partial")


def gqa_decode_merge(seq_lens, workspace, out, *, h_kv, n_splits=0, s_kv_hint=0, stream=None):
    """Merge the triplets a gqa_decode_partial call (same seq_lens, shapes,
    n_splits and s_kv_hint) wrote, into out [B, h_q, d] (fp32 or bf16)."""
    torch = _torch()
    B, h_q, d = out.shape
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_cuda:
        raise ValueError("seq_lens must be an int32 [B] GPU tensor")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    with torch.cuda.device(out.device):
        st = stream if stream is not None else torch.cuda.current_stream(out.device)
        r = lib.gqa_decode_merge(seq_lens.data_ptr(), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), out.data_ptr(),
                                 B, h_q, h_kv, d, int(n_splits), int(s_kv_hint),
                                 _dtype_code(out.dtype), ctypes.c_void_p(st.cuda_stream))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_merge")
    return out


def gqa_decode_attn(q, k_cache, v_cache, seq_lens, out=None, *, scale=None, n_splits=0):
    """The base entry point: bf16 inputs, packed cache, fp32 out, null stream,
    library-owned workspace (same names and arguments as the C function)."""
    torch = _torch()
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    if q.dtype != torch.bfloat16:
        raise TypeError("gqa_decode_attn takes bf16 q/k/v; use gqa_decode_attn_ex for fp32")
    if out is None:
        out = torch.empty((B, h_q, d), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(q.device):
        r = lib.gqa_decode_attn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                seq_lens.data_ptr(), out.data_ptr(), B, h_q, h_kv, d,
                                float(scale), int(n_splits))
    if r != GQA_OK:
        raise GQAError(r, "gqa_decode_attn")
    return out
