"""Seeded synthetic inputs for single-token grouped-query decode attention.

This module is shared by the fp64 oracle's tests, the GPU parity tests and the
benchmark. It holds no attention arithmetic: it only draws random numbers,
rounds them to the storage type and lays them out.

Layouts (one query token per sequence, packed KV cache):
  q        [B, h_q, d]          query of the token being decoded
  k, v     [sum_b S_b, h_kv, d] sequence b occupies token rows
                                [off_b, off_b + S_b), off_b = sum_{j<b} S_j
  seq_lens [B] int32

bf16 tensors are returned as their raw bit patterns (uint16 arrays) so that
both sides of a parity check start from identical bits; fp32 tensors as
float32 arrays.

The shapes follow the Llama-2 decode workloads the pages discuss: the 70B
model's config.json (64 attention heads, 8 key/value heads, hidden size 8192,
so head dim 128) in the exllama discussion "Llama 2 is out", and the 7B model
(32 heads, plain multi-head attention) in the same thread and in tinygrad
issue #5244 "llama speed tracking issue".  The 1M-token case is the long
context study named in the kernbench2 `_attention_mesh_mlo.py` page (commit
message).  No page fixes a value distribution or a seed; the recipe below
is this library's own choice (standard normals, per-tensor seeds).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Elements per independently seeded chunk.  Chunk c of tensor `tid` under
# seed s is drawn from PCG64 seeded with SeedSequence([s, tid, c]), so the
# bits do not depend on the number of threads used to draw them.
CHUNK = 1 << 22

TID_Q, TID_K, TID_V, TID_LENS = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h_q: int
    h_kv: int
    d: int
    dtype: str                 # "bf16" or "f32": storage type of q, k and v
    seed: int
    s_kv: int = 0              # fixed length for every sequence ...
    s_range: tuple = ()        # ... or (lo, hi): S_b ~ U{lo..hi}, inclusive
    k_sigma: float = 1.0       # standard deviation of K entries
    n_splits: int = 0          # forced split count (0: library heuristic)
    note: str = ""

    @property
    def n_rep(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.d))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_gqa_f32", B=1, h_q=8, h_kv=2, d=64, dtype="f32", seed=0,
                 s_kv=256, n_splits=4,
                 note="fp32 bring-up case, 4 forced splits"),
        Workload("llama2_7b_mha_s4096", B=1, h_q=32, h_kv=32, d=128, dtype="bf16",
                 seed=1, s_kv=4096,
                 note="Llama-2-7B multi-head attention, one user"),
        Workload("llama70b_gqa_b1_s8192", B=1, h_q=64, h_kv=8, d=128, dtype="bf16",
                 seed=2, s_kv=8192,
                 note="Llama-70B GQA, one user, 8k context"),
        Workload("llama70b_gqa_b8_ragged", B=8, h_q=64, h_kv=8, d=128, dtype="bf16",
                 seed=3, s_range=(1024, 32768),
                 note="Llama-70B GQA, 8 users, lengths U{1024..32768}"),
        Workload("llama70b_gqa_b1_s1m", B=1, h_q=64, h_kv=8, d=128, dtype="bf16",
                 seed=4, s_kv=1 << 20, k_sigma=2.0,
                 note="Llama-70B GQA, one user, 1M context, K ~ N(0, 4)"),
    ]
}

# Order of the five workloads as listed in the project's configuration.
WORKLOAD_ORDER = list(WORKLOADS)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return bits.

    Inputs are finite normals, so the NaN path of a general converter is not
    needed and not implemented.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normals(seed: int, tid: int, n: int, sigma: float = 1.0, dtype: str = "bf16",
            threads: int | None = None) -> np.ndarray:
    """n draws of N(0, sigma^2), drawn in float32, stored as `dtype`.

    Returns uint16 bf16 bits for dtype "bf16", float32 for "f32".
    """
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    nt = threads or _threads()
    if nchunks <= 1 or nt == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def seq_lens_for(w: Workload) -> np.ndarray:
    """Per-sequence KV lengths: fixed, or integers uniform in [lo, hi]."""
    if w.s_range:
        lo, hi = w.s_range
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, TID_LENS])))
        return rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)
    return np.full(w.B, w.s_kv, dtype=np.int32)


@dataclass
class Inputs:
    w: Workload
    q: np.ndarray          # [B, h_q, d]
    k: np.ndarray          # [sum S, h_kv, d]
    v: np.ndarray          # [sum S, h_kv, d]
    seq_lens: np.ndarray   # [B] int32
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> np.float32:
        return self.w.scale

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    def kv_bytes(self) -> int:
        """Bytes of K and V the attended ranges hold (each read once)."""
        elem = 2 if self.w.dtype == "bf16" else 4
        return 2 * self.total_tokens * self.w.h_kv * self.w.d * elem


def make_inputs(w: Workload | str, seq_lens=None, threads: int | None = None) -> Inputs:
    """Draw the seeded inputs of workload `w`.

    `seq_lens` may override the lengths (used for ragged edge cases); the
    tensors are then drawn for the overridden total length.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    lens = seq_lens_for(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
    T = int(lens.astype(np.int64).sum())
    q = normals(w.seed, TID_Q, w.B * w.h_q * w.d, 1.0, w.dtype, threads)
    k = normals(w.seed, TID_K, T * w.h_kv * w.d, w.k_sigma, w.dtype, threads)
    v = normals(w.seed, TID_V, T * w.h_kv * w.d, 1.0, w.dtype, threads)
    return Inputs(
        w=w,
        q=q.reshape(w.B, w.h_q, w.d),
        k=k.reshape(T, w.h_kv, w.d),
        v=v.reshape(T, w.h_kv, w.d),
        seq_lens=lens,
    )


def custom(name: str, B: int, h_q: int, h_kv: int, d: int, seq_lens, dtype: str = "bf16",
           seed: int = 100, k_sigma: float = 1.0, n_splits: int = 0) -> Inputs:
    """Inputs for an ad-hoc shape (edge cases in tests)."""
    lens = np.asarray(seq_lens, dtype=np.int32)
    assert lens.shape == (B,)
    w = Workload(name, B=B, h_q=h_q, h_kv=h_kv, d=d, dtype=dtype, seed=seed,
                 s_kv=int(lens.max()) if B else 0, k_sigma=k_sigma, n_splits=n_splits)
    return make_inputs(w, seq_lens=lens)
