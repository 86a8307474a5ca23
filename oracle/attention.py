"""fp64 CPU oracle for single-token grouped-query decode attention.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in
`__graft_entry__.py` and the `cpu_baseline` leg of `bench.py` may import this
module. The GPU library never calls it, and nothing here comes from the GPU
library: the two share no kernels, headers, helpers or constants. Only the
seeded input generator (`workloads`) feeds both.

What is computed (sources are web pages; each is cited by its title and the
part of it that defines the step):

* The result is plain softmax attention for one query token. For sequence b,
  query head h and cached position t in [0, S_b):
      s_t  = scale * <q[b, h, :], K[off_b + t, g, :]>
      out  = sum_t softmax(s)_t * V[off_b + t, g, :]
  This is what the kernbench2 page `_attention_mesh_mlo.py` computes in its
  "one-shot local partial attention" block (scores = Q.K^T, a row max, the
  exponentials of the centred scores, their sum, and P.V), followed by the
  exact merge and the final o / l step of the same function. Scale: that page
  multiplies by none; this library multiplies q.k by the caller's `scale`
  (1/sqrt(d) in every workload) before the softmax.
* Head grouping g = h // n_rep with n_rep = h_q / h_kv: contiguous groups of
  query heads share one key/value head. tinygrad issue #5244 "llama speed
  tracking issue", the `Attention.__call__` snippet, splits the query
  projection in pieces of n_rep * head_dim and the key/value projections in
  pieces of head_dim, so query heads [g*n_rep, (g+1)*n_rep) sit with kv head g.
  The exllama discussion "Llama 2 is out" gives 64 heads in 8 groups for 70B.
* The (m, l, o) triplet of a chunk of keys (running max, sum of
  exponentials, UNNORMALISED output sum_t exp(s_t - m) V_t), the merge of two
  triplets and the final division o / l follow the kernbench2 page: module
  docstring (partial attention per KV shard, bidirectional fan-out), the two
  receive-and-merge blocks, and the final normalisation. The page's
  local block builds `o` from the normalised softmax but merges and divides
  as if `o` were unnormalised; only the unnormalised reading makes the merge
  and the final division consistent, and it is the one taken here.

Everything is computed in float64 on the exact input values (bf16 bit
patterns are widened exactly). `attend` works on the whole score row at once:
no chunking, no online softmax. Parity pins for every function live in
`tests/test_oracle_*.py`.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------- decoding
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs (bf16 bits or float32)."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def token_offsets(seq_lens: np.ndarray) -> np.ndarray:
    """off_b = sum_{j<b} S_j (packed cache layout), as int64."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    off = np.zeros(lens.shape[0], dtype=np.int64)
    if lens.shape[0] > 1:
        off[1:] = np.cumsum(lens[:-1])
    return off


# ------------------------------------------------------- the plain result
def attend(q, k, v, seq_lens, scale, h_kv: int, dtype: str = "bf16",
           heads=None) -> np.ndarray:
    """Single-token GQA attention, float64.

    q [B, h_q, d], k/v [sum S, h_kv, d] in the packed layout, seq_lens [B].
    `scale` is widened from the float32 value the GPU receives.
    `heads`: optional iterable of (b, h) pairs; other rows of the result are
    left as NaN (used to check sampled outputs at full size).
    Returns out [B, h_q, d] float64; a sequence with S_b = 0 gives zeros.
    """
    q = np.asarray(q)
    B, h_q, d = q.shape
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    n_rep = h_q // h_kv
    sc = float(np.float32(scale))
    off = token_offsets(seq_lens)
    lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.full((B, h_q, d), np.nan if heads is not None else 0.0)
    want = None if heads is None else {(int(b), int(h)) for b, h in heads}
    for b in range(B):
        S = int(lens[b])
        for g in range(h_kv):
            hs = [h for h in range(g * n_rep, (g + 1) * n_rep)
                  if want is None or (b, h) in want]
            if not hs:
                continue
            if S == 0:
                out[b, hs, :] = 0.0
                continue
            Kg = widen(k[off[b]:off[b] + S, g, :], dtype)          # [S, d]
            Vg = widen(v[off[b]:off[b] + S, g, :], dtype)          # [S, d]
            Qg = widen(q[b, hs, :], dtype)                          # [r, d]
            s = sc * (Qg @ Kg.T)                                    # [r, S]
            s -= s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            out[b, hs, :] = p @ Vg
    return out


def attend_multi(q, k, v, seq_lens, scale, h_kv: int, dtype: str = "bf16") -> np.ndarray:
    """Several new query tokens per sequence, causal among themselves, fp64.

    q [B, S_q, h_q, d]; the S_q tokens are the last S_q positions of sequence
    b, whose K/V rows are already in the cache: token i sits at position
    p = S_b - S_q + i and attends cache positions [0, p]. A token with p < 0
    (fewer cached positions than query tokens) attends nothing: zeros. With
    S_q = 1 this is `attend`. This extension has no source on the pages; it is
    the plain causal-attention definition applied to the decode layout.
    Returns out [B, S_q, h_q, d].
    """
    q = np.asarray(q)
    B, S_q, h_q, d = q.shape
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    n_rep = h_q // h_kv
    sc = float(np.float32(scale))
    off = token_offsets(seq_lens)
    lens = np.asarray(seq_lens, dtype=np.int64)
    out = np.zeros((B, S_q, h_q, d))
    for b in range(B):
        S = int(lens[b])
        for g in range(h_kv):
            hs = list(range(g * n_rep, (g + 1) * n_rep))
            Kg = widen(k[off[b]:off[b] + S, g, :], dtype)
            Vg = widen(v[off[b]:off[b] + S, g, :], dtype)
            for i in range(S_q):
                p = S - S_q + i
                if p < 0:
                    continue
                Qi = widen(q[b, i, hs, :], dtype)                   # [r, d]
                s = sc * (Qi @ Kg[:p + 1].T)                          # [r, p+1]
                s -= s.max(axis=1, keepdims=True)
                e = np.exp(s)
                out[b, i, hs, :] = (e / e.sum(axis=1, keepdims=True)) @ Vg[:p + 1]
    return out


def kv_append(k_cache, v_cache, k_new, v_new, seq_lens, capacity: int, kv_offsets=None):
    """Write new tokens' K/V rows into a padded cache (a copy is returned).

    Sequence b owns token rows [off_b, off_b + capacity) with off_b =
    kv_offsets[b], or b * capacity; its cached length is seq_lens[b]. New row
    i (k_new[b, i]) goes to row off_b + seq_lens[b] + i when that position is
    below `capacity`, and is dropped otherwise. Returns (k_cache', v_cache',
    new lengths = min(seq_lens + n_new, capacity)). The step the tt-metal
    burndown calls update_cache, run before attention at every decode step.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, n_new = k_new.shape[0], k_new.shape[1]
    lens = np.asarray(seq_lens, dtype=np.int64)
    for b in range(B):
        off = int(kv_offsets[b]) if kv_offsets is not None else b * capacity
        for i in range(n_new):
            pos = int(lens[b]) + i
            if pos < capacity:
                kc[off + pos] = k_new[b, i]
                vc[off + pos] = v_new[b, i]
    return kc, vc, np.minimum(lens + n_new, capacity).astype(np.int32)


# ------------------------------------------- triplets, merge, final o / l
def scores(q_row: np.ndarray, k_rows: np.ndarray, scale) -> np.ndarray:
    """s_t = scale * <q, K_t> for one query head (float64 inputs)."""
    return float(np.float32(scale)) * (k_rows @ q_row)


def triplet(s: np.ndarray, v_rows: np.ndarray):
    """(m, l, o) of one chunk: max score, sum of exp(s - m), unnormalised
    sum_t exp(s_t - m) V_t. An empty chunk gives (-inf, 0, 0)."""
    s = np.asarray(s, dtype=np.float64)
    d = v_rows.shape[-1]
    if s.shape[0] == 0:
        return NEG_INF, 0.0, np.zeros(d)
    m = float(s.max())
    e = np.exp(s - m)
    return m, float(e.sum()), e @ v_rows


def merge(a, b):
    """Exact combination of two triplets.

    m_c = max(m, m'); each side is rescaled by exp(own m - m_c); the sums and
    the unnormalised outputs add. An empty side (m = -inf) contributes
    nothing; two empty sides stay empty.
    """
    m1, l1, o1 = a
    m2, l2, o2 = b
    if m1 == NEG_INF and m2 == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(o1)
    mc = max(m1, m2)
    f1 = math.exp(m1 - mc) if m1 != NEG_INF else 0.0
    f2 = math.exp(m2 - mc) if m2 != NEG_INF else 0.0
    return mc, l1 * f1 + l2 * f2, o1 * f1 + o2 * f2


def finalize(t) -> np.ndarray:
    """o / l; an empty triplet (l = 0) gives zeros."""
    m, l, o = t
    if l == 0.0:
        return np.zeros_like(o)
    return o / l


# --------------------------------------- the pages' multi-rank schedule
def fanout(trips):
    """Simulate the bidirectional fan-out over an open chain of ranks.

    Rank i starts with its own triplet. For step = 1 .. n-1 each rank sends
    eastward what it received from the west in the previous step (its own
    triplet at step 1) and westward what it received from the east, then
    merges the triplet arriving from the west (originating at rank i - step)
    and the one arriving from the east (rank i + step), in that order. A
    rank forwards the triplet it received, not its running merge, so every
    triplet reaches every rank exactly once (the kernbench2
    `_attention_mesh_mlo.py` page: module docstring and the fan-out loop).
    Returns the final o / l of every rank and the order in which each rank
    merged origins, so a test can check the exactly-once property.
    """
    n = len(trips)
    state = list(trips)
    order = [[i] for i in range(n)]
    east = [trips[i] if i < n - 1 else None for i in range(n)]   # to send E
    west = [trips[i] if i > 0 else None for i in range(n)]       # to send W
    east_origin = [i for i in range(n)]
    west_origin = [i for i in range(n)]
    for step in range(1, n):
        # messages in flight this step: rank i's east-bound goes to i + 1
        inbox_w = [None] * n   # arriving from the west neighbour
        inbox_e = [None] * n   # arriving from the east neighbour
        inbox_w_org = [None] * n
        inbox_e_org = [None] * n
        for i in range(n):
            if i < n - 1 and east[i] is not None:
                inbox_w[i + 1] = east[i]
                inbox_w_org[i + 1] = east_origin[i]
            if i > 0 and west[i] is not None:
                inbox_e[i - 1] = west[i]
                inbox_e_org[i - 1] = west_origin[i]
        for i in range(n):
            if inbox_w[i] is not None:
                state[i] = merge(state[i], inbox_w[i])
                order[i].append(inbox_w_org[i])
            if inbox_e[i] is not None:
                state[i] = merge(state[i], inbox_e[i])
                order[i].append(inbox_e_org[i])
        east = [inbox_w[i] if i < n - 1 else None for i in range(n)]
        west = [inbox_e[i] if i > 0 else None for i in range(n)]
        east_origin = inbox_w_org
        west_origin = inbox_e_org
    return [finalize(s) for s in state], order
