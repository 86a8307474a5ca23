// Exact log-sum-exp merge of the per-chunk (m, l, o) triplets of each
// (sequence, query head) and the final division o / l.
//
// The combination follows the kernbench2 page `_attention_mesh_mlo.py`
// (receive-and-merge blocks, then o / l), applied to many chunks at once:
// with M = max_s m_s and w_s = exp(m_s - M) (exp2 here: m is in log2 units),
//   out = (sum_s w_s o_s) / (sum_s w_s l_s).
// Every chunk below n_active is non-empty, so M is finite and l > 0 unless
// the sequence is empty.
//
// One workgroup per (sequence, head). Its threads form SLOTS row slots of
// D/4 lanes (a float4 of the row each); a slot takes every SLOTS-th chunk,
// U chunks per round with all their loads issued before any is used, and
// keeps its own running (m, l, o) - the same merge rule applied
// incrementally. The slots' states are merged once more through LDS.
#pragma once

#include "gqa_common.h"

namespace gqa {

template <typename TO>
__device__ __forceinline__ void store4(TO* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float4 v) {
  // round to nearest even (the conversion instruction's rounding)
  __bf16 h[4] = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
  *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, h);
}

// exp2(m - M) for a state that may be empty (m = -inf); M is finite or -inf.
__device__ __forceinline__ float rescale(float m, float M) {
  return (m == -INFINITY) ? 0.f : fast_exp2(m - M);
}

template <int D, typename TO>
__global__ __launch_bounds__(256) void merge_splits(MergeArgs a) {
  constexpr int LPS = D / 4;                 // lanes per chunk row (float4 each)
  constexpr int SLOTS = 256 / LPS;           // chunks processed side by side
  constexpr int U = 8;                       // chunks per slot per round
  const int bh = blockIdx.x;                 // row (b, query token, head)
  const int b = bh / (a.h_q * a.s_q);
  const int tid = threadIdx.x;
  const int64_t ps = a.part_stride;
  const float2* ml = a.ws_ml + (int64_t)bh * a.row_stride;
  const float* o = a.ws_o + (int64_t)bh * a.row_stride * D;
  const int slot = tid / LPS, q = tid % LPS;

  // The loads of a round do not wait for seq_lens: indices are clamped into
  // [0, n_splits), so every load is in bounds and none sits in a branch, and
  // rows of chunks that turn out to be empty (never written by the split
  // kernel) are discarded, before any use, once seq_lens has arrived.
  float m = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float2 mv[U];
  float4 ov[U];
  auto load_round = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(base + u * SLOTS + slot, a.n_splits - 1);
      mv[u] = ml[i * ps];
      ov[u] = *reinterpret_cast<const float4*>(o + i * ps * D + 4 * q);
    }
  };
  auto merge_round = [&](int base, int n_active) {
    bool act[U];
    float mn = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      act[u] = base + u * SLOTS + slot < n_active;
      if (act[u]) mn = fmaxf(mn, mv[u].x);
    }
    const float f0 = rescale(m, mn);
    acc.x *= f0; acc.y *= f0; acc.z *= f0; acc.w *= f0;
    L *= f0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (act[u]) {
        const float f = rescale(mv[u].x, mn);     // a causal column can have empty chunks
        acc.x += f * ov[u].x;
        acc.y += f * ov[u].y;
        acc.z += f * ov[u].z;
        acc.w += f * ov[u].w;
        L += f * mv[u].y;
      }
    }
    m = mn;
  };
  load_round(0);
  __builtin_amdgcn_sched_barrier(0);           // keep the first loads ahead of the seq_lens wait
  int c, n_active = a.n_splits;
  if (a.seq_lens) chunking(a.seq_lens[b], a.n_splits, a.min_chunk, c, n_active);
  merge_round(0, n_active);
  for (int base = SLOTS * U; base < n_active; base += SLOTS * U) {
    load_round(base);
    merge_round(base, n_active);
  }

  __shared__ float sm[SLOTS], sl[SLOTS];
  __shared__ float4 sacc[SLOTS][LPS];
  sacc[slot][q] = acc;
  if (q == 0) {
    sm[slot] = m;
    sl[slot] = L;
  }
  __syncthreads();
  if (tid < LPS) {
    float M = sm[0];
#pragma unroll
    for (int k = 1; k < SLOTS; ++k) M = fmaxf(M, sm[k]);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lt = 0.f;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      const float f = rescale(sm[k], M);
      const float4 y = sacc[k][tid];
      r.x += f * y.x;
      r.y += f * y.y;
      r.z += f * y.z;
      r.w += f * y.w;
      Lt += f * sl[k];
    }
    if (a.tri_ml) {                          // merged triplet, relative to M
      if (tid == 0) a.tri_ml[bh] = make_float2(M, Lt);
      *reinterpret_cast<float4*>(a.tri_o + (int64_t)bh * D + 4 * tid) = r;
    } else {
      // Lt = 0 only when nothing was attended (empty sequence): out = 0.
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
      TO* out = static_cast<TO*>(a.out) + (int64_t)bh * D;
      store4<TO>(out + 4 * tid, make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv));
    }
  }
}

}  // namespace gqa
