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
// Three kernels by chunks per row: merge_rows (up to 8; several rows per
// workgroup), merge_wave (9 to 32; one wave per 32-column slice) and
// merge_splits (more). Each takes a row's global max first, then sums the
// weighted chunks (the order of the additions differs between them).
//
// merge_splits: grid (row, 32-column slice of d). A workgroup's 256 threads form 32 chunk
// slots of 8 lanes (a float4 of the slice each); slot j takes chunks j,
// j + 32, ... U of them per round, with every load of a round issued before
// any is used, so up to 32 * U chunks cost one memory latency. The global
// max M is taken first (over the m values of all chunks), so each chunk's
// weight is final when its o arrives and the slots' partial sums add up
// without rescaling: in-wave shuffles, then one LDS step over the 4 waves.
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

template <int D, typename TO, int U>
__global__ __launch_bounds__(256) void merge_splits(MergeArgs a) {
  constexpr int LPS = 8;                     // lanes per chunk: a float4 each of a 32-column slice
  constexpr int SLOTS = 256 / LPS;           // chunks processed side by side
  constexpr int R = SLOTS * U;               // chunks per round
  const int bh = blockIdx.x;                 // row (b, query token, head)
  const int d0 = blockIdx.y * 4 * LPS;       // first column of the slice
  const int b = bh / (a.h_q * a.s_q);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t ps = a.part_stride;
  const float2* ml = a.ws_ml + (int64_t)bh * a.row_stride;
  const int slot = tid / LPS, q = tid % LPS;
  const float* o = a.ws_o + (int64_t)bh * a.row_stride * D + d0 + 4 * q;

  // The first round's loads do not wait for seq_lens: indices are clamped
  // into [0, n_splits), so every load is in bounds and none sits in a branch,
  // and rows of chunks that turn out to be empty (never written by the split
  // kernel) are discarded, before any use, once seq_lens has arrived.
  float2 mv[U];
  float4 ov[U];
  auto load_round = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = ml[min(base + u * SLOTS + slot, a.n_splits - 1) * ps];
#pragma unroll
    for (int u = 0; u < U; ++u)
      ov[u] = *reinterpret_cast<const float4*>(o + min(base + u * SLOTS + slot, a.n_splits - 1) * ps * D);
  };
  load_round(0);
  __builtin_amdgcn_sched_barrier(0);           // keep the first loads ahead of the seq_lens wait
  int c, n_active = a.n_splits;
  if (a.seq_lens) chunking(a.seq_lens[b], a.n_splits, a.min_chunk, c, n_active);

  // M = max over the row's chunks (a causal column can hold empty chunks, m = -inf).
  __shared__ float s_max[4];
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u * SLOTS + slot < n_active) mx = fmaxf(mx, mv[u].x);
  for (int i = R + tid; i < n_active; i += 256) mx = fmaxf(mx, ml[i * ps].x);
  mx = wave_max(mx);
  if ((tid & 63) == 0) s_max[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  auto accumulate = [&](int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * SLOTS + slot < n_active) {
        const float w = rescale(mv[u].x, M);
        acc.x += w * ov[u].x;
        acc.y += w * ov[u].y;
        acc.z += w * ov[u].z;
        acc.w += w * ov[u].w;
        L += w * mv[u].y;
      }
    }
  };
  accumulate(0);
  for (int base = R; base < n_active; base += R) {
    load_round(base);
    accumulate(base);
  }

  // Sum over the 8 slots of each wave (lane bits 3..5), then over the 4 waves.
  acc.x = sum_x32(sum_x16(sum_x8(acc.x)));
  acc.y = sum_x32(sum_x16(sum_x8(acc.y)));
  acc.z = sum_x32(sum_x16(sum_x8(acc.z)));
  acc.w = sum_x32(sum_x16(sum_x8(acc.w)));
  L = sum_x32(sum_x16(sum_x8(L)));
  __shared__ float4 s_acc[4][LPS];
  __shared__ float s_l[4];
  if ((tid & 63) < LPS) s_acc[wave][q] = acc;
  if ((tid & 63) == 0) s_l[wave] = L;
  __syncthreads();
  if (tid < LPS) {
    float4 r = s_acc[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 y = s_acc[w][tid];
      r.x += y.x;
      r.y += y.y;
      r.z += y.z;
      r.w += y.w;
    }
    const float Lt = (s_l[0] + s_l[1]) + (s_l[2] + s_l[3]);
    if (a.tri_ml) {                          // merged triplet, relative to M
      if (tid == 0 && blockIdx.y == 0) a.tri_ml[bh] = make_float2(M, Lt);
      *reinterpret_cast<float4*>(a.tri_o + (int64_t)bh * D + d0 + 4 * tid) = r;
    } else {
      // Lt = 0 only when nothing was attended (empty sequence): out = 0.
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
      TO* out = static_cast<TO*>(a.out) + (int64_t)bh * D + d0;
      store4<TO>(out + 4 * tid, make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv));
    }
  }
}

// The same merge for 9 to 32 chunks per row, one wave per SL 32-column
// slices of a row: slot j of the wave (8 lanes, SL float4s each, 32 columns
// apart) holds chunks j, j + 8, ..., U of them, all loaded at once; the max
// and the sums over the 8 slots are lane butterflies (xor 8, 16, 32), so no
// LDS step and no barrier. Grid: one workgroup of D / (32 * SL) waves per
// row. SL = 2 halves the waves of a call with many rows (multi-token calls),
// so that they fit the GPU's wave slots at once and the merge pays one
// memory latency instead of two.
template <int D, typename TO, int U, int SL = 1>
__global__ __launch_bounds__(64 * (D / (32 * SL))) void merge_wave(MergeArgs a) {
  constexpr int LPS = 8, SLOTS = 64 / LPS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPS, q = lane % LPS;
  const int wg = blockIdx.x, R = a.xcd_rep;
  const int bh = R > 0 ? wg - wg % (8 * R) + (wg % 8) * R + (wg / 8) % R : wg;   // see MergeArgs::xcd_rep
  const int b = bh / (a.h_q * a.s_q);
  const int d0 = wave * 4 * LPS * SL;
  const int64_t ps = a.part_stride;
  const float2* ml = a.ws_ml + (int64_t)bh * a.row_stride;
  const float* o = a.ws_o + (int64_t)bh * a.row_stride * D + d0 + 4 * q;
  // Clamped indices: every load is in bounds and issued before the wait for
  // seq_lens; chunks at or past n_active are selected out before any use.
  float2 mv[U];
  float4 ov[U][SL];
#pragma unroll
  for (int u = 0; u < U; ++u) mv[u] = ml[min(u * SLOTS + slot, a.n_splits - 1) * ps];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
      ov[u][sl] = *reinterpret_cast<const float4*>(o + min(u * SLOTS + slot, a.n_splits - 1) * ps * D + 32 * sl);
  __builtin_amdgcn_sched_barrier(0);
  int c, n_active = a.n_splits;
  if (a.seq_lens) chunking(a.seq_lens[b], a.n_splits, a.min_chunk, c, n_active);
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u * SLOTS + slot < n_active) M = fmaxf(M, mv[u].x);
  M = max_x32(max_x16(max_x8(M)));
  float4 acc[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) acc[sl] = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u * SLOTS + slot < n_active) {
      const float w = rescale(mv[u].x, M);   // a causal column can have empty chunks (m = -inf)
#pragma unroll
      for (int sl = 0; sl < SL; ++sl) {
        acc[sl].x += w * ov[u][sl].x;
        acc[sl].y += w * ov[u][sl].y;
        acc[sl].z += w * ov[u][sl].z;
        acc[sl].w += w * ov[u][sl].w;
      }
      L += w * mv[u].y;
    }
  }
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    acc[sl].x = sum_x32(sum_x16(sum_x8(acc[sl].x)));
    acc[sl].y = sum_x32(sum_x16(sum_x8(acc[sl].y)));
    acc[sl].z = sum_x32(sum_x16(sum_x8(acc[sl].z)));
    acc[sl].w = sum_x32(sum_x16(sum_x8(acc[sl].w)));
  }
  L = sum_x32(sum_x16(sum_x8(L)));
  if (slot != 0) return;
  if (a.tri_ml) {                            // merged triplet, relative to M
    if (q == 0 && wave == 0) a.tri_ml[bh] = make_float2(M, L);
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
      *reinterpret_cast<float4*>(a.tri_o + (int64_t)bh * D + d0 + 32 * sl + 4 * q) = acc[sl];
  } else {
    const float inv = L > 0.f ? 1.f / L : 0.f;   // L = 0 only when nothing was attended
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
      store4<TO>(static_cast<TO*>(a.out) + (int64_t)bh * D + d0 + 32 * sl + 4 * q,
                 make_float4(acc[sl].x * inv, acc[sl].y * inv, acc[sl].z * inv, acc[sl].w * inv));
  }
}

// The same merge for many rows with few chunks each (n_splits <= 8): the 32
// chunk slots of a workgroup form groups of SPR consecutive slots, one row
// per group (32 / SPR rows per workgroup), so each row's reductions run over
// lane bits 3.. of one wave and need no LDS step. Each lane holds SL float4s,
// 32 columns apart. Grid (row groups, (32 * SL)-column slices of d). Rows
// past `rows` load clamped, in-bounds data and store nothing; chunks at or
// past a row's n_active are selected out before any arithmetic touches their
// (possibly never written) workspace values.
template <int D, typename TO, int SPR, int SL = 1>
__global__ __launch_bounds__(256) void merge_rows(MergeArgs a, int rows) {
  static_assert(SPR == 1 || SPR == 2 || SPR == 4 || SPR == 8, "a row's slots lie within one wave");
  constexpr int LPS = 8;                     // lanes per chunk: SL float4s each of a slice
  constexpr int RPW = 32 / SPR;              // rows per workgroup
  const int tid = threadIdx.x;
  const int slot = tid / LPS, q = tid % LPS;
  const int c = slot % SPR;                  // this slot's chunk of its row
  const int r = blockIdx.x * RPW + slot / SPR;
  const bool live = r < rows;
  const int64_t rr = live ? r : rows - 1;
  const int d0 = blockIdx.y * 4 * LPS * SL;
  const int64_t at = rr * a.row_stride + (int64_t)min(c, a.n_splits - 1) * a.part_stride;
  const float2 mv = a.ws_ml[at];
  float4 ov[SL];
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) ov[sl] = *reinterpret_cast<const float4*>(a.ws_o + at * D + d0 + 32 * sl + 4 * q);
  int n_active = a.n_splits;
  if (a.seq_lens) {
    int cc;
    chunking(a.seq_lens[rr / (a.h_q * a.s_q)], a.n_splits, a.min_chunk, cc, n_active);
  }
  const bool act = c < n_active;
  float M = act ? mv.x : -INFINITY;
  if constexpr (SPR >= 2) M = max_x8(M);
  if constexpr (SPR >= 4) M = max_x16(M);
  if constexpr (SPR >= 8) M = max_x32(M);
  const float w = act ? rescale(mv.x, M) : 0.f;   // a causal column can have empty chunks (m = -inf)
  float4 acc[SL];                            // sums from +0, as the one-row merge does
  float L = 0.f;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    acc[sl] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (act) {
      acc[sl].x += w * ov[sl].x;
      acc[sl].y += w * ov[sl].y;
      acc[sl].z += w * ov[sl].z;
      acc[sl].w += w * ov[sl].w;
    }
  }
  if (act) L += w * mv.y;
#pragma unroll
  for (int sl = 0; sl < SL; ++sl) {
    float4& v = acc[sl];
    if constexpr (SPR >= 2) { v.x = sum_x8(v.x); v.y = sum_x8(v.y); v.z = sum_x8(v.z); v.w = sum_x8(v.w); }
    if constexpr (SPR >= 4) { v.x = sum_x16(v.x); v.y = sum_x16(v.y); v.z = sum_x16(v.z); v.w = sum_x16(v.w); }
    if constexpr (SPR >= 8) { v.x = sum_x32(v.x); v.y = sum_x32(v.y); v.z = sum_x32(v.z); v.w = sum_x32(v.w); }
  }
  if constexpr (SPR >= 2) L = sum_x8(L);
  if constexpr (SPR >= 4) L = sum_x16(L);
  if constexpr (SPR >= 8) L = sum_x32(L);
  if (!live || c != 0) return;
  if (a.tri_ml) {                            // merged triplet, relative to M
    if (q == 0 && blockIdx.y == 0) a.tri_ml[r] = make_float2(M, L);
#pragma unroll
    for (int sl = 0; sl < SL; ++sl) *reinterpret_cast<float4*>(a.tri_o + (int64_t)r * D + d0 + 32 * sl + 4 * q) = acc[sl];
  } else {
    const float inv = L > 0.f ? 1.f / L : 0.f;   // L = 0 only when nothing was attended
#pragma unroll
    for (int sl = 0; sl < SL; ++sl)
      store4<TO>(static_cast<TO*>(a.out) + (int64_t)r * D + d0 + 32 * sl + 4 * q,
                 make_float4(acc[sl].x * inv, acc[sl].y * inv, acc[sl].z * inv, acc[sl].w * inv));
  }
}

}  // namespace gqa
