// Exact log-sum-exp merge of the per-chunk (m, l, o) triplets of each
// (sequence, query head) and the final division o / l.
//
// The combination follows the kernbench2 page `_attention_mesh_mlo.py`
// (receive-and-merge blocks, then o / l), applied to all chunks at once:
// with M = max_s m_s and w_s = exp(m_s - M) (exp2 here: m is in log2 units),
//   out = (sum_s w_s o_s) / (sum_s w_s l_s).
// Every chunk below n_active is non-empty, so M is finite and l > 0.
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

template <int D, typename TO>
__global__ __launch_bounds__(256) void merge_splits(MergeArgs a) {
  constexpr int LPS = D / 4;                 // lanes per chunk row (float4 each)
  constexpr int SLOTS = 256 / LPS;           // chunks processed side by side
  const int bh = blockIdx.x;
  const int b = bh / a.h_q;
  const int tid = threadIdx.x;
  TO* out = static_cast<TO*>(a.out) + (int64_t)bh * D;

  int64_t c;
  int n_active;
  chunking(a.seq_lens[b], a.n_splits, a.min_chunk, c, n_active);
  if (n_active == 0) {                       // empty sequence: nothing attended
    if (tid < LPS) store4<TO>(out + 4 * tid, make_float4(0.f, 0.f, 0.f, 0.f));
    return;
  }
  const float2* ml = a.ws_ml + (int64_t)bh * a.n_splits;
  const float* o = a.ws_o + (int64_t)bh * a.n_splits * D;

  __shared__ float red[4];
  __shared__ float4 sacc[SLOTS][LPS];
  __shared__ float sl[SLOTS];

  float mx = -INFINITY;
  for (int i = tid; i < n_active; i += 256) mx = fmaxf(mx, ml[i].x);
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) mx = fmaxf(mx, __shfl_xor(mx, k));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const int slot = tid / LPS, q = tid % LPS;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
  for (int i = slot; i < n_active; i += SLOTS) {
    const float2 v = ml[i];
    const float f = fast_exp2(v.x - M);
    const float4 x = *reinterpret_cast<const float4*>(o + (int64_t)i * D + 4 * q);
    acc.x += f * x.x;
    acc.y += f * x.y;
    acc.z += f * x.z;
    acc.w += f * x.w;
    L += f * v.y;
  }
  sacc[slot][q] = acc;
  if (q == 0) sl[slot] = L;
  __syncthreads();
  if (tid < LPS) {
    float4 r = sacc[0][tid];
    float Lt = sl[0];
#pragma unroll
    for (int k = 1; k < SLOTS; ++k) {
      const float4 y = sacc[k][tid];
      r.x += y.x;
      r.y += y.y;
      r.z += y.z;
      r.w += y.w;
      Lt += sl[k];
    }
    const float inv = 1.f / Lt;
    store4<TO>(out + 4 * tid, make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv));
  }
}

}  // namespace gqa
