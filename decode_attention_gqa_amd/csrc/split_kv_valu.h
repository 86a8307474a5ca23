// Split-KV partial attention on the vector ALUs (fp32 or bf16 q, K, V).
//
// Same decomposition and output as split_kv_mfma (one workgroup per chunk of
// a (sequence, kv head) pair, 4 waves, one (m, l, o) triplet per query head),
// with plain fp32 FMAs instead of matrix-core products:
//   scores: lane = token; each lane reads its token's K row and forms the
//           n_rep dot products against q, which sits in LDS (broadcast reads);
//   softmax: per-head wave reductions of the max; p goes to LDS;
//   P.V:    lane = D/64 consecutive dimensions; the wave walks the block's
//           tokens, reading each V row once (coalesced) and p from LDS.
// It serves the fp32 inputs and measures what the matrix cores buy for bf16.
#pragma once

#include "fused_tail.h"
#include "gqa_common.h"

namespace gqa {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int i) { return p[i]; }
  // 8 consecutive values starting at p (16-byte aligned for bf16, 32 for fp32)
  // the N (1 or 2) consecutive values at p, which is N-element aligned
  template <int N>
  static __device__ __forceinline__ void get_lane(const float* p, float (&f)[N]) {
    if constexpr (N == 2) {
      const uint2 u = load_stream8(p);
      f[0] = __uint_as_float(u.x);
      f[1] = __uint_as_float(u.y);
    } else {
      f[0] = __uint_as_float(load_stream4(p));
    }
  }
  static __device__ __forceinline__ void get8(const float* p, float (&f)[8]) {
    const uint4 a = load_stream16(p);
    const uint4 b = load_stream16(p + 4);
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
  }
};
template <>
struct Elem<__bf16> {
  static __device__ __forceinline__ float get(const __bf16* p, int i) { return (float)p[i]; }
  template <int N>
  static __device__ __forceinline__ void get_lane(const __bf16* p, float (&f)[N]) {
    if constexpr (N == 2) {
      const uint32_t w = load_stream4(p);
      f[0] = __uint_as_float(w << 16);
      f[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      const unsigned short h = __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
      f[0] = __uint_as_float((uint32_t)h << 16);
    }
  }
  static __device__ __forceinline__ void get8(const __bf16* p, float (&f)[8]) {
    const uint4 u = load_stream16(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// (wave_max: gqa_common.h.) A sum in butterfly order, so every lane holds the same bits.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <typename T, int D, int NREP>
__global__ __launch_bounds__(kThreads) void split_kv_valu(SplitArgs a) {
  constexpr int DPL = D / 64;                      // output dimensions per lane
  constexpr int TB = 64;                           // tokens per block (one per lane)
  const WgCoord wc = wg_coord();
  const int s = wc.s, g = wc.g;
  int b = wc.b;                                    // the sequence (batch slot wc.b runs it)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  int S;
  int64_t off;
  if (a.ranked)
    seq_info_ranked(a.seq_lens, a.kv_off, a.ranked, wc.b, lane, b, S, off);
  else
    seq_info(a.seq_lens, a.kv_off, b, lane, S, off);
  int c, n_active;
  chunking(S, a.n_splits, a.min_chunk, c, n_active);
  if (s >= n_active) {
    if (a.fused && n_active == 0 && s == 0) fused_empty<D, NREP>(a, g, b);
    return;
  }
  const int64_t t0 = (int64_t)s * c;
  const int ntok = (int)min<int64_t>((int64_t)S - t0, c);
  const int64_t rs = (int64_t)a.h_kv * D;
  const T* kbase = static_cast<const T*>(a.k) + ((off + t0) * a.h_kv + g) * D;
  const T* vbase = static_cast<const T*>(a.v) + ((off + t0) * a.h_kv + g) * D;

  __shared__ float sq[NREP][D];                    // the group's queries, fp32
  __shared__ float sp[kWaves][NREP][TB];           // probabilities of the current block
  {
    const T* qg = static_cast<const T*>(a.q) + ((int64_t)b * a.h_q + (int64_t)g * NREP) * D;
    for (int i = tid; i < NREP * D; i += kThreads) sq[i / D][i % D] = Elem<T>::get(qg, i);
  }
  __syncthreads();

  float m[NREP], l[NREP], o[NREP][DPL];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }

  const int nblk = ntok / TB + (ntok % TB != 0);
  for (int blk = w; blk < nblk; blk += kWaves) {
    const int nv = min(TB, ntok - blk * TB);
    const bool valid = lane < nv;
    const T* krow = kbase + ((int64_t)blk * TB + (valid ? lane : nv - 1)) * rs;
    float x[NREP];
#pragma unroll
    for (int h = 0; h < NREP; ++h) x[h] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 8) {
      float kf[8];
      Elem<T>::get8(krow + d0, kf);
#pragma unroll
      for (int h = 0; h < NREP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[h] = fmaf(sq[h][d0 + e], kf[e], x[h]);
    }
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      const float xs = valid ? x[h] * a.scale_log2 : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(xs));
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      const float p = fast_exp2(xs - mn);
      l[h] = l[h] * alpha + p;
      sp[w][h][lane] = p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] *= alpha;
    }
    // p of this wave is read back by the same wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const T* vblk = vbase + (int64_t)blk * TB * rs + lane * DPL;
    for (int t = 0; t < nv; ++t) {
      float vv[DPL];
      Elem<T>::template get_lane<DPL>(vblk + (int64_t)t * rs, vv);
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        const float p = sp[w][h][t];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[h][e] = fmaf(p, vv[e], o[h][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // Merge the waves' states in LDS and write one triplet per head.
  constexpr int OP = D + 4;
  __shared__ float sm_m[kWaves][NREP], sm_l[kWaves][NREP];
  __shared__ float sm_o[kWaves][NREP][OP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    const float lt = wave_sum(l[h]);
    if (lane == 0) {
      sm_m[w][h] = m[h];
      sm_l[w][h] = lt;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) sm_o[w][h][lane * DPL + e] = o[h][e];
  }
  __syncthreads();
  for (int idx = tid; idx < NREP * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][h]);
    float ov = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm_m[ww][h];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      L += f * sm_l[ww][h];
      ov += f * sm_o[ww][h][d];
    }
    const int64_t row = ((int64_t)b * a.h_q + g * NREP + h) * a.n_splits + s;
    a.ws_o[row * D + d] = ov;
    if (d == 0) a.ws_ml[row] = make_float2(M, L);
  }
  if (a.fused) fused_epilogue<D, NREP>(a, g, b, n_active);
}

}  // namespace gqa
