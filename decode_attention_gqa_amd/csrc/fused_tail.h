// Single-launch form of the split-KV attention (4- and 8-wave workgroups,
// THREADS = 256 or 512): the split workgroups of a
// (sequence b, kv head g) group count their arrivals on a per-group counter;
// the workgroup that arrives last merges the group's (m, l, o) triplets with
// the same rule as merge_splits and writes out = o / l for the group's n_rep
// query heads, then clears the counter.
//
// A counter word holds (call tag << 16) | arrivals. The host gives every call
// its own 48-bit tag, and an arrival that finds a different tag starts the
// count at 1, so whatever the word held before (a previous call that reset
// it, or unrelated workspace data) cannot be taken for this call's count.
// The counting loop ends: a failed swap means the word changed, to this
// call's tag (the next pass adds) or by another arrival's successful swap,
// and at most n_active workgroups arrive.
//
// Ordering: every thread waits until its own triplet stores are complete
// (accepted by the L2 of its XCD), the workgroup meets at a barrier, and one
// thread then makes them visible to the whole device with a single
// agent-scope release - one L2 write-back per workgroup instead of one per
// thread - before it counts the arrival. The thread that finds its
// workgroup last acquires at agent scope before a second barrier, and every
// thread of that workgroup acquires again before it reads the other
// workgroups' triplets. No workgroup waits for another, so the grid always
// drains.
#pragma once

#include "gqa_common.h"
#include "merge.h"

namespace gqa {

template <int D, int NREP, typename TO, int THREADS = kThreads>
__device__ __forceinline__ void merge_group(const SplitArgs& a, int b, int g, int n_active) {
  constexpr int Q4 = D / 4;                          // float4 per row
  constexpr int PAIRS = NREP * Q4;                   // (head, float4) items of the group
  constexpr int SL = PAIRS >= THREADS ? 1 : THREADS / PAIRS;   // chunk slots per item
  constexpr int U = 16;                              // chunks per slot per round
  const int tid = threadIdx.x;
  const int slot = tid / (PAIRS >= THREADS ? THREADS : PAIRS);
  const int64_t row0 = ((int64_t)b * a.h_q + (int64_t)g * NREP) * a.n_splits;   // (head 0, chunk 0)
  TO* out = static_cast<TO*>(a.out) + ((int64_t)b * a.h_q + (int64_t)g * NREP) * D;

  __shared__ float sm[SL][NREP], sl[SL][NREP];
  __shared__ float4 sacc[SL > 1 ? SL : 1][SL > 1 ? PAIRS : 1];

  for (int p = tid % (PAIRS >= THREADS ? THREADS : PAIRS); p < PAIRS; p += THREADS) {
    const int h = p / Q4, q4 = p % Q4;
    const float2* ml = a.ws_ml + row0 + (int64_t)h * a.n_splits;
    const float* o = a.ws_o + (row0 + (int64_t)h * a.n_splits) * D + 4 * q4;
    float m = -INFINITY, L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = slot; base < n_active; base += SL * U) {
      float2 mv[U];
      float4 ov[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = min(base + u * SL, n_active - 1);   // in bounds, no branch
        mv[u] = ml[i];
        ov[u] = *reinterpret_cast<const float4*>(o + (int64_t)i * D);
      }
      float mn = m;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (base + u * SL < n_active) mn = fmaxf(mn, mv[u].x);
      const float f0 = rescale(m, mn);
      acc.x *= f0; acc.y *= f0; acc.z *= f0; acc.w *= f0;
      L *= f0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (base + u * SL < n_active) {
          const float f = fast_exp2(mv[u].x - mn);
          acc.x += f * ov[u].x;
          acc.y += f * ov[u].y;
          acc.z += f * ov[u].z;
          acc.w += f * ov[u].w;
          L += f * mv[u].y;
        }
      }
      m = mn;
    }
    if constexpr (SL == 1) {
      const float inv = 1.f / L;                     // n_active >= 1 non-empty chunks: L > 0
      store4<TO>(out + (int64_t)h * D + 4 * q4, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
    } else {
      sacc[slot][p] = acc;
      if (q4 == 0) {
        sm[slot][h] = m;
        sl[slot][h] = L;
      }
    }
  }
  if constexpr (SL > 1) {
    __syncthreads();
    if (tid < PAIRS) {
      const int h = tid / Q4, q4 = tid % Q4;
      float M = sm[0][h];
#pragma unroll
      for (int k = 1; k < SL; ++k) M = fmaxf(M, sm[k][h]);
      float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
      float Lt = 0.f;
#pragma unroll
      for (int k = 0; k < SL; ++k) {
        const float f = rescale(sm[k][h], M);
        const float4 y = sacc[k][tid];
        r.x += f * y.x;
        r.y += f * y.y;
        r.z += f * y.z;
        r.w += f * y.w;
        Lt += f * sl[k][h];
      }
      const float inv = 1.f / Lt;
      store4<TO>(out + (int64_t)h * D + 4 * q4, make_float4(r.x * inv, r.y * inv, r.z * inv, r.w * inv));
    }
  }
}

// s_waitcnt immediate that waits for every outstanding vector memory
// operation of the wave (vmcnt = 0) and leaves the other counters alone.
constexpr int kWaitVmem = 0x0F70;

// Called by every thread of a split workgroup after its triplets are stored.
template <int D, int NREP, int THREADS = kThreads>
__device__ __forceinline__ void fused_epilogue(const SplitArgs& a, int g, int b, int n_active) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(kWaitVmem);             // this thread's triplet stores are in L2
  __syncthreads();
  unsigned long long* cnt = a.counters + (int64_t)b * a.h_kv + g;
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // the workgroup's stores, device-wide
    // Once a word holds this call's tag it keeps it until every chunk has
    // arrived (only the last workgroup resets it), so arrivals that see the
    // tag add 1; the first one installs (tag, 1) with a compare-and-swap
    // (a loop of compare-and-swaps for every arrival measured several times
    // slower: they contend for the one word).
    unsigned long long old = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), nw;
    while (true) {
      if ((old >> 16) == a.tag) {
        nw = __hip_atomic_fetch_add(cnt, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1ull;
        break;
      }
      const unsigned long long first = (a.tag << 16) | 1ull;
      if (__hip_atomic_compare_exchange_strong(cnt, &old, first, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        nw = first;
        break;
      }
    }
    const int last = (int)(nw & 0xFFFFull) == n_active;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // before this thread reads other workgroups' triplets
  if (a.out_bf16)
    merge_group<D, NREP, __bf16, THREADS>(a, b, g, n_active);
  else
    merge_group<D, NREP, float, THREADS>(a, b, g, n_active);
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A sequence with S_b = 0 has no split workgroup to merge: workgroup s = 0
// of each group writes zeros for the group's heads instead.
template <int D, int NREP, int THREADS = kThreads>
__device__ __forceinline__ void fused_empty(const SplitArgs& a, int g, int b) {
  constexpr int Q4 = D / 4;
  for (int p = threadIdx.x; p < NREP * Q4; p += THREADS) {
    const int64_t off = ((int64_t)b * a.h_q + (int64_t)g * NREP + p / Q4) * D + 4 * (p % Q4);
    if (a.out_bf16)
      store4<__bf16>(static_cast<__bf16*>(a.out) + off, make_float4(0.f, 0.f, 0.f, 0.f));
    else
      store4<float>(static_cast<float*>(a.out) + off, make_float4(0.f, 0.f, 0.f, 0.f));
  }
}

}  // namespace gqa
