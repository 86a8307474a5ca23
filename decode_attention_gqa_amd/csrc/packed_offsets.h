// Token bases of the packed cache layout, computed once per call for large
// batches: off[b] = sum_{j<b} seq_lens[j] (sequence b's first token row; the
// packed layout stores the sequences one after another in batch order).
//
// The split kernels can sum seq_lens[0..b) themselves (one wave pass per 64
// sequences), which costs nothing for small batches but is quadratic in B over
// the grid; past a batch size threshold the host runs this one-workgroup scan
// first and hands its output to the split kernel as explicit offsets.
#pragma once

#include "gqa_common.h"

namespace gqa {

// One workgroup of 1024 threads; each pass covers 4096 sequences (4 adjacent
// lengths per thread), carrying the running total into the next pass.
__global__ __launch_bounds__(1024) void packed_offsets(const int32_t* seq_lens, int B, int64_t* off) {
  constexpr int T = 1024, E = 4, WAVES = T / 64;
  __shared__ long long s_wave[WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long carry = 0;
  for (int base = 0; base < B; base += T * E) {
    int v[E];
    long long own = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = base + tid * E + e;
      v[e] = j < B ? seq_lens[j] : 0;
      own += v[e];
    }
    // inclusive scan of the per-thread sums across the wave (Hillis-Steele)
    long long x = own;
#pragma unroll
    for (int dist = 1; dist < 64; dist <<= 1) {
      const long long y = __shfl_up(x, dist, 64);
      if (lane >= dist) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    long long before = carry, total = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const long long t = s_wave[w];
      if (w < wave) before += t;
      total += t;
    }
    __syncthreads();                            // s_wave is rewritten by the next pass
    long long run = before + x - own;           // exclusive prefix at this thread's first element
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = base + tid * E + e;
      if (j < B) off[j] = run;
      run += v[e];
    }
    carry += total;
  }
}

}  // namespace gqa
