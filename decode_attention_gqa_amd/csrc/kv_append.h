// KV-cache append: copy the K/V rows of the new tokens into a padded cache.
//
// One workgroup per (new token i, sequence b): it moves the token's h_kv * D
// elements of K and of V (2 KiB each at 70B shapes) in 16-byte units, from
// k_new[b, i] to token row off_b + S_b + i. The new lengths go to a separate
// array, so no workgroup reads a length another one has already advanced.
#pragma once

#include "gqa_common.h"

namespace gqa {

struct AppendArgs {
  const void* k_new;          // [B, n_new, h_kv, D]
  const void* v_new;
  void* k;                    // cache rows [T, h_kv, D]
  void* v;
  const int64_t* kv_off;      // [B] first row of each sequence, or nullptr: b * capacity
  const int32_t* seq_lens;    // [B] cached lengths before the append
  int32_t* lens_out;          // [B] lengths after the append, or nullptr
  int n_new;
  int row_units;              // 16-byte units per token row: h_kv * D * elem / 16
  int64_t capacity;           // token rows per sequence
};

__global__ __launch_bounds__(256) void kv_append_rows(AppendArgs a) {
  const int i = blockIdx.x, b = blockIdx.y;
  const int old = a.seq_lens[b];
  const int64_t pos = (int64_t)old + i;
  if (pos < a.capacity) {                         // rows past the capacity are dropped
    const int64_t off = a.kv_off ? a.kv_off[b] : (int64_t)b * a.capacity;
    const int64_t src = ((int64_t)b * a.n_new + i) * a.row_units;
    const int64_t dst = (off + pos) * a.row_units;
    const uint4* ks = static_cast<const uint4*>(a.k_new) + src;
    const uint4* vs = static_cast<const uint4*>(a.v_new) + src;
    uint4* kd = static_cast<uint4*>(a.k) + dst;
    uint4* vd = static_cast<uint4*>(a.v) + dst;
    for (int u = threadIdx.x; u < a.row_units; u += 256) {
      kd[u] = ks[u];
      vd[u] = vs[u];
    }
  }
  if (a.lens_out && i == 0 && threadIdx.x == 0) {
    const int64_t nl = (int64_t)old + a.n_new;
    a.lens_out[b] = (int32_t)(nl < a.capacity ? nl : a.capacity);
  }
}

}  // namespace gqa
