// Shared device-side definitions of the split-KV decode attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kWaves = 4;            // waves per workgroup of the split kernels
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Arguments of the split kernels (one struct so launches stay readable).
struct SplitArgs {
  const void* q;              // [B, h_q, D]
  const void* k;              // [T, h_kv, D]
  const void* v;              // [T, h_kv, D]
  const int32_t* seq_lens;    // [B]
  const int64_t* kv_off;      // [B] or nullptr (packed)
  float* ws_o;                // [B, h_q, n_splits, D] unnormalised partial outputs
  float2* ws_ml;              // [B, h_q, n_splits] (m, l), m in log2 units
  int h_q;
  int h_kv;
  int n_splits;
  int min_chunk;              // lower bound of the chunk length (tokens); 0: chunk_floor's rule
  float scale_log2;           // scale * log2(e): scores are kept in log2 units
  // single-launch form only (see fused_tail.h)
  int fused;                  // 1: the last workgroup of each group merges and writes out
  int out_bf16;               // out is bf16 (else fp32)
  void* out;                  // [B, h_q, D]
  unsigned long long* counters;   // [B * h_kv] arrival counters: (call tag << 16) | arrivals
  unsigned long long tag;     // this call's tag (48 bits), see fused_tail.h
  // several query tokens per sequence (matrix-core kernel only)
  int s_q;                    // query tokens per sequence (1: single-token decode)
  int tpt;                    // query tokens per 16-column tile: min(s_q, 16 / n_rep)
  int qtiles;                 // tiles per sequence: ceil(s_q / tpt)
  int passes;                 // tile groups per sequence (qtiles / tiles per workgroup); grid z = B * passes
  // decode step with the new token appended on the way (APPEND kernels only)
  const void* k_new;          // [B, h_kv, D] the new token's K and V rows
  const void* v_new;
  int32_t* lens_out;          // [B] lengths after the append: min(S_b + 1, capacity)
  int capacity;               // token rows per sequence; rows start at kv_off[b] or b * capacity
  // one chunk per sequence (n_splits = 1): write out = o / l directly, no merge kernel
  int direct;
  // tile-per-wave kernel: the grid is (h_kv, n_splits, B * passes), kv heads
  // fastest (split_grid_heads_fastest), instead of split_grid's order
  int heads_fastest;
  // B (2 to kRankedMaxBatch sequences): the grid's batch slot z runs the
  // sequence of rank z by length, longest first (seq_info_ranked); 0: slot z
  // runs sequence z
  int ranked;
};

struct MergeArgs {
  int s_q;                    // query tokens per sequence: rows are (b, token, head)
  const int32_t* seq_lens;    // nullptr: every one of the n_splits parts is present
  const float* ws_o;          // part i of row r: o at ((r * row_stride + i * part_stride) * D)
  const float2* ws_ml;        //                  (m, l) at r * row_stride + i * part_stride
  void* out;                  // [rows, D] fp32 or bf16 (o / l), unless tri_ml is set
  int h_q;
  int n_splits;
  int min_chunk;
  int64_t row_stride, part_stride;
  float2* tri_ml;             // if set: write the merged (m, l) per row here ...
  float* tri_o;               // ... and the merged unnormalised o [rows, D], instead of out
  // merge_wave only. 0: workgroup L merges row L. R > 0 (8 kv heads, R query
  // heads per group, split kernel launched kv heads fastest so that kv head g
  // ran on XCD g): within each block of 8R rows, workgroup L merges row
  // (L mod 8) * R + (L / 8) mod R, a head of group L mod 8, on the XCD that
  // wrote its triplets.
  int xcd_rep;
};

// Chunk length and number of non-empty chunks of a sequence of S tokens.
// The split kernels and the merge kernel both use this, so they agree on
// which chunks exist: chunk s covers tokens [s*c, min(S, (s+1)*c)).
// 32-bit unsigned arithmetic suffices: S < 2^31 and n_splits <= 4096, so
// S + c - 1 < 2^32.
// The shortest chunk: min_chunk tokens, or, for a call planned without the
// lengths (min_chunk = 0), a floor that grows with the sequence: S / 32
// rounded up to whole 32-token blocks, from 32 to 128 tokens. A short
// sequence then still spreads over up to 32 one-block chunks, a longer one
// gets chunks of at least one block per wave of a 4-wave workgroup, and a
// very long one ceil(S / n_splits).
__device__ __forceinline__ uint32_t chunk_floor(int S, int min_chunk) {
  if (min_chunk > 0) return (uint32_t)min_chunk;
  const uint32_t f = (((uint32_t)S + 1023u) >> 10) << 5;
  return f < 32u ? 32u : (f > 128u ? 128u : f);
}

__device__ __forceinline__ void chunking(int S, int n_splits, int min_chunk, int& c, int& n_active) {
  if (S <= 0) {
    c = 0;
    n_active = 0;
    return;
  }
  unsigned uc = ((unsigned)S + (unsigned)n_splits - 1u) / (unsigned)n_splits;
  const unsigned floor_c = chunk_floor(S, min_chunk);
  if (uc < floor_c) uc = floor_c;
  c = (int)uc;
  n_active = (int)(((unsigned)S + uc - 1u) / uc);
}

// The split kernels' chunk length, the same value chunking() gives; a chunk s
// is empty when s * c >= S (no second division for the count of non-empty
// chunks on the path to the first K/V load).
__device__ __forceinline__ int split_chunk(int S, const SplitArgs& a) {
  const uint32_t q = ((uint32_t)S + (uint32_t)a.n_splits - 1u) / (uint32_t)a.n_splits;
  return (int)max(q, chunk_floor(S, a.min_chunk));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Butterfly steps of a wave-wide reduction as VALU operations instead of LDS
// permutes: each returns op(x, x of lane ^ 32 / ^ 16 / ^ 8) in every lane,
// with the two operands in the same order in both lanes of a pair (so both
// hold the same bits). gfx950's permlane swaps exchange the two 32-lane
// halves (or adjacent 16-lane rows) of two registers; given x twice they
// return the pair's lower and upper values side by side. A DPP rotation by 8
// within each 16-lane row pairs lane j with lane j ^ 8.
__device__ __forceinline__ void halves32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void halves16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x32(float x) { float a, b; halves32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x32(float x) { float a, b; halves32(x, a, b); return a + b; }
__device__ __forceinline__ float max_x16(float x) { float a, b; halves16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x16(float x) { float a, b; halves16(x, a, b); return a + b; }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {   // row_ror:8 = 0x128, quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_x8(float x) {     // lanes j and j ^ 8 of each 16-lane row
  const float y = dpp<0x128>(x);
  return (__lane_id() & 8) ? y + x : x + y;            // lower lane's value first in both
}
__device__ __forceinline__ float max_x8(float x) { return fmaxf(x, dpp<0x128>(x)); }
// Maximum over all 64 lanes, in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));                          // lane ^ 1
  x = fmaxf(x, dpp<0x4E>(x));                          // lane ^ 2
  x = fmaxf(x, dpp<0x124>(x));                         // row rotation by 4: with the next, the whole row
  x = max_x8(x);
  return max_x32(max_x16(x));
}

// Sum of a 64-bit integer over all 64 lanes, in every lane (exact in any
// order): quad butterflies and row rotations by 4 and 8 (DPP) cover each
// 16-lane row, the permlane swaps the rows and halves.
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  auto add = [&](uint32_t plo, uint32_t phi) { v += ((uint64_t)phi << 32) | plo; };
  auto lo = [&]() { return (uint32_t)v; };
  auto hi = [&]() { return (uint32_t)(v >> 32); };
#define GQA_DPP_STEP(CTRL) \
  add((uint32_t)__builtin_amdgcn_mov_dpp((int)lo(), CTRL, 0xF, 0xF, true), \
      (uint32_t)__builtin_amdgcn_mov_dpp((int)hi(), CTRL, 0xF, 0xF, true))
  GQA_DPP_STEP(0xB1);                                  // lane ^ 1
  GQA_DPP_STEP(0x4E);                                  // lane ^ 2
  GQA_DPP_STEP(0x124);                                 // row rotation by 4
  GQA_DPP_STEP(0x128);                                 // row rotation by 8: every lane holds its row's sum
#undef GQA_DPP_STEP
  {
    const auto rl = __builtin_amdgcn_permlane16_swap(lo(), lo(), false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap(hi(), hi(), false, false);
    const bool up = __lane_id() & 16;                  // partner = the other row of the pair
    add(up ? rl[0] : rl[1], up ? rh[0] : rh[1]);
  }
  {
    const auto rl = __builtin_amdgcn_permlane32_swap(lo(), lo(), false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi(), hi(), false, false);
    const bool up = __lane_id() & 32;
    add(up ? rl[0] : rl[1], up ? rh[0] : rh[1]);
  }
  return v;
}


// Length S_b and first token row of sequence b, with one round of loads:
// explicit offsets are loaded next to seq_lens[b]; for the packed layout the
// wave reads seq_lens[0..b] (lane j holds S_j of its 64-sequence slice),
// takes S_b from lane b and sums the lanes below b (every lane gets both).
__device__ __forceinline__ void seq_info(const int32_t* seq_lens, const int64_t* kv_off, int b,
                                         int lane, int& S, int64_t& off) {
  if (kv_off) {
    S = seq_lens[b];
    off = kv_off[b];
    return;
  }
  if (b == 0) {
    S = seq_lens[0];
    off = 0;
    return;
  }
  int64_t acc = 0;
  int sb = 0;
  for (int base = 0; base <= b; base += 64) {     // one pass when b < 64
    const int j = base + lane;
    const int v = (j <= b) ? seq_lens[j] : 0;
    if (j < b) acc += v;
    if (base + 64 > b) sb = __builtin_amdgcn_readlane(v, b - base);
  }
  S = sb;
  off = (int64_t)wave_sum_u64((uint64_t)acc);
}

// Longest sequences first. The hardware starts workgroups in grid order, and
// with the batch as the grid's slowest dimension a ragged batch whose
// longest sequence comes late starts that sequence's chunks (every sequence
// gets the same number, so its chunks are the longest) in the last rounds,
// where they form the launch's tail. Here batch slot z (z < B <=
// kRankedMaxBatch) runs the sequence of rank z by length, longest first,
// ties in batch order: the longest chunks start first (the
// longest-processing-time-first order of list scheduling). One wave loads
// the B lengths (and explicit offsets), one lane per sequence; each lane
// counts the sequences that rank before its own, with keys (length, 63 -
// lane) that are all distinct, so exactly one lane holds rank z (the ballot
// is never empty; should it be, the slot keeps sequence z). The count takes
// one step per sequence, so the host asks for it only where the order pays
// (ranked_batch). The same loads give the chosen sequence's length and its
// packed token base (the lengths of the sequences before it in the batch),
// so this costs no memory round trip over seq_info. Which workgroup computes
// which chunk changes no arithmetic: the bits are those of the batch order.
constexpr int kRankedMaxBatch = 64;
// The sequence b of rank z given lane j's length v (lanes below B), ties in
// batch order.
__device__ __forceinline__ int rank_slot(int v, int B, int z, int lane) {
  const bool in = lane < B;
  // Keys: the length (clamped to 2^26 - 1; longer ones tie and keep the batch
  // order) above the lane's 6 bits, reversed so that an earlier sequence
  // wins a tie. Groups of 8 lanes per step: j0 <= 56 when B <= 64, so every
  // lane index read is below 64.
  const uint32_t key = (min((uint32_t)v, (1u << 26) - 1u) << 6) | (uint32_t)(63 - lane);
  int rank = 0;
  for (int j0 = 0; j0 < B; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;                       // uniform: readlane takes it as a scalar
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
      rank += (j < B && kj > key) ? 1 : 0;
    }
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(in && rank == z);
  return hit ? (int)__builtin_ctzll(hit) : z;
}
__device__ __forceinline__ void seq_info_ranked(const int32_t* seq_lens, const int64_t* kv_off, int B, int z,
                                                int lane, int& b, int& S, int64_t& off) {
  const bool in = lane < B;
  const int v = in ? seq_lens[lane] : 0;
  const int64_t o = (in && kv_off) ? kv_off[lane] : 0;
  b = rank_slot(v, B, z, lane);
  S = __builtin_amdgcn_readlane(v, b);
  if (kv_off) {
    off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(o >> 32), b) << 32) |
                    (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)o, b));
  } else {
    off = (int64_t)wave_sum_u64(lane < b ? (uint64_t)(uint32_t)v : 0ull);
  }
}

// Streaming loads of the KV cache: every K/V byte is read once per call, so
// the loads carry the non-temporal hint (measured: 1M-token split kernel
// 716 us -> 647 us, 6.0 -> 6.6 TB/s).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_stream4(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

// (split s, kv head g, sequence b) of a split workgroup. Splits vary fastest
// in the grid: measured against kv-head-fastest and an XCD-grouped order, this
// order streams long sequences fastest (1M tokens: 722 us vs 769 and 747 us).
struct WgCoord {
  int s, g, b;
};
__device__ __forceinline__ WgCoord wg_coord() {
  return {(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
}
inline dim3 split_grid(int n_splits, int h_kv, int B) {
  return dim3((unsigned)n_splits, (unsigned)h_kv, (unsigned)B);
}
// The 8-wave forms (one round of one workgroup per CU) take kv heads
// fastest instead. Measured at 70B shapes: split kernel 0.26 µs faster at
// 8k tokens (the same loads alone: 6.58 µs in this order against 7.14 µs
// with splits fastest) and 0.4 µs at 16k; two-tile multi-token decode with
// 4 query tokens at 8k 15.8 -> 14.9 µs per call. Workgroup L then runs on
// XCD L mod 8, so each XCD reads one kv head's rows. Splits fastest stays
// the order for several rounds (at 32k tokens in one-block chunks the same
// loads take 21.2 µs splits fastest and 21.9 µs heads fastest).
inline dim3 split_grid_heads_fastest(int n_splits, int h_kv, int B) {
  return dim3((unsigned)h_kv, (unsigned)n_splits, (unsigned)B);
}

}  // namespace gqa
