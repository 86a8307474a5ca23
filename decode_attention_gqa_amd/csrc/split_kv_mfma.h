// Split-KV partial attention on the gfx950 matrix cores (bf16 q, K, V).
//
// One workgroup owns one chunk of one (sequence b, kv head g) pair and the
// n_rep query heads of that group. Each of its waves (4 by default) walks
// 32-token blocks of the chunk (wave w of W takes blocks w, w+W, ...), two
// register buffers in turn so the next block is in flight while one is
// computed, and keeps an online-softmax state (m, l, o) for the group's
// heads; at the end the waves' states are merged in LDS and the workgroup
// writes one (m, l, o) triplet per head. Two template options widen the same kernel: APPEND (a decode
// step that appends the new token on the way) and TILES = 2 (two 16-column
// tiles of several query tokens per workgroup); see the kernel. WAVES = 1
// gives one-wave workgroups for chunks of a few blocks (many short
// sequences), where some of four waves would have nothing to read; WAVES = 8
// gives one workgroup per CU for a single sequence cut into one round of
// chunks (half as many chunks to store and merge as two 4-wave workgroups).
//
// Per 32-token block, with 16x16x32 bf16 MFMAs:
//   scores  S^T[t, h] = K[t, :] . Q[h, :]      A = K rows, B = Q^T (2 tiles x D/32 steps)
//   output  O^T[i, h] += V[t, i] * P[h, t]     A = V^T,    B = P^T (D/16 tiles)
// Computing the transposed products makes the MFMA output layout of the
// scores (lane = head, registers = 4 tokens) exactly the B-operand layout the
// P.V product needs, and puts the per-head softmax statistics in the same
// lanes as the output rows they rescale - no cross-lane exchange besides the
// max over a column's 4 lane groups (two permlane swaps). Query heads
// n_rep..15 of the 16-wide tile are zero padding.
//
// Data movement: K and V go from HBM to registers with 16-byte non-temporal
// loads, each instruction reading whole rows (the group's heads share each
// K/V register inside the MFMA; no workgroup-wide staging). A lane's 8 V
// loads are 8 tokens x 8 consecutive dimensions; an in-register 8x8
// transpose of 16-bit values turns them into the MFMA A operand (8 tokens of
// one dimension). K, loaded a row piece per lane, passes through a small
// per-wave LDS region on its way to the A-operand layout (a row per lane%16).
// Every K and V byte of the chunk is read exactly once.
//
// The softmax probabilities are split into bf16 hi + lo parts and both are
// multiplied with V, so P.V keeps about 16 significant bits of P (bf16 alone
// would keep 8); l is accumulated from the fp32 values.
#pragma once

#include "fused_tail.h"
#include "gqa_common.h"

namespace gqa {

template <int D>
struct MfmaTile {
  static constexpr int KS = D / 32;   // k-steps of the score product
  static constexpr int NT = D / 16;   // output tiles (16 dims each) of P.V
  static constexpr int VW = NT / 2;   // dwords per lane per V token load (8 or 4 bf16)
};

// Per-lane registers of one 32-token block.
template <int D>
struct KVRegs {
  // K: as loaded, piece i is row KRowsPerLoad*i + lane / KPieces, bytes
  // 16*(lane % KPieces) (whole rows per load instruction); after
  // k_to_operand, k[x][kk] is the MFMA A operand: row 16x + lane%16, bytes
  // 16*(lane/16) + 64*kk.
  uint4 k[2][MfmaTile<D>::KS];
  uint32_t v[8][MfmaTile<D>::VW];     // V: token slot j, VW dwords of consecutive dims
};

// K rows in the layout they are loaded in: a 16-byte piece per lane, whole
// rows per instruction (4 rows of 256 bytes at d = 128, 8 of 128 at d = 64).
// The MFMA wants 16 rows per instruction instead (a row per lane%16), which as
// loads reach 16 rows x 64 bytes per instruction and measured 0.9 µs slower
// over 32 MiB than whole rows; the wave turns one layout into the other
// through LDS (k_to_operand).
template <int D>
struct KLoad {
  static constexpr int KPieces = D * 2 / 16;          // 16-byte pieces per row
  static constexpr int KRowsPerLoad = 64 / KPieces;   // rows per load instruction
  static constexpr int ROW = D * 2 + 16;              // padded row in LDS: the 16 lanes of a lane
                                                      // group read 16 rows at one column
  static constexpr int BYTES = 32 * ROW;              // one wave's block of K rows
};

// Token (within the 32-token block) that lane group `grp` holds in slot j of
// the P operand. It follows from the score output layout: tile 0 gives
// tokens 4*grp + r, tile 1 gives 16 + 4*grp + r (r = 0..3).
__device__ __forceinline__ int slot_token(int grp, int j) {
  return (j < 4) ? (4 * grp + j) : (16 + 4 * grp + (j - 4));
}

// Byte offsets, from the first K (or V) row of a block, of the 16-byte
// pieces a lane loads: K piece i (see KVRegs), V row of token
// slot_token(grp, j) at dims NT*n. Tokens at or past nv (a chunk's last,
// partial block) are clamped to nv - 1: read again, and masked out of the
// softmax.
template <int D>
struct LaneOffsets {
  uint32_t k[2 * MfmaTile<D>::KS];
  uint32_t v[8];
};

template <int D>
__device__ __forceinline__ LaneOffsets<D> lane_offsets(uint32_t row_bytes, int grp, int n, int nv) {
  constexpr int NT = MfmaTile<D>::NT, KS = MfmaTile<D>::KS;
  using KL = KLoad<D>;
  const int lane = 16 * grp + n;
  LaneOffsets<D> o;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i)
    o.k[i] = (uint32_t)min(KL::KRowsPerLoad * i + lane / KL::KPieces, nv - 1) * row_bytes +
             16u * (lane % KL::KPieces);
#pragma unroll
  for (int j = 0; j < 8; ++j) o.v[j] = (uint32_t)min(slot_token(grp, j), nv - 1) * row_bytes + 2u * NT * n;
  return o;
}

template <int D>
__device__ __forceinline__ void load_block(KVRegs<D>& r, const char* kb, const char* vb,
                                           const LaneOffsets<D>& o) {
  constexpr int KS = MfmaTile<D>::KS, VW = MfmaTile<D>::VW;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) r.k[i / KS][i % KS] = load_stream16(kb + o.k[i]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (VW == 4) {
      const uint4 u = load_stream16(vb + o.v[j]);
      r.v[j][0] = u.x; r.v[j][1] = u.y; r.v[j][2] = u.z; r.v[j][3] = u.w;
    } else {
      const uint2 u = load_stream8(vb + o.v[j]);
      r.v[j][0] = u.x; r.v[j][1] = u.y;
    }
  }
}

// The block that holds a decode step's new token (its last valid token,
// nv - 1), after load_block has read it from the cache (whose row for the new
// token is not written yet): lanes whose (clamped) token is nv - 1 load the
// caller's new K/V row over it. The block's other loads stay those of
// load_block (measured: a decode step 0.15 µs faster than building every
// address of that block per lane).
template <int D>
__device__ __forceinline__ void patch_new_row(KVRegs<D>& r, int grp, int n, int nv, const char* k_row,
                                              const char* v_row) {
  constexpr int KS = MfmaTile<D>::KS, NT = MfmaTile<D>::NT, VW = MfmaTile<D>::VW;
  using KL = KLoad<D>;
  const int lane = 16 * grp + n;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i)
    if (min(KL::KRowsPerLoad * i + lane / KL::KPieces, nv - 1) == nv - 1)
      r.k[i / KS][i % KS] = load_stream16(k_row + 16 * (lane % KL::KPieces));
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (min(slot_token(grp, j), nv - 1) == nv - 1) {
      if constexpr (VW == 4) {
        const uint4 u = load_stream16(v_row + 2 * NT * n);
        r.v[j][0] = u.x; r.v[j][1] = u.y; r.v[j][2] = u.z; r.v[j][3] = u.w;
      } else {
        const uint2 u = load_stream8(v_row + 2 * NT * n);
        r.v[j][0] = u.x; r.v[j][1] = u.y;
      }
    }
}

// A operand of output tile nt: dimension NT*(lane%16) + nt of the 8 slot tokens.
template <int D>
__device__ __forceinline__ bf16x8 v_tile(const KVRegs<D>& r, int nt) {
  // Even nt: the low 16-bit halves of slots 2i, 2i+1; odd nt: the high
  // halves. One byte permute each (selector bytes 0-3 pick from the second
  // operand, 4-7 from the first).
  const int w = nt >> 1;
  const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
  uint4 a;
  uint32_t* pa = reinterpret_cast<uint32_t*>(&a);
#pragma unroll
  for (int i = 0; i < 4; ++i) pa[i] = __builtin_amdgcn_perm(r.v[2 * i + 1][w], r.v[2 * i][w], sel);
  return __builtin_bit_cast(bf16x8, a);
}

// K from its load layout to the MFMA A-operand layout, through this wave's
// KLoad<D>::BYTES of LDS (rows padded to KLoad<D>::ROW bytes). Only this wave
// touches the region, and a wave's LDS accesses complete in order.
template <int D>
__device__ __forceinline__ void k_to_operand(KVRegs<D>& r, char* kt, int grp, int n) {
  constexpr int KS = MfmaTile<D>::KS;
  using KL = KLoad<D>;
  const int lane = 16 * grp + n;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i)
    *reinterpret_cast<uint4*>(kt + (KL::KRowsPerLoad * i + lane / KL::KPieces) * KL::ROW +
                              16 * (lane % KL::KPieces)) = r.k[i / KS][i % KS];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      r.k[x][kk] = *reinterpret_cast<const uint4*>(kt + (16 * x + n) * KL::ROW + 16 * grp + 64 * kk);
}

struct SoftmaxState {
  float m;   // running max of this lane's head (log2 units), shared by the 4 lane groups
  float l;   // partial sum of exponentials over this lane's tokens
};

// P^T as bf16 hi + lo parts in the B-operand layout: two values per
// conversion (round to nearest even, as the scalar cast); a bf16 read back as
// fp32 is its bits in the upper half, and the part it misses is rounded again.
__device__ __forceinline__ void split_p(const float (&p)[8], bf16x8& ph, bf16x8& pl) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const bf16x2_t h = __builtin_convertvector((f32x2_t){p[j], p[j + 1]}, bf16x2_t);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xFFFF0000u);
    const bf16x2_t l = __builtin_convertvector((f32x2_t){p[j] - h0, p[j + 1] - h1}, bf16x2_t);
    ph[j] = h[0];
    ph[j + 1] = h[1];
    pl[j] = l[0];
    pl[j + 1] = l[1];
  }
}

// Scores of one 16-column tile for a block in log2 units: x[j] is the score of
// token slot_token(grp, j) for this lane's column.
template <int D>
__device__ __forceinline__ void tile_scores(const KVRegs<D>& r, const bf16x8 (&qop)[MfmaTile<D>::KS],
                                            float scale_log2, float (&x)[8]) {
  constexpr int KS = MfmaTile<D>::KS;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[0][kk]), qop[kk], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[1][kk]), qop[kk], s1, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i] * scale_log2;
    x[4 + i] = s1[i] * scale_log2;
  }
}

// The block's max of this lane's column (over the 4 lane groups), after the
// masked positions (slot tokens at or past nvl) are set to -inf.
__device__ __forceinline__ float block_max(float (&x)[8], int grp, bool mask, int nvl) {
  if (mask) {                                // tail of the chunk, or causal limit of the column
    // slot_token(grp, j) >= nvl, with the lane group's part on the right so
    // that the slot's part stays an immediate (no registers held for it).
    const int rel = nvl - 4 * grp;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j < 4 ? j : 12 + j) >= rel) x[j] = -INFINITY;
  }
  float mb = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mb = fmaxf(mb, x[j]);
  return max_x32(max_x16(mb));
}

// Slack of the lazy reference max (log2 units): see softmax_update.
constexpr float kRescaleSlack = 8.f;

// The online-softmax update of a tile's state for a block (running max, sum,
// and the rescale of its accumulators) from the block's scores x and their
// max mb; gives P^T as bf16 hi + lo parts.
//
// LAZY: st.m is a reference point instead of the running max. It moves (to
// the block's max) only when a column's block max exceeds it by more than
// kRescaleSlack, so the exponentials are taken against a reference up to 8
// below the max: values up to 2^8, exact in fp32 and split into bf16 hi + lo
// as before, and l and o stay consistent with the reference (o / l is the
// same; m + log2(l) is the log-sum-exp either way). The accumulators are then
// rescaled only in the rare blocks where the reference moves, instead of in
// nearly every block of a chunk's first few dozen, where some of a tile's 16
// columns finds a new max.
template <int D, bool LAZY = false>
__device__ __forceinline__ void softmax_update(const float (&x)[8], float mb, f32x4 (&acc)[MfmaTile<D>::NT],
                                               SoftmaxState& st, bf16x8& ph, bf16x8& pl) {
  constexpr int NT = MfmaTile<D>::NT;
  // -inf + slack = -inf: the first block with a position moves the reference.
  const float mn = LAZY ? (mb > st.m + kRescaleSlack ? mb : st.m) : fmaxf(st.m, mb);
  // mn = -inf only while every position this column has seen is masked (a
  // causal column before its first position); keep alpha and p at 0 then.
  const float mref = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = fast_exp2(st.m - mref);  // 0 on the first block (m = -inf)
  const bool grew = mn > st.m;
  st.m = mn;
  float p[8], ls = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fast_exp2(x[j] - mref);
    ls += p[j];
  }
  st.l = st.l * alpha + ls;
  // alpha is exactly 1 in every lane whose max did not grow: the rescale of
  // the accumulators is skipped unless some lane's max grew (rare after the
  // first blocks). A lane whose state was empty has acc = 0 either way.
  if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
  }
  split_p(p, ph, pl);
}

// Scores of one 16-column tile for a block and the online-softmax update of
// its state; gives P^T as bf16 hi + lo parts in the B-operand layout.
template <int D, bool LAZY = false>
__device__ __forceinline__ void softmax_block(const KVRegs<D>& r, const bf16x8 (&qop)[MfmaTile<D>::KS],
                                              f32x4 (&acc)[MfmaTile<D>::NT], SoftmaxState& st,
                                              float scale_log2, int grp, bool mask, int nvl,
                                              bf16x8& ph, bf16x8& pl) {
  float x[8];
  tile_scores<D>(r, qop, scale_log2, x);
  const float mb = block_max(x, grp, mask, nvl);
  softmax_update<D, LAZY>(x, mb, acc, st, ph, pl);
}

// O^T += V^T P^T for TILES column tiles that share the block's V: each V^T
// operand is formed once and multiplied with every tile's P^T (hi and lo).
template <int D, int TILES>
__device__ __forceinline__ void pv_block(const KVRegs<D>& r, f32x4 (&acc)[TILES][MfmaTile<D>::NT],
                                         const bf16x8 (&ph)[TILES], const bf16x8 (&pl)[TILES]) {
  constexpr int NT = MfmaTile<D>::NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bf16x8 a = v_tile<D>(r, nt);
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph[t], acc[t][nt], 0, 0, 0);
      acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[t], acc[t][nt], 0, 0, 0);
    }
  }
}

// APPEND: one decode step with the new token appended on the way (single
// query token; padded cache). The sequence is S = min(S_b + 1, capacity)
// tokens long; when S_b < capacity its last token is the new one, read from
// k_new / v_new by the workgroup whose chunk holds it, which also copies that
// row into the cache (no other workgroup reads it), and lens_out[b] = S.
//
// TILES = 2 (several query tokens): the workgroup carries two 16-column tiles
// of (query token, head) columns through the chunk, so each K/V block is read
// once for both; each tile has its own softmax state and accumulators, and
// they share the block's V^T operands. Twice the accumulators leave room for
// one workgroup per CU only (one wave per SIMD).
template <int D, int NREP, bool APPEND = false, int TILES = 1, int WAVES = kWaves>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(TILES == 1 || WAVES == 8 ? 2 : 1)))
void split_kv_mfma(SplitArgs a) {
  constexpr int KS = MfmaTile<D>::KS, NT = MfmaTile<D>::NT;
  constexpr int THREADS = 64 * WAVES;
  static_assert(WAVES == kWaves || (WAVES == 1 && TILES == 1) || WAVES == 8, "1 wave: one column tile");
  static_assert(!APPEND || 2 * (D * 2 / 16) <= 64 * WAVES, "the new row's copy takes one thread per 16 bytes");
  static_assert(NREP >= 1 && NREP <= 16, "one 16-wide MFMA tile holds the query heads of a group");
  static_assert(TILES == 1 || (TILES == 2 && !APPEND), "two tiles serve multi-token decode only");
  // 8 waves: the grid has kv heads fastest (split_grid_heads_fastest).
  const WgCoord wc = WAVES == 8 ? WgCoord{(int)blockIdx.y, (int)blockIdx.x, (int)blockIdx.z} : wg_coord();
  const int s = wc.s, g = wc.g;
  const int zb = a.passes == 1 ? wc.b : wc.b / a.passes, pass = wc.b - zb * a.passes;
  int b = zb;                                      // the sequence (batch slot zb runs it)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int grp = lane >> 4, n = lane & 15;
  // Column n of tile t: query token qi[t], head g*NREP + hh.
  const int ti = n / NREP, hh = n % NREP;
  int qi[TILES];
  bool col[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    qi[t] = (pass * TILES + t) * a.tpt + ti;
    col[t] = ti < a.tpt && qi[t] < a.s_q;
  }
  const bool causal = a.s_q > 1;

  int S;
  int64_t off;
  bool appended = false;                           // APPEND: the new token is position S - 1
  if constexpr (APPEND) {
    int old;
    if (a.ranked) {                                // longest first, as seq_info_ranked
      const int v = lane < a.ranked ? a.seq_lens[lane] : 0;
      b = rank_slot(v, a.ranked, zb, lane);
      old = __builtin_amdgcn_readlane(v, b);
    } else {
      old = a.seq_lens[b];
    }
    off = a.kv_off ? a.kv_off[b] : (int64_t)b * a.capacity;
    appended = old < a.capacity;                   // else the new row is dropped
    S = appended ? old + 1 : a.capacity;
  } else if (a.ranked) {
    seq_info_ranked(a.seq_lens, a.kv_off, a.ranked, zb, lane, b, S, off);
  } else {
    seq_info(a.seq_lens, a.kv_off, b, lane, S, off);
  }
  // Every lane holds the same S and off; saying so keeps the block base
  // addresses in scalar registers (loads then add only a 32-bit lane offset).
  S = __builtin_amdgcn_readfirstlane(S);
  off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)off));
  const int c = split_chunk(S, a);                 // chunk s: tokens [s*c, min(S, (s+1)*c))
  // APPEND: the new length is stored last (a store early in the kernel would
  // sit in the wave's memory counter ahead of its K/V loads and every wait for
  // them would wait for its acknowledgement too: 0.25 µs per decode step).
  const bool lens_writer = APPEND && a.lens_out && s == 0 && g == 0 && tid == 0;
  if ((int64_t)s * c >= S) {                       // an empty chunk: the merge reads non-empty ones only
    if (lens_writer) a.lens_out[b] = S;
    if constexpr ((WAVES == kWaves || WAVES == 8) && TILES == 1 && !APPEND)
      if (a.fused && S == 0 && s == 0) fused_empty<D, NREP, THREADS>(a, g, b);
    if (a.direct && S == 0 && s == 0) {            // nothing attended: out = 0
      constexpr int Q4 = D / 4;
      for (int t = 0; t < TILES; ++t)
        for (int idx = tid; idx < NREP * a.tpt * Q4; idx += THREADS) {
          const int h = idx / Q4, cqi = (pass * TILES + t) * a.tpt + h / NREP;
          if (cqi >= a.s_q) continue;
          const int64_t e = (((int64_t)b * a.s_q + cqi) * a.h_q + g * NREP + h % NREP) * D + (idx % Q4) * 4;
          if (a.out_bf16)
            store4<__bf16>(static_cast<__bf16*>(a.out) + e, make_float4(0.f, 0.f, 0.f, 0.f));
          else
            store4<float>(static_cast<float*>(a.out) + e, make_float4(0.f, 0.f, 0.f, 0.f));
        }
    }
    return;
  }
  const int64_t t0 = (int64_t)s * c;
  const int ntok = (int)min<int64_t>((int64_t)S - t0, c);

  const int64_t rs = (int64_t)a.h_kv * D;          // elements between consecutive tokens
  const __bf16* kbase = static_cast<const __bf16*>(a.k) + ((off + t0) * a.h_kv + g) * D;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + ((off + t0) * a.h_kv + g) * D;

  // Q^T as the B operand: lane (grp, n) holds q[token qi][head g*NREP + hh][32*kk + 8*grp .. +8].
  bf16x8 qop[TILES][KS];
  int lim[TILES];                                  // last position each column's token attends
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int h = g * NREP + hh;
    const __bf16* qrow =
        static_cast<const __bf16*>(a.q) + (((int64_t)b * a.s_q + qi[t]) * a.h_q + h) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (col[t]) u = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qop[t][kk] = __builtin_bit_cast(bf16x8, u);
    }
    lim[t] = S - a.s_q + qi[t];                    // causal among the new tokens
  }
  int lim0[TILES];                                 // the tile's smallest limit (its first token's)
#pragma unroll
  for (int t = 0; t < TILES; ++t) lim0[t] = S - a.s_q + (pass * TILES + t) * a.tpt;

  f32x4 acc[TILES][NT];
  SoftmaxState st[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[t] = SoftmaxState{-INFINITY, 0.f};
  }

  // APPEND: the workgroup whose chunk ends the sequence also copies the new
  // token's K and V rows of head g into the cache: 16-byte pieces loaded
  // before the block loop and stored after it (a store inside the loop would
  // make every wait in it drain the prefetched block too).
  const int64_t src_new = ((int64_t)b * a.h_kv + g) * D * 2;            // row in k_new / v_new (bytes)
  const int64_t row_new = ((off + S - 1) * a.h_kv + g) * D * 2;         // its cache row (bytes)
  constexpr int U16 = D * 2 / 16;                                       // 16-byte pieces per row
  const bool copier = APPEND && appended && (int64_t)(s + 1) * c >= S && tid < 2 * U16;   // the last chunk
  uint4 piece = make_uint4(0u, 0u, 0u, 0u);
  if (copier)
    piece = *reinterpret_cast<const uint4*>(static_cast<const char*>(tid < U16 ? a.k_new : a.v_new) + src_new +
                                            16 * (tid % U16));

  const int nblk = (ntok >> 5) + ((ntok & 31) != 0);
  if (w < nblk) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);   // <= 65535 * 256 < 2^24: 32 rows fit 32 bits
    const char* kb0 = reinterpret_cast<const char*>(kbase);
    const char* vb0 = reinterpret_cast<const char*>(vbase);
    const LaneOffsets<D> full = lane_offsets<D>(row_bytes, grp, n, 32);
    __shared__ __attribute__((aligned(16))) char kt[WAVES][KLoad<D>::BYTES];   // each wave's K transpose
    // APPEND: the block whose last token ends the sequence holds the new token.
    auto holds_new = [&](int bk, int nvb) { return APPEND && appended && t0 + bk * 32 + nvb == S; };
    auto load = [&](KVRegs<D>& r, int bk) {
      const int64_t base = (int64_t)bk * 32 * row_bytes;
      const int nvb = min(32, ntok - bk * 32);
      // Only the offsets depend on the branch: the loads after it are the
      // same instructions on both paths.
      LaneOffsets<D> o = full;
      if (nvb < 32) o = lane_offsets<D>(row_bytes, grp, n, nvb);
      load_block<D>(r, kb0 + base, vb0 + base, o);
      if (holds_new(bk, nvb))
        patch_new_row<D>(r, grp, n, nvb, static_cast<const char*>(a.k_new) + src_new,
                         static_cast<const char*>(a.v_new) + src_new);
    };
    auto step = [&](KVRegs<D>& r, int bk) {
      k_to_operand<D>(r, kt[w], grp, n);
      const int nv = min(32, ntok - bk * 32);
      bf16x8 ph[TILES], pl[TILES];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int nvl = causal ? min(nv, lim[t] - ((int)t0 + bk * 32) + 1) : nv;
        // The causal mask matters only in blocks past the tile's first token's limit.
        const bool mask = nv < 32 || (causal && (int)t0 + bk * 32 + nv - 1 > lim0[t]);
        // Two tiles serve only multi-token calls, whose triplets stay inside
        // the library: the lazy reference applies (see softmax_update).
        softmax_block<D, TILES == 2>(r, qop[t], acc[t], st[t], a.scale_log2, grp, mask, nvl, ph[t], pl[t]);
      }
      pv_block<D, TILES>(r, acc, ph, pl);
    };
    // Two register buffers in turn: the next block of this wave is in flight
    // while the current one is computed.
    KVRegs<D> ra, rb;
    int blk = w;
    load(ra, blk);
    if constexpr (TILES == 2 && WAVES == 8) {
      // Two tiles with eight waves: one register buffer (two would not fit
      // next to two tiles' state at two waves per SIMD); the host takes this
      // form only where every wave has one block, so nothing waits on a load
      // that a second buffer could have hidden.
      while (true) {
        step(ra, blk);
        blk += WAVES;
        if (blk >= nblk) break;
        load(ra, blk);
      }
    } else if constexpr (TILES == 2) {
      // The loads of the next block are issued on every path that then
      // computes the current one (the last block is computed outside the
      // loop), so the wait before computing covers the current block's loads
      // only: after a load that some path skips, the compiler waits for
      // every load in flight. (With one tile the extra copies of the block
      // code this takes would spill registers.)
      while (blk + WAVES < nblk) {
        load(rb, blk + WAVES);
        step(ra, blk);
        blk += WAVES;
        if (blk + WAVES >= nblk) {
          step(rb, blk);
          blk = -1;                                // done
          break;
        }
        load(ra, blk + WAVES);
        step(rb, blk);
        blk += WAVES;
      }
      if (blk >= 0) step(ra, blk);
    } else {
      while (true) {
        int nb = blk + WAVES;
        if (nb < nblk) load(rb, nb);
        step(ra, blk);
        if (nb >= nblk) break;
        blk = nb;
        nb = blk + WAVES;
        if (nb < nblk) load(ra, nb);
        step(rb, blk);
        if (nb >= nblk) break;
        blk = nb;
      }
    }
  }

  if (copier)
    *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(tid < U16 ? a.k : a.v)) + row_new +
                              16 * (tid % U16)) = piece;

  // Merge the waves' states in LDS and write the workgroup's triplets, one
  // tile at a time through the same LDS.
  constexpr int OP = D + 4;                        // padded row (fewer bank conflicts)
  constexpr int Q4 = D / 4;
  const int cols = NREP * a.tpt;                   // columns in use (<= 16)
  __shared__ float sm_m[WAVES][16], sm_l[WAVES][16];
  __shared__ float sm_o[WAVES][16][OP];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    // l: sum the 4 lane groups' partial sums (m is already shared by them).
    const float l = sum_x32(sum_x16(st[t].l));
    if (t > 0) __syncthreads();                    // the previous tile's reads are done
    if (grp == 0) {
      sm_m[w][n] = st[t].m;
      sm_l[w][n] = l;
    }
    if (n < cols) {
      // lane (grp, n) holds o[column n][NT*(4*grp + r) + nt]
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sm_o[w][n][NT * (4 * grp + r) + nt] = acc[t][nt][r];
    }
    __syncthreads();
    for (int idx = tid; idx < cols * Q4; idx += THREADS) {
      const int h = idx / Q4, d4 = (idx % Q4) * 4;      // h: column of the tile
      const int cqi = (pass * TILES + t) * a.tpt + h / NREP;
      if (cqi >= a.s_q) continue;
      float M = sm_m[0][h];
#pragma unroll
      for (int ww = 1; ww < WAVES; ++ww) M = fmaxf(M, sm_m[ww][h]);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      float L = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        const float mw = sm_m[ww][h];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);   // a wave with no block
        L += f * sm_l[ww][h];
        o.x += f * sm_o[ww][h][d4 + 0];
        o.y += f * sm_o[ww][h][d4 + 1];
        o.z += f * sm_o[ww][h][d4 + 2];
        o.w += f * sm_o[ww][h][d4 + 3];
      }
      const int64_t orow = ((int64_t)b * a.s_q + cqi) * a.h_q + g * NREP + h % NREP;   // (b, token, head)
      if (a.direct) {                              // the sequence's only chunk: out = o / l here
        const float inv = L > 0.f ? 1.f / L : 0.f;   // L = 0: nothing attended (a causal column)
        const float4 r = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        if (a.out_bf16)
          store4<__bf16>(static_cast<__bf16*>(a.out) + orow * D + d4, r);
        else
          store4<float>(static_cast<float*>(a.out) + orow * D + d4, r);
      } else {
        const int64_t row = orow * a.n_splits + s;
        *reinterpret_cast<float4*>(a.ws_o + row * D + d4) = o;
        if (d4 == 0) a.ws_ml[row] = make_float2(M, L);
      }
    }
  }
  if (lens_writer) a.lens_out[b] = S;
  if constexpr ((WAVES == kWaves || WAVES == 8) && TILES == 1 && !APPEND)   // the single-launch forms
    if (a.fused) fused_epilogue<D, NREP, THREADS>(a, g, b, (S + c - 1) / c);
}

}  // namespace gqa
