// Multi-token split-KV partial attention with each K/V block shared by the
// waves of a workgroup through LDS.
//
// With several query tokens per sequence, the (query token, head) columns of
// a kv head fill ceil(S_q * n_rep / 16) tiles of 16 MFMA columns. Here each
// of the workgroup's 8 waves owns one tile, and the workgroup stages every
// 32-token K/V block of its chunk in LDS once for all 8: each wave computes
// its tile against the staged block exactly as split_kv_mfma computes one
// tile (the same operand layouts, softmax and P.V code), reading the
// operands from LDS instead of HBM. So HBM delivers each K/V byte once per 8
// tiles (split_kv_mfma with two tiles per workgroup reads it once per 2, and
// a long sequence's passes then miss in the caches), and a wave holds one
// tile's state and no prefetch buffer (128 registers: two workgroups, 16 waves,
// per CU). Each wave's state covers the whole chunk, so the workgroup writes
// one triplet per (query token, head) of its tiles, or o / l when the
// sequence has one chunk.
//
// Staging: two LDS buffers in turn. While the waves compute block i from one
// buffer, each thread has its pieces of block i + 1 in flight from HBM to
// registers; it stores them into the other buffer afterwards, and one
// workgroup barrier per block orders the two. K rows are padded by 16 bytes
// in LDS, so the 16 lanes of a lane group, which read the same columns of 16
// different rows, hit 16 different bank groups.
#pragma once

#include "split_kv_mfma.h"

namespace gqa {

constexpr int kTileWaves = 8;                       // waves (= tiles) per workgroup

template <int D>
struct LdsBlock {
  static constexpr int ROW = D * 2;                 // bytes of one head's K (or V) row
  static constexpr int KROW = ROW + 16;             // padded K row in LDS
  static constexpr int VROW = ROW;                  // V rows: a lane group reads one row across
  static constexpr int KBYTES = 32 * KROW;
  static constexpr int BYTES = KBYTES + 32 * VROW;  // one staged block
  static constexpr int RP = ROW / 16;               // 16-byte pieces per row
  static constexpr int PIECES = 2 * 32 * RP;        // pieces of a block's K and V rows
};

template <int D, int NREP>
__global__ __launch_bounds__(64 * kTileWaves) __attribute__((amdgpu_waves_per_eu(4)))
void split_kv_tiles(SplitArgs a) {
  constexpr int NT = MfmaTile<D>::NT, KS = MfmaTile<D>::KS, VW = MfmaTile<D>::VW;
  constexpr int TW = kTileWaves, THREADS = 64 * TW;
  using L = LdsBlock<D>;
  static_assert(L::PIECES % THREADS == 0, "a block's pieces spread evenly over the threads");
  constexpr int PPT = L::PIECES / THREADS;
  constexpr int OP = D + 4;                         // padded row of the epilogue's o
  constexpr int Q4 = D / 4;
  constexpr int STAGE = 2 * L::BYTES;
  constexpr int EPI = TW * 16 * OP * 4;
  constexpr int LDS_BYTES = STAGE > EPI ? STAGE : EPI;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  __shared__ float sm_m[TW][16], sm_l[TW][16];

  const WgCoord wc = wg_coord();
  const int s = wc.s, g = wc.g;
  const int b = wc.b / a.passes, pass = wc.b - b * a.passes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, n = lane & 15;
  const int tile = pass * TW + w;                   // this wave's tile of the sequence
  const bool has_tile = tile < a.qtiles;
  const int ti = n / NREP, hh = n % NREP;
  const int qi = tile * a.tpt + ti;                 // column n: query token qi, head g*NREP + hh
  const bool col = has_tile && ti < a.tpt && qi < a.s_q;
  const int cols = NREP * a.tpt;                    // columns in use (<= 16)

  int S;
  int64_t off;
  seq_info(a.seq_lens, a.kv_off, b, lane, S, off);
  S = __builtin_amdgcn_readfirstlane(S);
  off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)off));
  int c, n_active;
  chunking(S, a.n_splits, a.min_chunk, c, n_active);
  if (s >= n_active) {                              // the merge reads chunks < n_active only
    if (a.direct && n_active == 0 && s == 0) {      // nothing attended: out = 0
      for (int idx = tid; idx < TW * cols * Q4; idx += THREADS) {
        const int t = pass * TW + idx / (cols * Q4), h = (idx / Q4) % cols;
        const int cqi = t * a.tpt + h / NREP;
        if (t >= a.qtiles || cqi >= a.s_q) continue;
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
  const uint32_t row_bytes = (uint32_t)((int64_t)a.h_kv * D * 2);
  const char* kb0 = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + ((off + t0) * a.h_kv + g) * D);
  const char* vb0 = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + ((off + t0) * a.h_kv + g) * D);

  // Q^T as the B operand, as in split_kv_mfma.
  bf16x8 qop[KS];
  {
    const __bf16* qrow =
        static_cast<const __bf16*>(a.q) + (((int64_t)b * a.s_q + qi) * a.h_q + g * NREP + hh) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (col) u = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qop[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const int lim = S - a.s_q + qi;                   // last position column n attends (causal)
  const int lim0 = S - a.s_q + tile * a.tpt;        // the tile's smallest limit (its first token's)
  const bool causal = a.s_q > 1;

  f32x4 acc[1][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  SoftmaxState st{-INFINITY, 0.f};

  const int nblk = (ntok >> 5) + ((ntok & 31) != 0);

  // This thread's pieces of a block: piece p = tid + i*THREADS is row
  // (p / RP) % 32 of K (p < 32*RP) or V, bytes 16*(p % RP); rows at or past
  // the block's valid count are clamped to its last valid row (masked in the
  // softmax).
  uint4 stage[PPT];
  auto gload = [&](int bk) {
    const int nv = min(32, ntok - bk * 32);
    const char* kb = kb0 + (int64_t)bk * 32 * row_bytes;
    const char* vb = vb0 + (int64_t)bk * 32 * row_bytes;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * THREADS;
      const int r = min((p / L::RP) % 32, nv - 1), pc = p % L::RP;
      stage[i] = load_stream16((p < 32 * L::RP ? kb : vb) + (uint32_t)r * row_bytes + 16 * pc);
    }
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * L::BYTES;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * THREADS;
      const int r = (p / L::RP) % 32, pc = p % L::RP;
      char* dst = p < 32 * L::RP ? base + r * L::KROW + 16 * pc : base + L::KBYTES + r * L::VROW + 16 * pc;
      *reinterpret_cast<uint4*>(dst) = stage[i];
    }
  };
  auto compute = [&](int buf, int bk) {
    const char* base = lds + buf * L::BYTES;
    KVRegs<D> r;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        r.k[x][kk] = *reinterpret_cast<const uint4*>(base + (16 * x + n) * L::KROW + 16 * grp + 64 * kk);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const char* vp = base + L::KBYTES + slot_token(grp, j) * L::VROW + 2 * NT * n;
      if constexpr (VW == 4) {
        const uint4 u = *reinterpret_cast<const uint4*>(vp);
        r.v[j][0] = u.x; r.v[j][1] = u.y; r.v[j][2] = u.z; r.v[j][3] = u.w;
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(vp);
        r.v[j][0] = u.x; r.v[j][1] = u.y;
      }
    }
    const int nv = min(32, ntok - bk * 32);
    const int nvl = causal ? min(nv, lim - ((int)t0 + bk * 32) + 1) : nv;
    // The causal mask matters only in blocks past the tile's first token's limit.
    const bool mask = nv < 32 || (causal && (int)t0 + bk * 32 + nv - 1 > lim0);
    bf16x8 ph[1], pl[1];
    softmax_block<D>(r, qop, acc[0], st, a.scale_log2, grp, mask, nvl, ph[0], pl[0]);
    pv_block<D, 1>(r, acc, ph, pl);
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int bk = 0; bk < nblk; ++bk) {
    const bool more = bk + 1 < nblk;               // uniform over the workgroup
    if (more) gload(bk + 1);
    if (has_tile) compute(bk & 1, bk);
    if (more) {
      lstore((bk + 1) & 1);
      __syncthreads();                              // the next block is staged; this one is read
    }
  }
  __syncthreads();                                  // the staging buffers become the epilogue's

  // Write the tiles' triplets (or o / l) through LDS, 4 floats per thread and step.
  float* sm_o = reinterpret_cast<float*>(lds);      // [TW][16][OP]
  const float l = sum_x32(sum_x16(st.l));
  if (grp == 0) {
    sm_m[w][n] = st.m;
    sm_l[w][n] = l;
  }
  if (n < cols) {
    // lane (grp, n) holds o[column n][NT*(4*grp + r) + nt]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm_o[(w * 16 + n) * OP + NT * (4 * grp + r) + nt] = acc[0][nt][r];
  }
  __syncthreads();
  for (int idx = tid; idx < TW * cols * Q4; idx += THREADS) {
    const int ww = idx / (cols * Q4), h = (idx / Q4) % cols, d4 = (idx % Q4) * 4;
    const int cqi = (pass * TW + ww) * a.tpt + h / NREP;
    if (pass * TW + ww >= a.qtiles || cqi >= a.s_q) continue;
    const float4 o = *reinterpret_cast<const float4*>(sm_o + (ww * 16 + h) * OP + d4);
    const float M = sm_m[ww][h], Lsum = sm_l[ww][h];
    const int64_t orow = ((int64_t)b * a.s_q + cqi) * a.h_q + g * NREP + h % NREP;   // (b, token, head)
    if (a.direct) {                                 // the sequence's only chunk: out = o / l here
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;   // L = 0: nothing attended (a causal column)
      const float4 rr = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      if (a.out_bf16)
        store4<__bf16>(static_cast<__bf16*>(a.out) + orow * D + d4, rr);
      else
        store4<float>(static_cast<float*>(a.out) + orow * D + d4, rr);
    } else {
      const int64_t row = orow * a.n_splits + s;
      *reinterpret_cast<float4*>(a.ws_o + row * D + d4) = o;
      if (d4 == 0) a.ws_ml[row] = make_float2(M, Lsum);
    }
  }
}

}  // namespace gqa
