// Multi-token split-KV partial attention with each K/V block shared by the
// waves of a workgroup through LDS.
//
// With several query tokens per sequence, the (query token, head) columns of
// a kv head fill ceil(S_q * n_rep / 16) tiles of 16 MFMA columns. Here each
// of the workgroup's 8 waves owns one tile, and the workgroup stages every
// 32-token K/V block of its chunk in LDS once for all 8: each wave computes
// its tile against the staged block with split_kv_mfma's score layout and
// softmax (the lazy reference of softmax_update, as the triplets of a
// multi-token call stay inside the library), reading the operands from LDS
// instead of HBM (V^T through the transposing read below; the output tiles
// are then 16 consecutive dimensions). So HBM delivers each K/V byte once per 8
// tiles (split_kv_mfma with two tiles per workgroup reads it once per 2, and
// a long sequence's passes then miss in the caches), and a wave holds one
// tile's state and no prefetch buffer (128 registers: two workgroups, 16 waves,
// per CU). Each wave's state covers the whole chunk, so the workgroup writes
// one triplet per (query token, head) of its tiles, or o / l when the
// sequence has one chunk.
//
// TPW = 2: each wave carries two tiles (tiles w and w + 8 of the workgroup's
// 16), with their own softmax states and accumulators; the block's K and V^T
// operands are read from LDS once for both, and the two tiles' independent
// softmax chains give the wave work to interleave with the other's matrix
// products. Twice the state takes about 200 registers: one workgroup (8
// waves) per CU.
//
// Staging: two LDS buffers in turn. While the waves compute block i from one
// buffer, each thread has its pieces of block i + 1 in flight from HBM to
// registers; it stores them into the other buffer afterwards, and one
// workgroup barrier per block orders the two. K rows are padded by 16 bytes
// in LDS, so the 16 lanes of a lane group, which read the same columns of 16
// different rows, hit 16 different bank groups.
//
// V^T operands come straight from LDS through gfx950's transposing read
// (ds_read_b64_tr_b16): in each 16-lane group the lanes' 8-byte reads form a
// 4 x 16 matrix of 16-bit values, 4 lanes per row, and lane i receives its
// column i. With row r = token 4*grp + r (+ 16) and the 16 columns = 16
// consecutive dimensions, lane (grp, n) receives dimension n of the tile's
// 16 at the 4 tokens of its operand slots, which is the MFMA A operand of
// O^T = V^T P^T with no byte permutes (split_kv_mfma forms it with 32
// permutes per block from whole-row loads). V rows are padded by 32 bytes so
// that the 4 rows a lane group reads fall in different banks.
#pragma once

#include "split_kv_mfma.h"

namespace gqa {

constexpr int kTileWaves = 8;                       // waves (= tiles) per workgroup
constexpr int kTilePairs = 2 * kTileWaves;          // tiles per workgroup at two per wave

template <int D>
struct LdsBlock {
  static constexpr int ROW = D * 2;                 // bytes of one head's K (or V) row
  static constexpr int KROW = ROW + 16;             // padded K row in LDS
  static constexpr int VROW = ROW + 32;             // padded V row (transposing reads)
  static constexpr int KBYTES = 32 * KROW;
  static constexpr int BYTES = KBYTES + 32 * VROW;  // one staged block
  static constexpr int RP = ROW / 16;               // 16-byte pieces per row
  static constexpr int PIECES = 2 * 32 * RP;        // pieces of a block's K and V rows
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// 8 bytes through the transposing LDS read (see above); p points into LDS.
__device__ __forceinline__ s16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
}

template <int D, int NREP, int TPW = 1>
__global__ __launch_bounds__(64 * kTileWaves) __attribute__((amdgpu_waves_per_eu(TPW == 1 ? 4 : 2)))
void split_kv_tiles(SplitArgs a) {
  static_assert(TPW == 1 || TPW == 2, "one or two tiles per wave");
  constexpr int NT = MfmaTile<D>::NT, KS = MfmaTile<D>::KS;
  constexpr int TW = kTileWaves, THREADS = 64 * TW;
  constexpr int TPG = TW * TPW;                     // tiles of a workgroup (one pass)
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

  const WgCoord wc = a.heads_fastest ? WgCoord{(int)blockIdx.y, (int)blockIdx.x, (int)blockIdx.z} : wg_coord();
  const int s = wc.s, g = wc.g;
  const int zb = wc.b / a.passes, pass = wc.b - zb * a.passes;
  int b = zb;                                       // the sequence (batch slot zb runs it)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, n = lane & 15;
  const int ti = n / NREP, hh = n % NREP;
  int tile[TPW], qi[TPW];                           // this wave's tiles of the sequence
  bool col[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    tile[t] = pass * TPG + t * TW + w;
    qi[t] = tile[t] * a.tpt + ti;                   // column n: query token qi, head g*NREP + hh
    col[t] = tile[t] < a.qtiles && ti < a.tpt && qi[t] < a.s_q;
  }
  const bool has_tile = tile[0] < a.qtiles;         // a wave's second tile comes after every first one
  const int cols = NREP * a.tpt;                    // columns in use (<= 16)

  int S;
  int64_t off;
  if (a.ranked)
    seq_info_ranked(a.seq_lens, a.kv_off, a.ranked, zb, lane, b, S, off);
  else
    seq_info(a.seq_lens, a.kv_off, b, lane, S, off);
  S = __builtin_amdgcn_readfirstlane(S);
  off = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)off));
  int c, n_active;
  chunking(S, a.n_splits, a.min_chunk, c, n_active);
  if (s >= n_active) {                              // the merge reads chunks < n_active only
    if (a.direct && n_active == 0 && s == 0) {      // nothing attended: out = 0
      for (int idx = tid; idx < TPG * cols * Q4; idx += THREADS) {
        const int t = pass * TPG + idx / (cols * Q4), h = (idx / Q4) % cols;
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
  bf16x8 qop[TPW][KS];
  int lim[TPW], lim0[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const __bf16* qrow =
        static_cast<const __bf16*>(a.q) + (((int64_t)b * a.s_q + qi[t]) * a.h_q + g * NREP + hh) * D + 8 * grp;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (col[t]) u = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qop[t][kk] = __builtin_bit_cast(bf16x8, u);
    }
    lim[t] = S - a.s_q + qi[t];                     // last position column n attends (causal)
    lim0[t] = S - a.s_q + tile[t] * a.tpt;          // the tile's smallest limit (its first token's)
  }
  const bool causal = a.s_q > 1;
  // The largest limit among the wave's query tokens: a block that starts
  // past it is masked for every column of the wave, which skips it (the
  // upper triangle of a prefill-sized call; its state stays as it was).
  int lim_hi = -1;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
    if (tile[t] < a.qtiles) lim_hi = max(lim_hi, S - a.s_q + min(tile[t] * a.tpt + a.tpt, a.s_q) - 1);

  f32x4 acc[TPW][NT];
  SoftmaxState st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[t] = SoftmaxState{-INFINITY, 0.f};
  }

  const int nblk = (ntok >> 5) + ((ntok & 31) != 0);

  // This thread's pieces of a block: piece p = tid + i*THREADS is row
  // (p / RP) % 32 of K (p < 32*RP) or V, bytes 16*(p % RP); rows at or past
  // the block's valid count are clamped to its last valid row (masked in the
  // softmax).
  uint4 stage[PPT];
  uint32_t goff[PPT], loff[PPT];                    // a piece's byte offset in a full block / in LDS
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = tid + i * THREADS;
    const int r = (p / L::RP) % 32, pc = p % L::RP;
    goff[i] = (uint32_t)r * row_bytes + 16 * pc;
    loff[i] = p < 32 * L::RP ? r * L::KROW + 16 * pc : L::KBYTES + r * L::VROW + 16 * pc;
  }
  auto gload = [&](int bk) {
    const int nv = min(32, ntok - bk * 32);
    const char* kb = kb0 + (int64_t)bk * 32 * row_bytes;
    const char* vb = vb0 + (int64_t)bk * 32 * row_bytes;
    if (nv == 32) {                                 // every block but a chunk's partial last one
#pragma unroll
      for (int i = 0; i < PPT; ++i) stage[i] = load_stream16((tid + i * THREADS < 32 * L::RP ? kb : vb) + goff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int p = tid + i * THREADS;
        const int r = min((p / L::RP) % 32, nv - 1), pc = p % L::RP;
        stage[i] = load_stream16((p < 32 * L::RP ? kb : vb) + (uint32_t)r * row_bytes + 16 * pc);
      }
    }
  };
  auto lstore = [&](int buf) {
    char* base = lds + buf * L::BYTES;
#pragma unroll
    for (int i = 0; i < PPT; ++i) *reinterpret_cast<uint4*>(base + loff[i]) = stage[i];
  };
  // This lane's LDS offsets: K rows n (+ 16) at bytes 16*grp (+ 64*kk); the
  // transposing V reads at row 4*grp + n/4 (+ 16), bytes 8*(n%4) (+ 32*nt).
  const uint32_t kofs = n * L::KROW + 16 * grp;
  const uint32_t vofs = L::KBYTES + (4 * grp + n / 4) * L::VROW + 8 * (n % 4);
  auto compute = [&](int buf, int bk) {
    const char* base = lds + buf * L::BYTES;
    KVRegs<D> r;                                    // K only (V^T below)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        r.k[x][kk] = *reinterpret_cast<const uint4*>(base + kofs + 16 * x * L::KROW + 64 * kk);
    const int nv = min(32, ntok - bk * 32);
    bool mask[TPW];
    int nvl[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      nvl[t] = causal ? min(nv, lim[t] - ((int)t0 + bk * 32) + 1) : nv;
      // The causal mask matters only in blocks past the tile's first token's limit.
      mask[t] = nv < 32 || (causal && (int)t0 + bk * 32 + nv - 1 > lim0[t]);
    }
    // The scores first (the K registers are free once the products have
    // read them), then the V^T operands of output tile nt: dimension
    // 16*nt + n at tokens 4*grp + 0..3 and 16 + 4*grp + 0..3 (the slots of the
    // P^T operand).
    float x[TPW][8];
#pragma unroll
    for (int t = 0; t < TPW; ++t) tile_scores<D>(r, qop[t], a.scale_log2, x[t]);
    auto v_operand = [&](int nt) {
      const s16x4_t lo = lds_read_tr16(base + vofs + 32 * nt);
      const s16x4_t hi = lds_read_tr16(base + vofs + 16 * L::VROW + 32 * nt);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // Two tiles per wave read all of V^T before the softmax (its latency
    // hidden behind the softmax); one tile per wave reads each output tile's
    // V^T just before its products, 11 fewer registers (32k tokens, S_q =
    // 16, µs per call: 59.9 / 57.8 -> 54.7 / 52.7; the same order with two
    // tiles per wave measured 48.3 -> 49.9 at 16k, S_q = 32).
    bf16x8 vt[TPW == 2 ? NT : 1];
    if constexpr (TPW == 2) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vt[nt] = v_operand(nt);
    }
    bf16x8 ph[TPW], pl[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const float mb = block_max(x[t], grp, mask[t], nvl[t]);
      softmax_update<D, true>(x[t], mb, acc[t], st[t], ph[t], pl[t]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bf16x8 v = TPW == 2 ? vt[nt] : v_operand(nt);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, ph[t], acc[t][nt], 0, 0, 0);
        acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pl[t], acc[t][nt], 0, 0, 0);
      }
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int bk = 0; bk < nblk; ++bk) {
    const bool more = bk + 1 < nblk;               // uniform over the workgroup
    if (more) gload(bk + 1);
    if (has_tile && !(causal && (int)t0 + bk * 32 > lim_hi)) compute(bk & 1, bk);
    if (more) {
      lstore((bk + 1) & 1);
      __syncthreads();                              // the next block is staged; this one is read
    }
  }
  // Write the tiles' triplets (or o / l) through LDS, 4 floats per thread and
  // step, the waves' t-th tiles in round t.
  float* sm_o = reinterpret_cast<float*>(lds);      // [TW][16][OP]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
  __syncthreads();                                  // the staging buffers (or the last round's) are free
  const float l = sum_x32(sum_x16(st[t].l));
  if (grp == 0) {
    sm_m[w][n] = st[t].m;
    sm_l[w][n] = l;
  }
  if (n < cols) {
    // lane (grp, n) holds o[column n][16*nt + 4*grp + r]
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sm_o[(w * 16 + n) * OP + 16 * nt + 4 * grp + r] = acc[t][nt][r];
  }
  __syncthreads();
  for (int idx = tid; idx < TW * cols * Q4; idx += THREADS) {
    const int ww = idx / (cols * Q4), h = (idx / Q4) % cols, d4 = (idx % Q4) * 4;
    const int ct = pass * TPG + t * TW + ww;        // the tile of wave ww's round-t state
    const int cqi = ct * a.tpt + h / NREP;
    if (ct >= a.qtiles || cqi >= a.s_q) continue;
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
}

}  // namespace gqa
