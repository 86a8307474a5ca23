// Host side of the decode attention library: argument checks, split
// heuristic, workspace, kernel selection and launches. C ABI in gqa_decode.h.
#include "gqa_decode.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "gqa_common.h"
#include "fused_tail.h"
#include "kv_append.h"
#include "merge.h"
#include "packed_offsets.h"
#include "split_kv_mfma.h"
#include "split_kv_tiles.h"
#include "split_kv_valu.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_before = nullptr, g_ev_after = nullptr;
std::atomic<unsigned long long> g_call_tag{1};   // tags of single-launch calls (48 bits used)

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

// Heuristic constants (see gqa_decode_pick_splits).
constexpr int kMinChunk = 128;       // tokens: one 32-token block per wave of a workgroup
constexpr int kBlockTokens = 32;     // one block: the shortest chunk of a single short sequence
constexpr int kNoHintRounds = 4;     // rounds of resident workgroups a call without a length hint plans for
// How a split kernel wants its grid: resident workgroups per CU, rounds of
// those slots the longest sequence's chunks fill (one sequence / a batch, where
// only the longest length is known and more rounds keep it balanced), and the
// longest chunk in tokens. Measured per kernel at 70B shapes.
struct SplitPolicy {
  int wg_per_cu;
  int rounds_one, rounds_many;
  int64_t max_chunk;
  bool eight_wave;              // a single sequence may take one 8-wave workgroup per CU
  bool short_one;               // short sequences, B <= 4: chunks down to one block (single token)
  // > 0: a single sequence in one pass whose chunks, at one workgroup per CU,
  // hold at most this many tokens takes that one round instead of wg_per_cu
  // workgroups per CU (half the triplets to store and merge)
  int64_t one_per_cu_max_chunk = 0;
};
// One 16-column tile per workgroup, two workgroups per CU, one query token. A
// second round hides each workgroup's start-up behind another's streaming.
constexpr SplitPolicy kOneTile{2, 2, 4, 4096, true, true};
// The same without the 8-wave form: head size 64, where 4-wave workgroups
// fit three per CU and measured faster.
constexpr SplitPolicy kOneTile64{2, 2, 4, 4096, false, true};
// One tile of several query tokens (multi-token calls).
constexpr SplitPolicy kOneTileMulti{2, 2, 4, 4096, false, false};
// The same with 128-dimension heads: a single sequence may take the 8-wave
// round like a single-token call (one tile of several query tokens, e.g. two
// at 70B shapes: 8k 13.8 -> 12.5 µs per call, 16k 19.5 -> 17.7, 32k 31.8 ->
// 27.8; with the round up to 2048-token chunks, 40k 37.2 -> 32.8, 64k 54.1
// -> 49.4).
constexpr SplitPolicy kOneTileMulti8{2, 2, 4, 4096, true, false};
// Two tiles per workgroup (multi-token decode), one workgroup per CU: one
// round for a single sequence; chunks up to 16384 tokens.
constexpr SplitPolicy kTwoTiles{1, 1, 4, 16384, false, false};
// One tile per wave, eight per workgroup (multi-token decode), two workgroups
// per CU: one round for a single sequence, up to two for a batch (ragged
// B = 8, S_q = 16: 209.9 µs at two rounds, 227.9 at four).
constexpr SplitPolicy kTileWavesPolicy{2, 1, 2, 16384, false, false, 768};
// Two tiles per wave, sixteen per workgroup, one workgroup per CU.
constexpr SplitPolicy kTilePairsPolicy{1, 1, 2, 16384, false, false};

// single_token: a single-token entry point. The multi-token one takes the
// 8-wave count for one tile of several query tokens with 128-dimension heads
// (so its split count depends on d_head: gqa_decode_multi_splits_d), and the
// short-sequence count only for one query token, where it then plans like a
// single-token call outside the 8-wave range.
const SplitPolicy& split_policy(int tiles_per_wg, int d_head, bool single_token, int s_q) {
  if (tiles_per_wg == gqa::kTileWaves) return kTileWavesPolicy;
  if (tiles_per_wg == gqa::kTilePairs) return kTilePairsPolicy;
  if (tiles_per_wg == 2) return kTwoTiles;
  if (single_token && d_head == 128) return kOneTile;
  if (!single_token && s_q > 1 && d_head == 128) return kOneTileMulti8;
  return single_token || s_q == 1 ? kOneTile64 : kOneTileMulti;
}
// A single sequence with 128-dimension heads whose chunks, at one 8-wave
// workgroup per CU, hold this many tokens (each wave one to eight 32-token
// blocks) takes that form: measured faster at 70B shapes from 8k to 32k
// tokens (and at 1 to 16 kv heads in the same chunk range), slower below
// (waves without a block), and slower with 64-dimension heads. Up to 2048
// tokens per chunk (64k tokens at 8 kv heads; µs per call p50, two rounds of
// 4-wave workgroups vs one of 8-wave: 40k 32.98 vs 32.54, 64k 50.44 vs
// 48.88); above that two rounds of 4-wave workgroups balance better (128k
// 88.74 vs 90.79, 256k 168.36 vs 170.37; 1M 657.66 vs 648.66 is the
// exception, not fitted).
constexpr int64_t kEightWaveMinChunk = 256, kEightWaveMaxChunk = 2048;

// Library-owned fallback workspace, one grow-only buffer per device.
std::mutex g_ws_mu;
std::vector<std::pair<void*, size_t>> g_ws;  // index = device ordinal

// Compute units of the current device, queried once per device ordinal.
std::atomic<int> g_cus[64];

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    const int known = g_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) {
      *cus = known;
      return GQA_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (n < 1) return fail(GQA_ERR_HIP, "device %d reports %d compute units", dev, n);
  if (dev >= 0 && dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return GQA_OK;
}

int library_workspace(size_t bytes, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1, {nullptr, 0});
  auto& slot = g_ws[dev];
  if (slot.second < bytes) {
    // Older work on any stream may still read the old buffer: wait for it.
    if (slot.first) {
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
      (void)hipFree(slot.first);
      slot = {nullptr, 0};
    }
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    slot = {p, bytes};
  }
  *ptr = slot.first;
  return GQA_OK;
}

bool valid_nrep(int r) { return r == 1 || r == 2 || r == 4 || r == 8 || r == 16; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Workspace layout, 256-byte aligned parts: arrival counters [B * h_kv] (room
// for B * h_q) uint64 at 0, so their place does not depend on the split
// count; o [B, h_q, n, d] fp32 at o_off; (m, l) [B, h_q, n] fp32 at ml_off;
// packed-layout token bases [B] int64 at tok_off.
struct WsLayout {
  size_t o_off, ml_off, tok_off, total;
};
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
WsLayout ws_layout(int B, int h_q, int d, int n) {
  const size_t rows = (size_t)B * h_q * n;
  WsLayout l;
  l.o_off = round256((size_t)B * h_q * sizeof(unsigned long long));
  l.ml_off = l.o_off + round256(rows * d * sizeof(float));
  l.tok_off = l.ml_off + round256(rows * sizeof(float2));
  l.total = l.tok_off + round256((size_t)B * sizeof(int64_t));
  return l;
}

// Above this many sequences a packed-layout call computes the token bases
// with one scan launch instead of inside every split workgroup.
constexpr int kScanMinBatch = 256;
// Chunks of at most this many tokens (by the length hint) run in one-wave
// workgroups when there are enough of them: a 4-wave workgroup gives each
// wave 32-token blocks of the chunk, so shorter chunks leave waves without
// work, and one-wave workgroups fit four times as many chunks on a CU
// (measured faster up to 128 tokens).
constexpr int kOneWaveMaxTokens = 128;
size_t ws_bytes(int B, int h_q, int d, int n) { return ws_layout(B, h_q, d, n).total; }

// ---------------------------------------------------------------- launches
// Workgroup form of the matrix-core split kernel.
// kTiles / kTilePairs: the multi-token kernel with one / two query tiles per
// wave (split_kv_tiles).
enum class Form { kFourWave, kOneWave, kEightWave, kTiles, kTilePairs };

template <int D, int NREP>
hipError_t launch_split(bool bf16, bool valu, Form form, dim3 grid, hipStream_t st, const gqa::SplitArgs& a) {
  if (!bf16) {
    hipLaunchKernelGGL((gqa::split_kv_valu<float, D, NREP>), grid, dim3(gqa::kThreads), 0, st, a);
  } else if (valu) {
    hipLaunchKernelGGL((gqa::split_kv_valu<__bf16, D, NREP>), grid, dim3(gqa::kThreads), 0, st, a);
  } else if (form == Form::kTiles) {
    hipLaunchKernelGGL((gqa::split_kv_tiles<D, NREP>), grid, dim3(64 * gqa::kTileWaves), 0, st, a);
  } else if (form == Form::kTilePairs) {
    hipLaunchKernelGGL((gqa::split_kv_tiles<D, NREP, 2>), grid, dim3(64 * gqa::kTileWaves), 0, st, a);
  } else if (a.qtiles > a.passes) {               // two column tiles per workgroup
    if (form == Form::kEightWave)
      hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, false, 2, 8>), grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, false, 2>), grid, dim3(gqa::kThreads), 0, st, a);
  } else if (form == Form::kOneWave) {
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, false, 1, 1>), grid, dim3(64), 0, st, a);
  } else if (form == Form::kEightWave) {
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, false, 1, 8>), grid, dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP>), grid, dim3(gqa::kThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split_nrep(int nrep, bool bf16, bool valu, Form form, dim3 grid, hipStream_t st,
                             const gqa::SplitArgs& a) {
  switch (nrep) {
    case 1: return launch_split<D, 1>(bf16, valu, form, grid, st, a);
    case 2: return launch_split<D, 2>(bf16, valu, form, grid, st, a);
    case 4: return launch_split<D, 4>(bf16, valu, form, grid, st, a);
    case 8: return launch_split<D, 8>(bf16, valu, form, grid, st, a);
    default: return launch_split<D, 16>(bf16, valu, form, grid, st, a);
  }
}

template <int D, int NREP>
void launch_append_form(Form form, dim3 grid, hipStream_t st, const gqa::SplitArgs& a) {
  if (form == Form::kOneWave)
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, true, 1, 1>), grid, dim3(64), 0, st, a);
  else if (form == Form::kEightWave)
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, true, 1, 8>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((gqa::split_kv_mfma<D, NREP, true>), grid, dim3(gqa::kThreads), 0, st, a);
}

template <int D>
hipError_t launch_split_append(int nrep, Form form, dim3 grid, hipStream_t st, const gqa::SplitArgs& a) {
  switch (nrep) {
    case 1: launch_append_form<D, 1>(form, grid, st, a); break;
    case 2: launch_append_form<D, 2>(form, grid, st, a); break;
    case 4: launch_append_form<D, 4>(form, grid, st, a); break;
    case 8: launch_append_form<D, 8>(form, grid, st, a); break;
    default: launch_append_form<D, 16>(form, grid, st, a); break;
  }
  return hipGetLastError();
}

// Rows from which merge_wave takes two 32-column slices per wave (half the
// waves: a multi-token call's 4096 rows then fit the wave slots in one
// round). 70B B = 1, µs per call p50, two interleaved A/B runs of 9 rounds,
// one slice vs two (the same bits): 8k S_q = 64 44.7 / 44.7 vs 43.4 / 44.0,
// S_q = 32 31.4 / 31.0 vs 31.0 / 30.5; 32k S_q = 16 52.6 / 52.5 vs 52.1 /
// 51.3, S_q = 64 119.5 / 118.0 vs 117.1 / 117.5. One wave per row (four
// slices) measured the same as two. Calls with few rows keep one slice per
// wave (more waves, each with less to load): one query token, 64 rows, 8k
// 11.84 vs 11.99 (two slices) and 12.19 (four), 16k 16.77 vs 17.06 / 16.98.
constexpr int64_t kMergeWideRows = 1024;
// Split counts that merge_wave merges (one workgroup per row, which is what
// MergeArgs::xcd_rep remaps).
constexpr int kMergeWaveMinSplits = 9, kMergeWaveMaxSplits = 32;

template <int D, typename TO>
hipError_t launch_merge_t(int rows, hipStream_t st, const gqa::MergeArgs& a) {
  // Up to 8 chunks per row: several rows per workgroup (32 / SPR of them).
  auto packed = [&](auto spr) {
    constexpr int SPR = decltype(spr)::value;
    if (rows >= kMergeWideRows) {
      // A lane holds its chunk's whole row (D / 32 float4s), a quarter of
      // the workgroups. 70B B = 1, µs per call p50, 9 interleaved rounds, one
      // / two / four float4s per lane (the same bits): 8k S_q = 128 72.8 /
      // 71.4 / 70.6; 4k S_q = 256 73.1 / 71.9 / 71.6; 2.5k S_q = 512 84.3 /
      // 83.7 / 84.0; 1k S_q = 1024 62.6 / 62.6 / 62.5; one query token, B =
      // 32 x 4k and 64 x 2k 95.1 / 95.0 / 94.9 and 98.0 / 97.3 / 97.3.
      constexpr int SL = D / 32;
      const dim3 g((unsigned)((rows + 32 / SPR - 1) / (32 / SPR)), D / (32 * SL));
      hipLaunchKernelGGL((gqa::merge_rows<D, TO, SPR, SL>), g, dim3(256), 0, st, a, rows);
      return;
    }
    const dim3 g((unsigned)((rows + 32 / SPR - 1) / (32 / SPR)), D / 32);
    hipLaunchKernelGGL((gqa::merge_rows<D, TO, SPR>), g, dim3(256), 0, st, a, rows);
  };
  if (a.n_splits <= 8) {
    if (a.n_splits == 1) packed(std::integral_constant<int, 1>{});
    else if (a.n_splits == 2) packed(std::integral_constant<int, 2>{});
    else if (a.n_splits <= 4) packed(std::integral_constant<int, 4>{});
    else packed(std::integral_constant<int, 8>{});
    return hipGetLastError();
  }
  // Up to 32 chunks: one wave per 32-column slice, D / 32 waves per row
  // (measured faster than the workgroup-per-slice merge up to 32 chunks,
  // slower at 64).
  if (a.n_splits <= kMergeWaveMaxSplits) {
    const dim3 g((unsigned)rows);
    if (rows >= kMergeWideRows) {
      const dim3 blk(64 * (D / 64));
      if (a.n_splits <= 16)
        hipLaunchKernelGGL((gqa::merge_wave<D, TO, 2, 2>), g, blk, 0, st, a);
      else
        hipLaunchKernelGGL((gqa::merge_wave<D, TO, 4, 2>), g, blk, 0, st, a);
      return hipGetLastError();
    }
    const dim3 blk(64 * (D / 32));
    if (a.n_splits <= 16)
      hipLaunchKernelGGL((gqa::merge_wave<D, TO, 2>), g, blk, 0, st, a);
    else
      hipLaunchKernelGGL((gqa::merge_wave<D, TO, 4>), g, blk, 0, st, a);
    return hipGetLastError();
  }
  // One workgroup per row and 32-column slice; chunks per slot in the first
  // round: one round covers up to 32 * U chunks.
  const dim3 grid((unsigned)rows, D / 32);
  if (a.n_splits <= 64)
    hipLaunchKernelGGL((gqa::merge_splits<D, TO, 2>), grid, dim3(256), 0, st, a);
  else if (a.n_splits <= 128)
    hipLaunchKernelGGL((gqa::merge_splits<D, TO, 4>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gqa::merge_splits<D, TO, 8>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge(bool out_bf16, int B, int h_q, hipStream_t st, const gqa::MergeArgs& a) {
  const int64_t rows = (int64_t)B * h_q;
  return out_bf16 ? launch_merge_t<D, __bf16>((int)rows, st, a) : launch_merge_t<D, float>((int)rows, st, a);
}

// Multi-token calls whose sequences need this many query tiles, over at
// least this many tokens in all (B times the longest length), take the
// tile-per-wave kernel (split_kv_tiles: 8 or 16 tiles read each K/V block
// once, through LDS); others take two tiles per workgroup (split_kv_mfma),
// faster at fewer tiles and at shorter KV, where its repeated passes over the
// KV hit in the caches. Measured at 70B shapes, µs per call, two-tile vs
// one-tile-per-wave kernel: S = 8k, S_q = 16: 29.1 vs 31.9; 16k: 46.5 vs
// 41.6; 32k: 84.4 vs 65.8; 64k, S_q = 8 / 16 / 64: 92.7 / 163 / 579 vs 81.8 /
// 119.5 / 369; 16k, S_q = 8: 30.8 vs 32.5; ragged B = 8, S_q = 4 / 8 / 16:
// 108.7 / 179.9 / 294.6 vs 123.1 / 155.2 / 209.9. At the thresholds, after
// the two-tile kernel's K loads got faster: S_q = 16, 16383 vs 16384 tokens:
// 43.7 vs 42.1; S_q = 8, 65535 vs 65536: 85.6 vs 74.2.
constexpr int kTilesMinTiles = 8;
constexpr int64_t kTilesMinTokens = 16384;
// One sequence of 8 to 15 tiles takes it from 4096 tokens (8 tiles in one
// workgroup per CU, by the split rule below): 70B, S_q = 16, µs per call,
// tile-per-wave vs two-tile kernel: 4k 17.0 vs 18.1, 6k 19.6 vs 21.3, 8k 22.1
// vs 24.2, 9k 23.2 vs 25.8, 12k 26.8 vs 29.9, 15k 30.5 vs 35.1. Batches stay at 16384
// tokens (B = 2 x 4k 26.0 vs 24.0, ragged 4 x 1k-4k 45.6 vs 41.9), and
// shorter sequences on two tiles (1k 15.1 vs 12.9, 2k 15.9 vs 14.8; about
// even at 3k, 16.6 vs 17.0).
constexpr int64_t kTilesMinTokensOne = 4096;
constexpr int kTilesMinTilesLong = 4;          // fewer tiles take it only over longer KV
constexpr int64_t kTilesMinTokensLong = 65536;
// 12 or more tiles from 8192 tokens (after the whole-round split rule): 70B
// B = 1, 8k tokens, µs per call, tile-per-wave vs two-tile kernel: S_q = 24
// (12 tiles) 28.4 vs 30.7, S_q = 31 (16) 33.3 vs 36.5, S_q = 48 (24) 43.3 vs
// 53.6.
constexpr int kTilesMinTilesMid = 12;
constexpr int64_t kTilesMinTokensMid = 8192;
// 9 to 15 tiles (one per wave) from 4096 tokens, since the tile-per-wave
// kernel reads its V^T operands per output tile: 70B B = 1, µs per call,
// tile-per-wave vs two-tile kernel: 8k tokens, S_q = 18 (9 tiles) 24.1 vs
// 28.3, S_q = 20 (10) 24.9 vs 28.7; 4k, S_q = 18 18.6 vs 20.9, S_q = 24 (12)
// 21.1 vs 22.8. (8 tiles: the one-sequence rule above; with 64 chunks, two
// workgroups per CU, they lost at 8k, 30.0 vs 24.5.)
constexpr int kTilesMinTilesLow = 9;
constexpr int64_t kTilesMinTokensLow = 4096;
// 5 to 7 tiles from 32768 tokens (the two-tile kernel's 3 or 4 passes drift
// apart over long KV): 70B B = 1, 32k tokens, µs per call, tile-per-wave vs
// two-tile kernel: S_q = 10 46.6 vs 51.3, S_q = 12 50.2 vs 51.8, S_q = 14
// 52.4 vs 62.5; 4 tiles stay on two tiles up to 65536 tokens (32k S_q = 8:
// 43.7 vs 38.5; 48k 55.7 vs 52.9), and so do 5 to 7 tiles at 16k (S_q = 12:
// 35.5 vs 31.6).
constexpr int kTilesMinTilesFew = 5;
constexpr int64_t kTilesMinTokensFew = 32768;
// Calls that take the tile-per-wave kernel with at least this many tiles per
// sequence carry two tiles per wave (half the LDS reads per tile, one pass of
// 16 tiles instead of two of 8). 70B B = 1, µs per call, two tiles per wave
// vs one: 8k tokens S_q = 64 47.8 vs 50.1, S_q = 128 73.8 vs 81.3; 16k S_q =
// 32 52.0 vs 53.2, S_q = 48 70.7 vs 98.6; 32k S_q = 32 80.8 vs 86.3, S_q =
// 64 127.0 vs 144.7; 64k S_q = 32 134.7 vs 151.4.
constexpr int kTilePairsMinTiles = 16;
// Such calls (chunked-prefill sizes) take it once tiles x tokens reaches
// this. 70B B = 1, µs per call, two tiles per wave vs the two-tile kernel:
// 2^18 and above: 512 tokens S_q = 1024 42.1 vs 89.3; 1k S_q = 512 51.8 vs
// 74.2, S_q = 1024 67.7 vs 138.1; 2k S_q = 256 51.4 vs 63.8, S_q = 512 77.8
// vs 124.4; 2.5k S_q = 512 86.8 vs 138.5; 4k S_q = 128 53.1 vs 59.5, S_q =
// 256 77.7 vs 111.8; 8k S_q = 64 47.8 vs 64.8. Below: 1k S_q = 64 29.0 vs
// 18.2; 2k S_q = 32 27.1 vs 18.3, S_q = 128 39.2 vs 33.9; 8k S_q = 32 39.0
// vs 37.6 (4k S_q = 64: 36.6 vs 38.1, near even).
constexpr int64_t kTilesMinWork = int64_t(1) << 18;

// Query tokens per 16-column tile, tiles per sequence, tiles per workgroup
// (two once a sequence needs two or more, each K/V block then read once for
// both; kTileWaves / kTilePairs for the tile-per-wave kernel with one / two
// tiles per wave) and workgroup passes per sequence over the KV range. hint:
// the longest sequence (0: unknown).
void query_tiles(int s_q, int nrep, int B, int64_t hint, int* tpt, int* qtiles, int* tpw, int* passes) {
  *tpt = s_q < 16 / nrep ? s_q : 16 / nrep;
  *qtiles = (s_q + *tpt - 1) / *tpt;
  *tpw = *qtiles >= 2 ? 2 : 1;
  const int64_t tokens = hint > 0 ? (int64_t)B * hint : 0;
  // Two tiles over short KV: one per pass (twice the workgroups, each
  // reading the KV; the second read hits the caches). 70B shapes, S_q = 4,
  // µs per call, one vs two tiles per workgroup: B = 1, 1k 8.3 vs 10.2, 2k
  // 9.2 vs 10.7, 4k 10.7 vs 12.8, 6k 11.6 vs 13.1, 8k 14.1 vs 14.3; B = 4 x
  // 2k 19.7 vs 21.4; but B = 2 x 4k 15.8 vs 15.0, and 16k or 32k tokens
  // (20.6 vs 20.6, 52.5 vs 31.6) and the ragged B = 8 batch (144.0 vs 92.0)
  // read the KV twice from HBM. Grouped heads only (measured at 8 query
  // heads per KV head; many KV heads already fill the chip).
  if (*qtiles == 2 && nrep >= 4 && hint > 0 && ((B == 1 && hint <= 8192) || (hint <= 2048 && tokens <= 8192))) *tpw = 1;
  if ((*qtiles >= kTilesMinTiles && tokens >= kTilesMinTokens) ||
      (*qtiles >= kTilesMinTiles && *qtiles < kTilePairsMinTiles && B == 1 && tokens >= kTilesMinTokensOne) ||
      (*qtiles >= kTilesMinTilesLong && tokens >= kTilesMinTokensLong) ||
      (*qtiles >= kTilesMinTilesMid && tokens >= kTilesMinTokensMid) ||
      (*qtiles >= kTilesMinTilesLow && *qtiles < kTilePairsMinTiles && tokens >= kTilesMinTokensLow) ||
      (*qtiles >= kTilesMinTilesFew && tokens >= kTilesMinTokensFew) ||
      (*qtiles >= kTilePairsMinTiles && (int64_t)*qtiles * tokens >= kTilesMinWork))
    *tpw = *qtiles >= kTilePairsMinTiles ? gqa::kTilePairs : gqa::kTileWaves;
  *passes = (*qtiles + *tpw - 1) / *tpw;
}

// full_pass: every pass's workgroups give each wave a query tile (the
// tile-per-wave kernel with a multiple of 8 tiles).
int pick_splits_host(int B, int passes, int h_kv, int64_t s_kv_max, int num_cus, const SplitPolicy& p,
                     bool full_pass = false) {
  // Enough workgroups to fill every CU at B = 1 ...
  const int64_t units = (int64_t)B * passes * h_kv;
  const int64_t slots = (int64_t)p.wg_per_cu * num_cus;
  int64_t n = (slots + units - 1) / units;
  // A grid that overshoots the slots by part of a round pays for that round
  // in full: one sequence takes the whole rounds that fit when they keep at
  // least three quarters of the slots busy (multi-token, two tiles per
  // workgroup, 70B shapes, 8k tokens, µs per call: S_q = 12, 24 units, 10
  // instead of 11 splits: 31.7 -> 21.8; S_q = 20, 40 units, 6 instead of 7:
  // 43.3 -> 27.6; S_q = 24, 48 units, 5 instead of 6: 46.5 -> 30.7; S_q =
  // 40, 80 units, 3 instead of 4: 59.5 -> 42.5; S_q = 48, 96 units, 2
  // instead of 3: 74.7 -> 53.6).
  if (B == 1 && n * units > slots && slots / units >= 1 && 4 * (slots / units) * units >= 3 * slots)
    n = slots / units;
  if (s_kv_max > 0 && B == 1 && passes == 1 && full_pass && p.one_per_cu_max_chunk > 0 &&
      num_cus / units >= 1 && s_kv_max <= p.one_per_cu_max_chunk * (num_cus / units)) {
    // ... one round of one tile-per-wave workgroup per CU (70B, µs per call,
    // S_q = 16, 64 -> 32 chunks: 16k 36.1 / 36.1 -> 32.0 / 31.5 (and 36.5
    // -> 31.7 on another box), 18k 38.1 / 38.3 / 38.1 -> 35.0 / 34.4 / 35.2,
    // 20k 41.4 / 40.7 / 40.7 -> 37.3 / 37.0 / 37.8, 24k 45.6 / 43.8 / 46.0
    // -> 42.6 / 41.9 / 41.6, S_q = 15 at 22k 40.8 / 42.0 / 42.7 -> 39.6 /
    // 39.6 / 39.3; 32k even (53.4 / 59.2 -> 57.9 / 54.8), 64k
    // better on two per CU (105.1 / 109.4 against 110.2 / 120.6); not
    // measured better with waves left without a tile, 32k S_q = 12: 47.5
    // either way, nor with two passes, 8k S_q = 20: 24.8 -> 29.6).
    return (int)(num_cus / units);
  }
  if (s_kv_max > 0 && B == 1 && p.eight_wave) {
    // ... one sequence that one round of 8-wave workgroups, one per CU,
    // covers in chunks of kEightWaveMinChunk to kEightWaveMaxChunk tokens:
    // that round (the split form picks the 8-wave kernel for it).
    const int64_t n8 = num_cus / units;
    if (n8 >= 1 && s_kv_max >= kEightWaveMinChunk * n8 && s_kv_max <= kEightWaveMaxChunk * n8) return (int)n8;
  }
  if (s_kv_max > 0 && B == 1) {
    // ... one sequence: a whole number of such rounds, up to the policy's,
    // a second one only while its chunks keep at least two blocks per wave
    // (2 * kMinChunk tokens; a length just past a multiple of the chunk must
    // not leave a few workgroups for a last, nearly empty round), and chunks
    // of at most max_chunk tokens.
    int64_t k = s_kv_max / (2 * kMinChunk * n);
    if (k > p.rounds_one) k = p.rounds_one;
    if (k < 1) k = 1;
    n *= k;
    const int64_t by_max = (s_kv_max + p.max_chunk - 1) / p.max_chunk;
    if (by_max > n) n = by_max;
  } else if (s_kv_max > 0) {
    // ... several sequences: chunks short enough that the longest one's
    // workgroups are spread over rounds of the resident slots: only the
    // longest length is known, and more rounds keep a ragged batch balanced,
    // but a batch of few sequences can only be so uneven and pays for every
    // extra round in triplets to store and merge, so B / 2 rounds, from 1 up
    // to the policy's; chunks within [kMinChunk, max_chunk] tokens.
    const int64_t rounds = std::max<int64_t>(1, std::min<int64_t>(p.rounds_many, B / 2));
    int64_t chunk = (s_kv_max * units + rounds * slots - 1) / (rounds * slots);
    if (chunk > p.max_chunk) chunk = p.max_chunk;
    if (chunk < kMinChunk) chunk = kMinChunk;
    const int64_t by_len = (s_kv_max + chunk - 1) / chunk;
    if (by_len > n) n = by_len;
  }
  if (s_kv_max > 0) {
    const int64_t cap = (s_kv_max + kMinChunk - 1) / kMinChunk;   // no chunk shorter than kMinChunk
    if (n > cap) n = cap;
  }
  if (s_kv_max <= 0 && B == 1 && p.eight_wave && p.short_one && num_cus / units >= 1) {
    // ... no length known, one sequence, one query token, 128-dimension
    // heads: one round of 8-wave workgroups, one per CU, each sizing its
    // chunk on the device (c = S / n, at least chunk_floor's). 70B, µs per
    // call p50, no hint before / after (the hinted plan): 1k 9.74 / 7.65
    // (7.28), 4k 11.37 / 9.37 (9.26), 8k 13.49 / 12.59 (12.13), 16k 20.03 /
    // 17.93 (17.11), 32k 32.97 / 28.00 (27.28), 128k 92.86 / 90.92 (90.40),
    // 1M 655.98 / 648.86 (657.66).
    return (int)(num_cus / units);
  }
  if (s_kv_max <= 0 && p.short_one) {
    // ... no length known (one query token): enough chunks for a long
    // sequence, kNoHintRounds rounds of the resident slots, with a chunk
    // floor that grows with each sequence's length on the device (see
    // make_plan), so short sequences leave most chunks empty: 70B B = 1 gets
    // 256 chunks, 4096 tokens each at 1M, 128 at 8k (64 of them non-empty).
    n *= kNoHintRounds;
  }
  if (s_kv_max > 0 && B <= 4 && p.short_one) {
    // ... except short sequences in a batch of at most 4: up to one
    // workgroup per CU while chunks keep one block (more workgroups engage
    // more CUs' memory paths, even with waves that have no block; measured
    // faster below 4k tokens, and not for larger batches).
    const int64_t n1 = std::min<int64_t>(num_cus / units, (s_kv_max + kBlockTokens - 1) / kBlockTokens);
    if (n1 > n) n = n1;
  }
  if (n < 1) n = 1;
  if (n > GQA_MAX_SPLITS) n = GQA_MAX_SPLITS;
  return (int)n;
}

}  // namespace

extern "C" {

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case GQA_ERR_WORKSPACE: return "workspace too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* gqa_last_error(void) { return g_last_error.c_str(); }

int gqa_decode_set_split_events(hipEvent_t before, hipEvent_t after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(GQA_ERR_INVALID_ARG, "give both events or neither");
  g_ev_before = before;
  g_ev_after = after;
  return GQA_OK;
}

size_t gqa_decode_workspace_bytes(int B, int h_q, int d_head, int n_splits) {
  if (B < 1 || h_q < 1 || d_head < 1 || n_splits < 1) return 0;
  return ws_bytes(B, h_q, d_head, n_splits);
}

int gqa_decode_pick_splits_d(int B, int h_kv, int d_head, int64_t s_kv_max, int num_cus) {
  if (B < 1 || h_kv < 1) return fail(GQA_ERR_INVALID_ARG, "B and h_kv must be >= 1");
  if (d_head != 64 && d_head != 128) return fail(GQA_ERR_UNSUPPORTED, "d_head %d not in {64, 128}", d_head);
  if (num_cus <= 0) {
    int st = device_cus(&num_cus);
    if (st != GQA_OK) return st;
  }
  return pick_splits_host(B, 1, h_kv, s_kv_max, num_cus, split_policy(1, d_head, true, 1));
}

int gqa_decode_pick_splits(int B, int h_kv, int64_t s_kv_max, int num_cus) {
  return gqa_decode_pick_splits_d(B, h_kv, 128, s_kv_max, num_cus);
}

int gqa_decode_multi_splits_d(int B, int S_q, int h_q, int h_kv, int d_head, int64_t s_kv_max, int num_cus) {
  if (B < 1 || h_kv < 1 || h_q < h_kv || h_q % h_kv) return fail(GQA_ERR_INVALID_ARG, "bad B / h_q / h_kv");
  if (d_head != 64 && d_head != 128) return fail(GQA_ERR_UNSUPPORTED, "d_head %d not 64 or 128", d_head);
  if (S_q < 1 || S_q > GQA_MAX_QUERY_TOKENS)
    return fail(GQA_ERR_INVALID_ARG, "S_q %d not in [1, %d]", S_q, GQA_MAX_QUERY_TOKENS);
  if (num_cus <= 0) {
    int st = device_cus(&num_cus);
    if (st != GQA_OK) return st;
  }
  int tpt, qtiles, tpw, passes;
  query_tiles(S_q, h_q / h_kv, B, s_kv_max, &tpt, &qtiles, &tpw, &passes);
  return pick_splits_host(B, passes, h_kv, s_kv_max, num_cus, split_policy(tpw, d_head, false, S_q),
                          tpw == gqa::kTileWaves && qtiles % gqa::kTileWaves == 0);
}

int gqa_decode_multi_splits(int B, int S_q, int h_q, int h_kv, int64_t s_kv_max, int num_cus) {
  return gqa_decode_multi_splits_d(B, S_q, h_q, h_kv, 128, s_kv_max, num_cus);
}

}  // extern "C"

namespace {

// Checks shared by every compute entry point (host only, no HIP call).
int check_shape(int B, int h_q, int h_kv, int d_head, int n_splits, int64_t s_kv_hint) {
  if (B < 1 || h_q < 1 || h_kv < 1) return fail(GQA_ERR_INVALID_ARG, "B, h_q, h_kv must be >= 1");
  if (B > 65535 || h_kv > 65535) return fail(GQA_ERR_INVALID_ARG, "B and h_kv must be <= 65535");
  if ((int64_t)B * h_q > INT32_MAX) return fail(GQA_ERR_INVALID_ARG, "B * h_q must be < 2^31");
  if (h_q % h_kv) return fail(GQA_ERR_INVALID_ARG, "h_q (%d) is not a multiple of h_kv (%d)", h_q, h_kv);
  if (!valid_nrep(h_q / h_kv))
    return fail(GQA_ERR_UNSUPPORTED, "h_q / h_kv = %d not in {1, 2, 4, 8, 16}", h_q / h_kv);
  if (d_head != 64 && d_head != 128) return fail(GQA_ERR_UNSUPPORTED, "d_head %d not in {64, 128}", d_head);
  if (n_splits > GQA_MAX_SPLITS) return fail(GQA_ERR_INVALID_ARG, "n_splits %d > %d", n_splits, GQA_MAX_SPLITS);
  if (s_kv_hint < 0) return fail(GQA_ERR_INVALID_ARG, "s_kv_hint < 0");
  return GQA_OK;
}

int check_inputs(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                 const int64_t* kv_token_offsets, float scale, int in_dtype, int flags) {
  if (!q || !k_cache || !v_cache || !seq_lens) return fail(GQA_ERR_INVALID_ARG, "null tensor pointer");
  if (!std::isfinite(scale)) return fail(GQA_ERR_INVALID_ARG, "scale is not finite");
  if (in_dtype != GQA_DTYPE_F32 && in_dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "in_dtype %d", in_dtype);
  if (flags & ~(GQA_FLAG_VALU | GQA_FLAG_FUSED)) return fail(GQA_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  for (const void* p : {q, k_cache, v_cache})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(GQA_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) % 4 || reinterpret_cast<uintptr_t>(kv_token_offsets) % 8)
    return fail(GQA_ERR_INVALID_ARG, "seq_lens / kv_token_offsets misaligned");
  return GQA_OK;
}

int check_out(const void* out, int out_dtype, size_t qo_elems) {
  if (!out) return fail(GQA_ERR_INVALID_ARG, "null tensor pointer");
  if (out_dtype != GQA_DTYPE_F32 && out_dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(GQA_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
  (void)qo_elems;
  return GQA_OK;
}

// Query tokens per 16-column tile and tiles per sequence for s_q query tokens.

// Split count, chunk floor and workspace partition of one call.
struct Plan {
  int ns, min_chunk;
  size_t need;
  float* ws_o;
  float2* ws_ml;
  unsigned long long* counters;
  int64_t* tok;                 // room for the packed layout's token bases
  int64_t hint;                 // the caller's longest length (0: unknown)
};

// The split count of a call: n_splits if > 0, else the heuristic's (which
// queries the device's compute units once per device).
int plan_splits(int B, int h_q, int h_kv, int d_head, int n_splits, int64_t s_kv_hint, int s_q,
                bool multi_entry, int* ns) {
  *ns = n_splits;
  if (n_splits > 0) return GQA_OK;
  int num_cus = 0;
  int st = device_cus(&num_cus);
  if (st != GQA_OK) return st;
  int tpt, qtiles, tpw, passes;
  query_tiles(s_q, h_q / h_kv, B, s_kv_hint, &tpt, &qtiles, &tpw, &passes);
  *ns = pick_splits_host(B, passes, h_kv, s_kv_hint, num_cus, split_policy(tpw, d_head, !multi_entry, s_q),
                         tpw == gqa::kTileWaves && qtiles % gqa::kTileWaves == 0);
  return GQA_OK;
}

int make_plan(int B, int h_q, int h_kv, int d_head, int n_splits, int64_t s_kv_hint,
              void* workspace, size_t workspace_bytes, bool allow_library_ws, Plan* pl,
              int s_q = 1, bool multi_entry = false) {
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(GQA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  if (!workspace && !allow_library_ws) return fail(GQA_ERR_INVALID_ARG, "this entry point needs a workspace");
  int ns = 0;
  int st0 = plan_splits(B, h_q, h_kv, d_head, n_splits, s_kv_hint, s_q, multi_entry, &ns);
  if (st0 != GQA_OK) return st0;
  pl->ns = ns;
  // a heuristic call keeps chunks of at least kMinChunk tokens, a call of
  // one query token over at most 4 sequences of at least one block
  // (no length hint, one query token: the floor grows with each sequence's
  // length on the device, see chunk_floor, over the wider grid the split
  // count gives such a call)
  pl->min_chunk = n_splits > 0 ? 1 : (s_kv_hint <= 0 && s_q == 1) ? 0 : (B <= 4 && s_q == 1 ? kBlockTokens : kMinChunk);
  pl->hint = s_kv_hint;
  pl->need = ws_bytes(B * s_q, h_q, d_head, ns);
  if (workspace) {
    if (workspace_bytes < pl->need)
      return fail(GQA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, pl->need);
  } else {
    int st = library_workspace(pl->need, &workspace);
    if (st != GQA_OK) return st;
  }
  const WsLayout lay = ws_layout(B * s_q, h_q, d_head, ns);
  pl->counters = static_cast<unsigned long long*>(workspace);
  pl->ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.o_off);
  pl->ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + lay.ml_off);
  pl->tok = reinterpret_cast<int64_t*>(static_cast<char*>(workspace) + lay.tok_off);
  return GQA_OK;
}

// The matrix-core split kernel's workgroup form for a plan (one query tile
// per workgroup), from the length hint:
//  - one wave per workgroup when every chunk holds at most
//    kOneWaveMaxTokens and the grid is more than one round of 4-wave
//    workgroups (two per CU; with one round or less, four waves per chunk
//    finish it sooner);
//  - eight waves per workgroup for a single sequence with 128-dimension
//    heads whose chunks hold kEightWaveMinChunk to kEightWaveMaxChunk tokens
//    and fit one workgroup per CU in one round;
//  - else four waves.
// A wrong hint changes only the speed: every form takes any length. The
// forms give a chunk's blocks to their waves differently, so their results
// differ in rounding.
Form split_form(const Plan& pl, int B, int h_kv, int d_head) {
  if (pl.hint <= 0) {
    // no length known: the one-round 8-wave plan of a single sequence with
    // 128-dimension heads (pick_splits_host; min_chunk 0 marks the
    // heuristic's single-token plan without a hint)
    int cus = 0;
    if (B == 1 && d_head == 128 && pl.min_chunk == 0 && device_cus(&cus) == GQA_OK &&
        (int64_t)pl.ns * h_kv <= cus)
      return Form::kEightWave;
    return Form::kFourWave;
  }
  const int64_t per_chunk = (pl.hint + pl.ns - 1) / pl.ns;
  const int64_t tok = std::min<int64_t>(pl.hint, std::max<int64_t>(per_chunk, pl.min_chunk));
  int cus = 0;
  if (device_cus(&cus) != GQA_OK) return Form::kFourWave;
  const int64_t wgs = (int64_t)pl.ns * h_kv * B;
  if (tok <= kOneWaveMaxTokens) return wgs > 2 * (int64_t)cus ? Form::kOneWave : Form::kFourWave;
  if (B == 1 && d_head == 128 && wgs <= cus && tok >= kEightWaveMinChunk && tok <= kEightWaveMaxChunk)
    return Form::kEightWave;
  return Form::kFourWave;
}

// Two query tiles per workgroup: eight waves (one block each, one register
// buffer) instead of four when every chunk holds 5 to 8 blocks and the grid
// is one workgroup per CU or less. Measured on one GPU, 21 interleaved
// rounds each, µs per call p10 / p50 / p90 (eight waves against four): 70B
// shapes, 8k tokens, 3 query tokens 13.90 / 13.97 / 14.07 against 15.35 /
// 15.43 / 15.55, 4 tokens 14.23 / 14.28 / 14.40 against 16.24 / 16.28 /
// 16.40; 6k tokens, 4 tokens 12.85 / 12.92 / 13.01 against 14.31 / 14.34 /
// 14.42; 64-dimension heads, 8k tokens, 4 tokens 10.32 / 10.38 / 10.50
// against 10.95 / 10.98 / 11.13. (A single sequence of up to 8k tokens with
// exactly two tiles now takes one tile per pass instead, see query_tiles; this
// form still serves two-tile calls such as B = 2 x 4k tokens.)
bool two_tile_eight_waves(const Plan& pl, int64_t units, int h_kv) {
  if (pl.hint <= 0) return false;
  const int64_t per_chunk = (pl.hint + pl.ns - 1) / pl.ns;
  const int64_t tok = std::min<int64_t>(pl.hint, std::max<int64_t>(per_chunk, pl.min_chunk));
  int cus = 0;
  if (device_cus(&cus) != GQA_OK) return false;
  return tok > 4 * kBlockTokens && tok <= 8 * kBlockTokens && (int64_t)pl.ns * h_kv * units <= cus;
}

// The tile-per-wave forms launch kv heads fastest when that lets the merge
// run each kv head's rows on the XCD that wrote them (8 kv heads, a
// merge_wave split count): workgroup L runs on XCD L mod 8, so kv head g's
// workgroups then all run on XCD g. 70B B = 1, µs per call, 7 interleaved
// rounds: 8k S_q = 64 50.7 -> 47.3, 16k S_q = 32 52.4 -> 46.4, 32k S_q = 64
// 126.7 -> 121.8; other split counts, whose merges are not remapped, stay in
// split order (8k S_q = 128, 8 splits: 78.6 -> 80.2 in kv-head order).
bool tiles_heads_fastest(int h_kv, int ns) {
  return h_kv == 8 && ns >= kMergeWaveMinSplits && ns <= kMergeWaveMaxSplits;
}

// The matrix-core split kernel's form for a call (four waves for anything
// else: the vector-ALU kernel, fp32 inputs).
Form choose_form(const Plan& pl, int B, int h_q, int h_kv, int d_head, int s_q, bool mfma, bool fused) {
  if (!mfma) return Form::kFourWave;
  int tpt, qtiles, tpw, passes;
  query_tiles(s_q, h_q / h_kv, B, pl.hint, &tpt, &qtiles, &tpw, &passes);
  if (s_q == 1) {                                  // the single-launch tail: 4 or 8 waves
    const Form f = split_form(pl, B, h_kv, d_head);
    return fused && f == Form::kOneWave ? Form::kFourWave : f;
  }
  // one tile of several query tokens: the single-token 8-wave round when it applies
  if (tpw == 1 && !fused && split_form(pl, B, h_kv, d_head) == Form::kEightWave) return Form::kEightWave;
  if (tpw == gqa::kTileWaves) return Form::kTiles;
  if (tpw == gqa::kTilePairs) return Form::kTilePairs;
  if (tpw == 2 && !fused && two_tile_eight_waves(pl, B * passes, h_kv)) return Form::kEightWave;
  return Form::kFourWave;
}

// Sequences of a batch over several rounds of workgroups start longest
// first (gqa::seq_info_ranked): returns B for the kernels' `ranked`, else 0.
// Within one round the order gains nothing. The ranking takes one step per
// sequence in every workgroup, so batches of more than 8 are ranked only
// when the longest chunk (hint / split count) holds at least
// kRankedMinChunk tokens, long enough for the order to pay for it. 70B
// shapes, µs per call, batch order / longest first: ragged B = 8 80.2 /
// 75.4, 16 sequences of 1k-32k 178.4 / 165.0, 32 of 1k-16k 224.8 / 215.9,
// 64 of 512-8k 216.2 / 205.0; ranked without the chunk rule, 32 x 4k
// (512-token chunks) 94.6 / 97.1; with the earlier loop of one 64-bit step
// per sequence and no chunk rule, 32 of 64-2100 tokens 31.9 / 37.1 and
// 12k + 3k (one round) 16.3 / 16.5.
constexpr int64_t kRankedMinChunk = 1024;
int ranked_batch(int B, dim3 grid, int64_t hint, int ns) {
  int cus = 0;
  const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
  if (B < 2 || B > gqa::kRankedMaxBatch || device_cus(&cus) != GQA_OK || wgs <= 2 * (int64_t)cus) return 0;
  if (B > 8 && (hint <= 0 || (hint + ns - 1) / ns < kRankedMinChunk)) return 0;
  return B;
}

// direct: the caller merges nothing afterwards; with one chunk per sequence
// the split kernel then writes out itself (returned in *merged).
int run_split(const Plan& pl, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* seq_lens, const int64_t* kv_token_offsets, int B, int h_q, int h_kv,
              int d_head, float scale, int in_dtype, hipStream_t stream, int flags,
              void* out = nullptr, int out_dtype = GQA_DTYPE_F32, int s_q = 1, bool* merged = nullptr) {
  const int fused = (flags & GQA_FLAG_FUSED) ? 1 : 0;
  const bool mfma = in_dtype == GQA_DTYPE_BF16 && !(flags & GQA_FLAG_VALU);   // the kernel with the direct path
  const int direct = (merged && !fused && mfma && pl.ns == 1) ? 1 : 0;
  if (merged) *merged = fused || direct;
  int tpt, qtiles, tpw, passes;
  query_tiles(s_q, h_q / h_kv, B, pl.hint, &tpt, &qtiles, &tpw, &passes);
  const int64_t* tok = kv_token_offsets;
  if (!tok && B > kScanMinBatch) {             // packed layout, many sequences: scan once
    hipLaunchKernelGGL(gqa::packed_offsets, dim3(1), dim3(1024), 0, stream, seq_lens, B, pl.tok);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "token offset scan launch: %s", hipGetErrorString(e));
    tok = pl.tok;
  }
  gqa::SplitArgs sa{q, k_cache, v_cache, seq_lens, tok, pl.ws_o, pl.ws_ml,
                    h_q, h_kv, pl.ns, pl.min_chunk, scale * gqa::kLog2e,
                    fused, out_dtype == GQA_DTYPE_BF16 ? 1 : 0, out, pl.counters,
                    fused ? (g_call_tag.fetch_add(1) & 0xFFFFFFFFFFFFull) : 0ull,
                    s_q, tpt, qtiles, passes};
  sa.direct = direct;
  dim3 grid = gqa::split_grid(pl.ns, h_kv, B * passes);
  const bool bf16 = in_dtype == GQA_DTYPE_BF16;
  const bool valu = (flags & GQA_FLAG_VALU) != 0;
  const int nrep = h_q / h_kv;
  hipError_t e;
  if (g_ev_before && (e = hipEventRecord(g_ev_before, stream)) != hipSuccess)
    return fail(GQA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  const Form form = choose_form(pl, B, h_q, h_kv, d_head, s_q, mfma, fused);
  if (form == Form::kEightWave) grid = gqa::split_grid_heads_fastest(pl.ns, h_kv, B * passes);
  if ((form == Form::kTiles || form == Form::kTilePairs) && tiles_heads_fastest(h_kv, pl.ns)) {
    grid = gqa::split_grid_heads_fastest(pl.ns, h_kv, B * passes);
    sa.heads_fastest = 1;
  }
  sa.ranked = ranked_batch(B, grid, pl.hint, pl.ns);
  e = d_head == 128 ? launch_split_nrep<128>(nrep, bf16, valu, form, grid, stream, sa)
                    : launch_split_nrep<64>(nrep, bf16, valu, form, grid, stream, sa);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "split kernel launch: %s", hipGetErrorString(e));
  if (g_ev_after && (e = hipEventRecord(g_ev_after, stream)) != hipSuccess)
    return fail(GQA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  return GQA_OK;
}

// heads_fastest: the split kernel's grid ran kv heads fastest (the 8-wave
// forms, and the tile-per-wave forms where tiles_heads_fastest says so).
int run_merge(const Plan& pl, const int32_t* seq_lens, void* out, int B, int h_q, int h_kv, int d_head,
              int out_dtype, hipStream_t stream, bool heads_fastest, int s_q = 1, float2* tri_ml = nullptr,
              float* tri_o = nullptr) {
  // With 8 kv heads launched heads fastest, kv head g's chunks ran on XCD g;
  // merging its heads there measured faster for several query tokens (8k
  // tokens, 4 query tokens: 14.86 -> 14.02 us per call; one token: no change).
  const int xcd_rep = heads_fastest && h_kv == 8 ? h_q / 8 : 0;
  gqa::MergeArgs ma{s_q, seq_lens, pl.ws_o, pl.ws_ml, out, h_q, pl.ns, pl.min_chunk,
                    pl.ns, 1, tri_ml, tri_o, xcd_rep};
  const bool obf16 = out_dtype == GQA_DTYPE_BF16;
  hipError_t e = d_head == 128 ? launch_merge<128>(obf16, B * s_q, h_q, stream, ma)
                               : launch_merge<64>(obf16, B * s_q, h_q, stream, ma);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return GQA_OK;
}

// Argument checks of the single-token attention entry points (host only).
int check_attn_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                    const int64_t* kv_token_offsets, const void* out, int B, int h_q, int h_kv, int d_head,
                    float scale, int n_splits, int in_dtype, int out_dtype, int64_t s_kv_hint, int flags) {
  int st;
  if (!out) return fail(GQA_ERR_INVALID_ARG, "null tensor pointer");
  if ((st = check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets, scale, in_dtype, flags))) return st;
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, s_kv_hint))) return st;
  const size_t qo = (size_t)B * h_q * d_head;
  if ((st = check_out(out, out_dtype, qo))) return st;
  const size_t in_el = in_dtype == GQA_DTYPE_BF16 ? 2 : 4, out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if (overlap(out, qo * out_el, q, qo * in_el) || overlap(out, qo * out_el, seq_lens, (size_t)B * 4) ||
      out == k_cache || out == v_cache)
    return fail(GQA_ERR_INVALID_ARG, "out overlaps an input");
  return GQA_OK;
}

// Split kernel, then the merge unless the split kernel wrote out itself.
int run_attn(const Plan& pl, const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
             const int64_t* kv_token_offsets, void* out, int B, int h_q, int h_kv, int d_head, float scale,
             int in_dtype, int out_dtype, hipStream_t stream, int flags) {
  bool merged = false;
  int st = run_split(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, B, h_q, h_kv, d_head, scale, in_dtype,
                     stream, flags, out, out_dtype, 1, &merged);
  if (st != GQA_OK) return st;
  if (merged) return GQA_OK;
  const bool mfma = in_dtype == GQA_DTYPE_BF16 && !(flags & GQA_FLAG_VALU);
  const bool eight = choose_form(pl, B, h_q, h_kv, d_head, 1, mfma, flags & GQA_FLAG_FUSED) == Form::kEightWave;
  return run_merge(pl, seq_lens, out, B, h_q, h_kv, d_head, out_dtype, stream, eight);
}

}  // namespace

// Workspace of gqa_decode_attn_noalloc: a static device array, one copy per
// GPU, kept until the process ends. In host code this name stands for a
// host-side shadow, not for device memory: kernels and copies get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[GQA_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[64];                           // device address of `scratch`, per device ordinal

// The current device's copy of `scratch`, looked up once per device with
// that device current (the first gqa_decode_attn_noalloc call on it).
int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(GQA_ERR_HIP, "device ordinal %d not supported", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (!p || reinterpret_cast<uintptr_t>(p) % 256)
      return fail(GQA_ERR_HIP, "static scratch at %p: null or not 256-byte aligned", p);
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_decode_attn_ex(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int64_t* kv_token_offsets,
                       void* out, int B, int h_q, int h_kv, int d_head,
                       float scale, int n_splits, int in_dtype, int out_dtype,
                       int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, int flags) {
  int st;
  if ((st = check_attn_args(q, k_cache, v_cache, seq_lens, kv_token_offsets, out, B, h_q, h_kv, d_head, scale,
                            n_splits, in_dtype, out_dtype, s_kv_hint, flags)))
    return st;
  const size_t qo = (size_t)B * h_q * d_head, out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if (workspace && overlap(out, qo * out_el, workspace, workspace_bytes))
    return fail(GQA_ERR_INVALID_ARG, "out overlaps workspace");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, workspace, workspace_bytes, true, &pl))) return st;
  return run_attn(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, out, B, h_q, h_kv, d_head, scale,
                  in_dtype, out_dtype, stream, flags);
}

int gqa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int64_t* kv_token_offsets,
                            void* out, int B, int h_q, int h_kv, int d_head,
                            float scale, int n_splits, int in_dtype, int out_dtype,
                            int64_t s_kv_hint, hipStream_t stream, int flags) {
  int st;
  if ((st = check_attn_args(q, k_cache, v_cache, seq_lens, kv_token_offsets, out, B, h_q, h_kv, d_head, scale,
                            n_splits, in_dtype, out_dtype, s_kv_hint, flags)))
    return st;
  int ns = 0;
  if ((st = plan_splits(B, h_q, h_kv, d_head, n_splits, s_kv_hint, 1, false, &ns))) return st;
  const size_t need = ws_bytes(B, h_q, d_head, ns);
  if (need > (size_t)GQA_SCRATCH_BYTES)
    return fail(GQA_ERR_WORKSPACE,
                "gqa_decode_attn_noalloc: %d splits of %d x %d rows of %d need %zu bytes of workspace, more than "
                "the static scratch's %zu (GQA_SCRATCH_BYTES); pass fewer splits or use gqa_decode_attn_ex",
                ns, B, h_q, d_head, need, (size_t)GQA_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  const size_t qo = (size_t)B * h_q * d_head, out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if (overlap(out, qo * out_el, ws, GQA_SCRATCH_BYTES))
    return fail(GQA_ERR_INVALID_ARG, "out overlaps the static scratch");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, ws, GQA_SCRATCH_BYTES, false, &pl))) return st;
  return run_attn(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, out, B, h_q, h_kv, d_head, scale,
                  in_dtype, out_dtype, stream, flags);
}

int gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int64_t* kv_token_offsets,
                       int B, int h_q, int h_kv, int d_head, float scale, int n_splits,
                       int in_dtype, int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, int flags) {
  int st;
  if ((st = check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets, scale, in_dtype, flags))) return st;
  if (flags & GQA_FLAG_FUSED) return fail(GQA_ERR_INVALID_ARG, "gqa_decode_partial does not merge");
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, s_kv_hint))) return st;
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, workspace, workspace_bytes, false, &pl))) return st;
  return run_split(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, B, h_q, h_kv, d_head, scale,
                   in_dtype, stream, flags);
}

int gqa_decode_merge(const int32_t* seq_lens, const void* workspace, size_t workspace_bytes, void* out,
                     int B, int h_q, int h_kv, int d_head, int n_splits, int64_t s_kv_hint,
                     int out_dtype, hipStream_t stream) {
  int st;
  if (!seq_lens || !workspace) return fail(GQA_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(seq_lens) % 4) return fail(GQA_ERR_INVALID_ARG, "seq_lens misaligned");
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, s_kv_hint))) return st;
  const size_t qo = (size_t)B * h_q * d_head;
  if ((st = check_out(out, out_dtype, qo))) return st;
  const size_t out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if (overlap(out, qo * out_el, workspace, workspace_bytes) || overlap(out, qo * out_el, seq_lens, (size_t)B * 4))
    return fail(GQA_ERR_INVALID_ARG, "out overlaps an input");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, const_cast<void*>(workspace), workspace_bytes,
                      false, &pl)))
    return st;
  // (the split kernel's form only moves rows between workgroups: taken for bf16 inputs)
  const bool eight = choose_form(pl, B, h_q, h_kv, d_head, 1, true, false) == Form::kEightWave;
  return run_merge(pl, seq_lens, out, B, h_q, h_kv, d_head, out_dtype, stream, eight);
}

int gqa_decode_attn_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, const int64_t* kv_token_offsets, void* out,
                          int B, int S_q, int h_q, int h_kv, int d_head, float scale, int n_splits,
                          int out_dtype, int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int st;
  if (!out) return fail(GQA_ERR_INVALID_ARG, "null tensor pointer");
  if (S_q < 1 || S_q > GQA_MAX_QUERY_TOKENS)
    return fail(GQA_ERR_INVALID_ARG, "S_q %d not in [1, %d]", S_q, GQA_MAX_QUERY_TOKENS);
  if ((st = check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets, scale, GQA_DTYPE_BF16, 0))) return st;
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, s_kv_hint))) return st;
  int tpt, qtiles, tpw, passes;
  query_tiles(S_q, h_q / h_kv, B, s_kv_hint, &tpt, &qtiles, &tpw, &passes);
  if ((int64_t)B * passes > 65535)
    return fail(GQA_ERR_INVALID_ARG, "B * workgroup passes (ceil(query tiles / tiles per workgroup)) must be <= 65535");
  if ((int64_t)B * S_q * h_q > INT32_MAX) return fail(GQA_ERR_INVALID_ARG, "B * S_q * h_q must be < 2^31");
  const size_t qo = (size_t)B * S_q * h_q * d_head;
  if ((st = check_out(out, out_dtype, qo))) return st;
  const size_t out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4;
  if (overlap(out, qo * out_el, q, qo * 2) || overlap(out, qo * out_el, seq_lens, (size_t)B * 4) ||
      out == k_cache || out == v_cache)
    return fail(GQA_ERR_INVALID_ARG, "out overlaps an input");
  if (workspace && overlap(out, qo * out_el, workspace, workspace_bytes))
    return fail(GQA_ERR_INVALID_ARG, "out overlaps workspace");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, workspace, workspace_bytes, true, &pl, S_q,
                      true)))
    return st;
  bool merged = false;
  if ((st = run_split(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, B, h_q, h_kv, d_head, scale,
                      GQA_DTYPE_BF16, stream, 0, out, out_dtype, S_q, &merged)))
    return st;
  if (merged) return GQA_OK;
  // the split kernel's workgroups ran kv heads fastest: merge each head's rows on its XCD
  const Form fm = choose_form(pl, B, h_q, h_kv, d_head, S_q, true, false);
  const bool heads_fastest = fm == Form::kEightWave ||
                             ((fm == Form::kTiles || fm == Form::kTilePairs) && tiles_heads_fastest(h_kv, pl.ns));
  return run_merge(pl, seq_lens, out, B, h_q, h_kv, d_head, out_dtype, stream, heads_fastest, S_q);
}

int gqa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int64_t* kv_token_offsets, const int32_t* seq_lens, int32_t* seq_lens_out,
                  int B, int n_new, int h_kv, int d_head, int dtype, int64_t capacity,
                  hipStream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return fail(GQA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || B > 65535 || n_new < 1 || h_kv < 1 || capacity < 1)
    return fail(GQA_ERR_INVALID_ARG, "B, n_new, h_kv, capacity must be >= 1 (B <= 65535)");
  if (d_head != 64 && d_head != 128) return fail(GQA_ERR_UNSUPPORTED, "d_head %d not in {64, 128}", d_head);
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return fail(GQA_ERR_UNSUPPORTED, "dtype %d", dtype);
  for (const void* p : {k_new, v_new, (const void*)k_cache, (const void*)v_cache})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(GQA_ERR_INVALID_ARG, "tensor pointer not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(seq_lens) % 4 || reinterpret_cast<uintptr_t>(seq_lens_out) % 4 ||
      reinterpret_cast<uintptr_t>(kv_token_offsets) % 8)
    return fail(GQA_ERR_INVALID_ARG, "seq_lens / offsets misaligned");
  if (seq_lens_out && overlap(seq_lens_out, (size_t)B * 4, seq_lens, (size_t)B * 4))
    return fail(GQA_ERR_INVALID_ARG, "seq_lens_out overlaps seq_lens");
  const size_t el = dtype == GQA_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = (int64_t)h_kv * d_head * (int64_t)el;
  if (row_bytes / 16 > INT32_MAX) return fail(GQA_ERR_INVALID_ARG, "token row too large");
  gqa::AppendArgs aa{k_new, v_new, k_cache, v_cache, kv_token_offsets, seq_lens, seq_lens_out,
                     n_new, (int)(row_bytes / 16), capacity};
  hipLaunchKernelGGL(gqa::kv_append_rows, dim3((unsigned)n_new, (unsigned)B), dim3(256), 0, stream, aa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "append kernel launch: %s", hipGetErrorString(e));
  return GQA_OK;
}

int gqa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* seq_lens, int32_t* seq_lens_out, const int64_t* kv_token_offsets,
                    void* out, int B, int h_q, int h_kv, int d_head, float scale, int n_splits,
                    int in_dtype, int out_dtype, int64_t capacity, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  int st;
  if (!out || !k_new || !v_new || !seq_lens_out) return fail(GQA_ERR_INVALID_ARG, "null pointer");
  if ((st = check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets, scale, in_dtype, 0))) return st;
  if (in_dtype != GQA_DTYPE_BF16)
    return fail(GQA_ERR_UNSUPPORTED, "gqa_decode_step takes bf16 (use gqa_kv_append + gqa_decode_attn_ex)");
  if (capacity < 1 || capacity > INT32_MAX) return fail(GQA_ERR_INVALID_ARG, "capacity must be in [1, 2^31)");
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, capacity))) return st;
  const size_t qo = (size_t)B * h_q * d_head;
  if ((st = check_out(out, out_dtype, qo))) return st;
  if (reinterpret_cast<uintptr_t>(k_new) % 16 || reinterpret_cast<uintptr_t>(v_new) % 16 ||
      reinterpret_cast<uintptr_t>(seq_lens_out) % 4)
    return fail(GQA_ERR_INVALID_ARG, "k_new / v_new / seq_lens_out misaligned");
  const size_t out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4, row = (size_t)B * h_kv * d_head * 2;
  if (overlap(seq_lens_out, (size_t)B * 4, seq_lens, (size_t)B * 4))
    return fail(GQA_ERR_INVALID_ARG, "seq_lens_out overlaps seq_lens");
  if (overlap(out, qo * out_el, q, qo * 2) || overlap(out, qo * out_el, seq_lens, (size_t)B * 4) ||
      overlap(out, qo * out_el, seq_lens_out, (size_t)B * 4) || overlap(out, qo * out_el, k_new, row) ||
      overlap(out, qo * out_el, v_new, row) || out == k_cache || out == v_cache)
    return fail(GQA_ERR_INVALID_ARG, "out overlaps an input");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, capacity, workspace, workspace_bytes, true, &pl)))
    return st;
  gqa::SplitArgs sa{q, k_cache, v_cache, seq_lens, kv_token_offsets, pl.ws_o, pl.ws_ml,
                    h_q, h_kv, pl.ns, pl.min_chunk, scale * gqa::kLog2e,
                    0, out_dtype == GQA_DTYPE_BF16 ? 1 : 0, out, pl.counters, 0ull, 1, 1, 1, 1,
                    k_new, v_new, seq_lens_out, (int)capacity, pl.ns == 1 ? 1 : 0};
  const int nrep = h_q / h_kv;
  const Form form = split_form(pl, B, h_kv, d_head);   // the same form as gqa_decode_attn_ex with this hint
  const dim3 grid = form == Form::kEightWave ? gqa::split_grid_heads_fastest(pl.ns, h_kv, B)
                                             : gqa::split_grid(pl.ns, h_kv, B);
  sa.ranked = ranked_batch(B, grid, pl.hint, pl.ns);
  hipError_t e = d_head == 128 ? launch_split_append<128>(nrep, form, grid, stream, sa)
                               : launch_split_append<64>(nrep, form, grid, stream, sa);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "split kernel launch: %s", hipGetErrorString(e));
  if (sa.direct) return GQA_OK;                    // one chunk per sequence: out is written
  return run_merge(pl, seq_lens_out, out, B, h_q, h_kv, d_head, out_dtype, stream, form == Form::kEightWave);
}

int gqa_decode_attn_triplet(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int64_t* kv_token_offsets,
                            float* ml_out, float* o_out, int B, int h_q, int h_kv, int d_head,
                            float scale, int n_splits, int in_dtype, int64_t s_kv_hint,
                            void* workspace, size_t workspace_bytes, hipStream_t stream, int flags) {
  int st;
  if (!ml_out || !o_out) return fail(GQA_ERR_INVALID_ARG, "null pointer");
  if ((st = check_inputs(q, k_cache, v_cache, seq_lens, kv_token_offsets, scale, in_dtype, flags))) return st;
  if (flags & GQA_FLAG_FUSED) return fail(GQA_ERR_INVALID_ARG, "GQA_FLAG_FUSED does not apply here");
  if ((st = check_shape(B, h_q, h_kv, d_head, n_splits, s_kv_hint))) return st;
  if (reinterpret_cast<uintptr_t>(ml_out) % 8 || reinterpret_cast<uintptr_t>(o_out) % 16)
    return fail(GQA_ERR_INVALID_ARG, "ml_out / o_out misaligned");
  const size_t rows = (size_t)B * h_q;
  if (overlap(ml_out, rows * 8, o_out, rows * d_head * 4) ||
      (workspace && (overlap(ml_out, rows * 8, workspace, workspace_bytes) ||
                     overlap(o_out, rows * d_head * 4, workspace, workspace_bytes))))
    return fail(GQA_ERR_INVALID_ARG, "outputs overlap");
  Plan pl;
  if ((st = make_plan(B, h_q, h_kv, d_head, n_splits, s_kv_hint, workspace, workspace_bytes, true, &pl))) return st;
  if ((st = run_split(pl, q, k_cache, v_cache, seq_lens, kv_token_offsets, B, h_q, h_kv, d_head, scale,
                      in_dtype, stream, flags)))
    return st;
  const bool mfma = in_dtype == GQA_DTYPE_BF16 && !(flags & GQA_FLAG_VALU);
  const bool eight = choose_form(pl, B, h_q, h_kv, d_head, 1, mfma, false) == Form::kEightWave;
  return run_merge(pl, seq_lens, nullptr, B, h_q, h_kv, d_head, GQA_DTYPE_F32, stream, eight, 1,
                   reinterpret_cast<float2*>(ml_out), o_out);
}

int gqa_merge_triplets(const float* ml, const float* o, int parts, int rows, int d_head,
                       void* out, int out_dtype, hipStream_t stream) {
  int st;
  if (!ml || !o) return fail(GQA_ERR_INVALID_ARG, "null pointer");
  if (parts < 1 || rows < 1) return fail(GQA_ERR_INVALID_ARG, "parts and rows must be >= 1");
  if (d_head != 64 && d_head != 128) return fail(GQA_ERR_UNSUPPORTED, "d_head %d not in {64, 128}", d_head);
  if (reinterpret_cast<uintptr_t>(ml) % 8 || reinterpret_cast<uintptr_t>(o) % 16)
    return fail(GQA_ERR_INVALID_ARG, "ml / o misaligned");
  if ((st = check_out(out, out_dtype, (size_t)rows * d_head))) return st;
  const size_t out_el = out_dtype == GQA_DTYPE_BF16 ? 2 : 4, n = (size_t)parts * rows;
  if (overlap(out, (size_t)rows * d_head * out_el, ml, n * 8) ||
      overlap(out, (size_t)rows * d_head * out_el, o, n * d_head * 4))
    return fail(GQA_ERR_INVALID_ARG, "out overlaps an input");
  gqa::MergeArgs ma{1, nullptr, o, reinterpret_cast<const float2*>(ml), out, 1, parts, 1,
                    1, rows, nullptr, nullptr, 0};
  const bool obf16 = out_dtype == GQA_DTYPE_BF16;
  hipError_t e = d_head == 128 ? launch_merge<128>(obf16, rows, 1, stream, ma)
                               : launch_merge<64>(obf16, rows, 1, stream, ma);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return GQA_OK;
}

int gqa_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out,
                    int B, int h_q, int h_kv, int d_head,
                    float scale, int n_splits) {
  return gqa_decode_attn_ex(q, k_cache, v_cache, seq_lens, nullptr, out, B, h_q, h_kv, d_head,
                            scale, n_splits, GQA_DTYPE_BF16, GQA_DTYPE_F32, 0, nullptr, 0,
                            nullptr, 0);
}

}  // extern "C"
