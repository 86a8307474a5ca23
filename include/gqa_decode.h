/*
 * gqa_decode.h - single-token grouped-query decode attention on gfx950 (MI355X).
 *
 * What the library computes. For every sequence b, query head h and the
 * S_b cached positions of sequence b:
 *
 *     s_t      = scale * <q[b, h, :], K[off_b + t, g, :]>,   g = h / (h_q / h_kv)
 *     out[b,h] = sum_t softmax(s)_t * V[off_b + t, g, :]
 *
 * Query heads form contiguous groups of n_rep = h_q / h_kv that share one
 * key/value head (tinygrad issue #5244 "llama speed tracking issue",
 * `Attention.__call__`: q is split by n_rep * head_dim, k and v by head_dim;
 * the exllama discussion "Llama 2 is out": 70B has 64 heads in 8 groups).
 *
 * How. The KV range of each (sequence, kv head) is cut into n_splits chunks,
 * one per workgroup. Each chunk yields a partial (m, l, o) triplet - running
 * max, sum of exponentials, unnormalised output - and a second kernel merges
 * the triplets exactly and divides o by l (kernbench2 page
 * `_attention_mesh_mlo.py`: module docstring, the local partial-attention
 * block, the receive-and-merge blocks and the final normalisation). Here the
 * split runs across the workgroups of one GPU instead of across ranks.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library
 *    never frees or keeps them beyond the call.
 *  - All argument checks run on the host before any HIP call; on error
 *    nothing is launched and nothing is written.
 *  - Work is enqueued on the stream and the call returns without waiting for
 *    it (no host synchronisation). Results are valid once the stream has
 *    executed past the call.
 *  - Return value: GQA_OK (0) or a negative gqa status. gqa_last_error()
 *    gives a message for the calling thread's last failure.
 *  - No C++ exception crosses this interface.
 *  - `out` must not overlap q, k_cache, v_cache, seq_lens or the workspace.
 *
 * Layouts (row-major, element strides implied by the shapes):
 *  q        [B, h_q, d_head]
 *  k_cache  [T, h_kv, d_head]  T >= sum_b S_b. Packed: sequence b occupies
 *  v_cache  [T, h_kv, d_head]  token rows [off_b, off_b + S_b) with
 *                              off_b = sum_{j<b} S_j, unless per-sequence
 *                              offsets are given (`_ex`).
 *  seq_lens [B] int32, S_b >= 0 (device memory). S_b = 0 gives out = 0.
 *  out      [B, h_q, d_head]
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = -1, /* null pointer, bad count, h_q % h_kv != 0, non-finite scale,
                                 overlapping out, n_splits above GQA_MAX_SPLITS, unknown flag */
    GQA_ERR_UNSUPPORTED = -2, /* d_head not in {64, 128}, n_rep not in {1, 2, 4, 8, 16},
                                 unknown dtype or dtype combination */
    GQA_ERR_WORKSPACE = -3,   /* caller workspace smaller than gqa_decode_workspace_bytes() */
    GQA_ERR_HIP = -4          /* no device, allocation or launch failure (message kept) */
};

/* Element types of q/k_cache/v_cache (one type for all three) and of out. */
enum { GQA_DTYPE_F32 = 0, GQA_DTYPE_BF16 = 1 };

/* Flags of gqa_decode_attn_ex. */
enum {
    GQA_FLAG_VALU = 1,  /* use the vector-ALU split kernel instead of the matrix-core one
                           (bf16 inputs; fp32 inputs always use it). For comparison. */
    GQA_FLAG_FUSED = 2  /* one kernel launch: the last split workgroup of each (sequence,
                           kv head) merges that group's triplets and writes out (uses the
                           workspace's arrival counters, see gqa_decode_workspace_bytes).
                           Correct, but slower on MI355X than the default two launches
                           (70B shapes, 8k tokens: 27.4 us vs 11.5 us per call): the
                           device-scope counter load and add a workgroup makes to learn
                           whether it is the last take 3 and 7 us (median) when the 32
                           workgroups of a group arrive together, and the last one then
                           reads the group's triplets after an L2 invalidation (3.4 us). */
};

/* Largest split count. */
#define GQA_MAX_SPLITS 4096

/* Largest number of query tokens per sequence of gqa_decode_attn_multi
 * (speculative decoding verifies a few, chunked prefill sends hundreds to
 * thousands, the prefill of a whole prompt as many as it holds). */
#define GQA_MAX_QUERY_TOKENS 16384

/*
 * Attention for bf16 q/k_cache/v_cache in the packed layout, fp32 `out`, on
 * the null stream, with a library-owned workspace (allocated on first use on
 * each device and grown when needed; it is shared, so calls that may run
 * concurrently on different streams must use gqa_decode_attn_ex with their
 * own workspace).
 *  scale     multiplies q.k before the softmax (1/sqrt(d_head) for Llama).
 *  n_splits  > 0 forces the number of KV chunks per (sequence, kv head);
 *            <= 0 lets gqa_decode_pick_splits_d choose with no length hint:
 *            chunks sized on the device from each sequence's length; for
 *            one sequence with d_head = 128, num_cus / h_kv chunks run by
 *            one 8-wave workgroup per compute unit (32 for 8 kv heads on 256
 *            CUs), otherwise a grid of four rounds of workgroups whose
 *            chunks hold at least 32 to 128 tokens.
 */
int gqa_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out,
                    int B, int h_q, int h_kv, int d_head,
                    float scale, int n_splits);

/*
 * Full form.
 *  kv_token_offsets  [B] int64 device array of the first token row of each
 *                    sequence (e.g. b * S_max for a padded [B, S_max, h_kv, d]
 *                    cache); NULL means the packed layout.
 *  in_dtype          GQA_DTYPE_BF16 or GQA_DTYPE_F32 (q, k_cache, v_cache).
 *  out_dtype         GQA_DTYPE_F32, or GQA_DTYPE_BF16 (rounded to nearest even).
 *  s_kv_hint         host-side upper bound of max_b S_b, or 0 if unknown. The
 *                    split heuristic uses it, and so does the choice of the
 *                    matrix-core kernel's workgroup form (one wave per
 *                    workgroup when every chunk would hold at most 128
 *                    tokens and there are more than 2 chunks per compute
 *                    unit); the kernels read seq_lens, so a wrong hint costs
 *                    only speed. Different hints can give results that differ
 *                    in fp32 rounding (another split count or form).
 *  workspace         device buffer of at least gqa_decode_workspace_bytes(B, h_q,
 *                    d_head, n) bytes, n being the split count that will be used
 *                    (n_splits if > 0, else gqa_decode_pick_splits_d(B, h_kv,
 *                    d_head, s_kv_hint, 0)); 256-byte aligned. NULL:
 *                    library-owned.
 *  stream            HIP stream (NULL: null stream).
 *  flags             0 or an OR of GQA_FLAG_VALU and GQA_FLAG_FUSED.
 * With one chunk per sequence (n = 1) and the matrix-core kernel, the split
 * kernel writes out itself and no merge kernel runs (the same bits as the
 * merge would give: a single triplet's weight is exactly 1).
 */
int gqa_decode_attn_ex(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int64_t* kv_token_offsets,
                       void* out, int B, int h_q, int h_kv, int d_head,
                       float scale, int n_splits, int in_dtype, int out_dtype,
                       int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, int flags);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * gqa_decode_attn_ex without a workspace argument and without allocating.
 * Its split and merge kernels use a library-owned static device array of
 * GQA_SCRATCH_BYTES bytes (one per GPU, held until the process ends) as
 * their workspace. The call returns GQA_ERR_WORKSPACE, with nothing
 * launched, when gqa_decode_workspace_bytes(B, h_q, d_head, n) exceeds
 * GQA_SCRATCH_BYTES for the split count n it would use; pass a smaller
 * n_splits, or call gqa_decode_attn_ex with a workspace. It calls no
 * hipMalloc or hipFree; its first call on a device looks up that device's
 * copy of the array (hipGetSymbolAddress). Every call on one GPU shares the
 * array, and no kernel needs it cleared, but calls that overlap in time on
 * one GPU (different streams, or host threads) race on it: serialise them.
 * Same arguments, kernels and results (bit for bit) as gqa_decode_attn_ex
 * given a workspace.
 */
#define GQA_SCRATCH_BYTES (16u << 20)

int gqa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int64_t* kv_token_offsets,
                            void* out, int B, int h_q, int h_kv, int d_head,
                            float scale, int n_splits, int in_dtype, int out_dtype,
                            int64_t s_kv_hint, hipStream_t stream, int flags);

/*
 * Several new query tokens per sequence (e.g. verifying speculated tokens):
 * q and out are [B, S_q, h_q, d_head]; the S_q tokens are the last S_q
 * positions of sequence b, their K/V rows already in the cache, and token i
 * (position S_b - S_q + i) attends cache positions [0, S_b - S_q + i] - causal
 * among the new tokens. A token with S_b - S_q + i < 0 gets zeros. With
 * S_q = 1 this equals gqa_decode_attn_ex. bf16 inputs (matrix-core kernel),
 * fp32 or bf16 out, 1 <= S_q <= GQA_MAX_QUERY_TOKENS. The (token, head)
 * columns fill 16-wide MFMA tiles of t = min(S_q, 16 / n_rep) tokens (the
 * columns single-token decode leaves empty when n_rep < 16). A pass over the
 * KV range serves two tiles (2t tokens read the KV once), or eight tiles (one
 * per wave, the K/V blocks shared through LDS; sixteen, two per wave, from
 * 16 tiles on) when a sequence has at least 8 tiles and B * s_kv_hint >=
 * 16384 tokens, at least 4 tiles and B * s_kv_hint >= 65536, at least 5
 * tiles and B * s_kv_hint >= 32768, at least 12 tiles and B * s_kv_hint >=
 * 8192, or at least 16 tiles and tiles * B * s_kv_hint >= 2^18; more tokens
 * take more passes. Exactly two tiles with n_rep >= 4 over short KV (B == 1
 * and s_kv_hint <= 8192, or s_kv_hint <= 2048 and B * s_kv_hint <= 8192)
 * take one tile per pass. The hint only picks the kernel and the split
 * count: every kernel takes any length, and they round differently. Workspace: gqa_decode_workspace_bytes(B * S_q,
 * h_q, d_head, n) with n = n_splits if > 0, else gqa_decode_multi_splits_d(B,
 * S_q, h_q, h_kv, d_head, s_kv_hint, 0). B * passes <= 65535. Other
 * arguments as in gqa_decode_attn_ex.
 */
int gqa_decode_attn_multi(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seq_lens, const int64_t* kv_token_offsets, void* out,
                          int B, int S_q, int h_q, int h_kv, int d_head, float scale, int n_splits,
                          int out_dtype, int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * KV-cache append, the step before attention at each decode step (the
 * tt-metal Llama burndown's update_cache): for every sequence b and new token
 * i < n_new, copy k_new[b, i] and v_new[b, i] ([B, n_new, h_kv, d_head], the
 * cache's dtype) to token row off_b + seq_lens[b] + i of k_cache / v_cache,
 * where off_b = kv_token_offsets[b], or b * capacity if kv_token_offsets is
 * NULL (a padded [B, capacity, h_kv, d_head] cache). Each sequence owns
 * `capacity` rows: new rows at positions >= capacity are dropped. If
 * seq_lens_out is not NULL it receives min(seq_lens[b] + n_new, capacity);
 * it must not overlap seq_lens (alternate two length buffers across steps).
 * dtype: GQA_DTYPE_BF16 or GQA_DTYPE_F32. Asynchronous on `stream`.
 */
int gqa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int64_t* kv_token_offsets, const int32_t* seq_lens, int32_t* seq_lens_out,
                  int B, int n_new, int h_kv, int d_head, int dtype, int64_t capacity,
                  hipStream_t stream);

/*
 * One decode step in two launches instead of three: gqa_kv_append of one new
 * token per sequence (the tt-metal burndown's update_cache, the step before
 * attention) followed by gqa_decode_attn_ex on the new lengths, with the
 * append folded into the split kernel.
 *   k_new, v_new  [B, h_kv, d_head] bf16 device: the new token's K and V rows.
 *   k_cache, v_cache  padded cache [T, h_kv, d_head] bf16 (written: row
 *                 off_b + seq_lens[b] receives the new token when
 *                 seq_lens[b] < capacity; otherwise the token is dropped).
 *   seq_lens      [B] int32 device, lengths before the step (read only).
 *   seq_lens_out  [B] int32 device, required, must not overlap seq_lens:
 *                 receives min(seq_lens[b] + 1, capacity), the lengths the
 *                 attention used.
 *   kv_token_offsets  [B] int64 device first row of each sequence, or NULL
 *                 for b * capacity.
 *   out           [B, h_q, d_head] fp32 or bf16 (out_dtype).
 * Same result, bit for bit, as gqa_kv_append followed by gqa_decode_attn_ex
 * with explicit offsets (b * capacity when NULL here), s_kv_hint = capacity
 * and the same n_splits. The split count defaults to gqa_decode_pick_splits_d(B, h_kv,
 * d_head, capacity, 0), the workspace to gqa_decode_workspace_bytes for it (NULL:
 * library-owned). bf16 only (GQA_ERR_UNSUPPORTED otherwise). Asynchronous on
 * `stream`; no host synchronisation, allocation (given a workspace) or memset,
 * so a graph of one step can be replayed while the lengths grow.
 */
int gqa_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* seq_lens, int32_t* seq_lens_out, const int64_t* kv_token_offsets,
                    void* out, int B, int h_q, int h_kv, int d_head, float scale, int n_splits,
                    int in_dtype, int out_dtype, int64_t capacity, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Sequence-sharded attention (the kernbench2 page's scheme: every shard
 * holds a slice of each sequence's KV and all of q; shards exchange (m, l, o)
 * triplets and merge them exactly).
 *
 * gqa_decode_attn_triplet computes this shard's attention over its own KV
 * (same arguments as gqa_decode_attn_ex) but, instead of o / l, writes the
 * shard's merged triplet per (b, h): ml_out[2*(b*h_q + h) + {0, 1}] = (m, l)
 * and o_out[(b*h_q + h)*d_head + i], with m = max_t x_t, l = sum_t 2^(x_t - m),
 * o = sum_t 2^(x_t - m) V_t and x_t = scale * log2(e) * <q, K_t> (log2 units).
 * A shard with no tokens of a sequence gives (-inf, 0, 0).
 *
 * gqa_merge_triplets merges `parts` such triplet sets laid out part-major
 * (ml [parts][rows][2], o [parts][rows][d_head], e.g. gathered from the
 * shards) into out [rows, d_head] = (sum_p 2^(m_p - M) o_p) / (sum_p 2^(m_p - M) l_p),
 * M = max_p m_p; rows with nothing attended give zeros. fp32 or bf16 out.
 */
int gqa_decode_attn_triplet(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int64_t* kv_token_offsets,
                            float* ml_out, float* o_out, int B, int h_q, int h_kv, int d_head,
                            float scale, int n_splits, int in_dtype, int64_t s_kv_hint,
                            void* workspace, size_t workspace_bytes, hipStream_t stream, int flags);

int gqa_merge_triplets(const float* ml, const float* o, int parts, int rows, int d_head,
                       void* out, int out_dtype, hipStream_t stream);

/*
 * The two halves of gqa_decode_attn_ex, for callers that combine partial
 * results from several sources (e.g. KV sharded across GPUs along the
 * sequence: each GPU writes its triplets, they are exchanged, one merge
 * follows) or that time the kernels separately.
 *
 * gqa_decode_partial runs only the split kernel: for every sequence b, query
 * head h and chunk s < n_active(b) it writes, in `workspace`,
 *   o[((b*h_q + h)*n + s)*d_head + i]   unnormalised sum_t 2^(x_t - m) V_t[i]  (fp32)
 *   ml[(b*h_q + h)*n + s] = (m, l)      m = max_t x_t, l = sum_t 2^(x_t - m)  (fp32 pairs)
 * where x_t = scale * log2(e) * <q, K_t> (scores in log2 units), n is the
 * split count used, and `o` and `ml` sit where gqa_decode_workspace_bytes
 * describes. Chunk s covers tokens
 * [s*c, min(S_b, (s+1)*c)) with c = max(ceil(S_b / n), f), f = 1 when
 * n_splits > 0; with a length hint 32 for B <= 4 and 128 for larger
 * batches; without one (a single query token), ceil(S_b / 32) rounded up to
 * a multiple of 32, clamped to [32, 128]; n_active(b) = ceil(S_b / c). Other
 * slots are left untouched. A workspace is required.
 *
 * gqa_decode_merge reads those triplets and writes out = o / l per (b, h),
 * merged exactly over the chunks. It must be given the seq_lens, shape,
 * n_splits and s_kv_hint of the gqa_decode_partial call that filled the
 * workspace (they fix n and the chunking), and run after it on the stream.
 * Arguments otherwise as in gqa_decode_attn_ex.
 */
int gqa_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int64_t* kv_token_offsets,
                       int B, int h_q, int h_kv, int d_head, float scale, int n_splits,
                       int in_dtype, int64_t s_kv_hint, void* workspace, size_t workspace_bytes,
                       hipStream_t stream, int flags);

int gqa_decode_merge(const int32_t* seq_lens, const void* workspace, size_t workspace_bytes,
                     void* out, int B, int h_q, int h_kv, int d_head, int n_splits,
                     int64_t s_kv_hint, int out_dtype, hipStream_t stream);

/*
 * Split count the library uses when n_splits <= 0: enough workgroups that
 * every compute unit has work at B = 1 (s_kv_max = 0, no length known: one
 * sequence with d_head = 128 gets num_cus / h_kv chunks, one 8-wave
 * workgroup per compute unit, each chunk sized on the device; otherwise four
 * rounds of two workgroups per compute unit, with the chunk floor of a
 * hint-less call, see gqa_decode_partial, so short sequences leave most
 * chunks empty); when s_kv_max > 0 is known, also
 * enough that the longest sequence's chunks fill about two rounds of the
 * resident workgroup slots (B = 1) or B / 2 up to four (B > 1, where lengths
 * may differ),
 * with chunks of 128 to 4096 tokens; at most GQA_MAX_SPLITS. Exceptions for
 * a single sequence: with d_head = 128, one that one workgroup per compute
 * unit covers in chunks of 256 to 2048 tokens gets exactly that many chunks
 * (num_cus / h_kv), which the library runs with 8-wave workgroups; short
 * sequences in a batch of at most 4 get up to num_cus / (B * h_kv) chunks of
 * at least 32 tokens.
 * num_cus <= 0 queries the current device (returns a negative status if that
 * fails). Pure host arithmetic otherwise. GQA_ERR_UNSUPPORTED for a d_head
 * other than 64 or 128.
 */
int gqa_decode_pick_splits_d(int B, int h_kv, int d_head, int64_t s_kv_max, int num_cus);

/* gqa_decode_pick_splits_d for d_head = 128. */
int gqa_decode_pick_splits(int B, int h_kv, int64_t s_kv_max, int num_cus);

/* Split count gqa_decode_attn_multi uses when n_splits <= 0 (the same rule,
 * for its kernels: with two column tiles per workgroup, one workgroup per CU,
 * one round of them for a single sequence; with eight (one per wave), two
 * workgroups per CU, one round for a single sequence and up to two for a
 * batch; with sixteen (two per wave), one per CU; one tile of several query
 * tokens with d_head = 128 as gqa_decode_pick_splits_d, the 8-wave round
 * included; chunks of up to 16384 tokens). s_kv_max is also the hint that
 * picks the kernel (see gqa_decode_attn_multi). Negative status on invalid
 * arguments or a failed device query; GQA_ERR_UNSUPPORTED for a d_head other
 * than 64 or 128. */
int gqa_decode_multi_splits_d(int B, int S_q, int h_q, int h_kv, int d_head, int64_t s_kv_max, int num_cus);

/* gqa_decode_multi_splits_d for d_head = 128. */
int gqa_decode_multi_splits(int B, int S_q, int h_q, int h_kv, int64_t s_kv_max, int num_cus);

/* Workspace bytes for n_splits chunks. Layout, each part starting on a
 * 256-byte boundary:
 *   counters  B*h_q uint64 at byte 0 (arrival counters of GQA_FLAG_FUSED calls;
 *             any initial contents are fine, each call tags its counts)
 *   o         [B, h_q, n_splits, d_head] fp32 at C = round_up(B*h_q*8, 256)
 *   (m, l)    [B, h_q, n_splits] fp32 pairs at C + round_up(B*h_q*n_splits*d_head*4, 256)
 *   tok       [B] int64 after (m, l), at the next 256-byte boundary: with the
 *             packed layout (no kv_token_offsets) and more than 256 sequences,
 *             a call first writes each sequence's first token row here (one
 *             scan launch) instead of summing seq_lens in every split workgroup
 * Calls that share a workspace must not overlap in time.
 * 0 for invalid arguments. */
size_t gqa_decode_workspace_bytes(int B, int h_q, int d_head, int n_splits);

/*
 * Profiling: make the calling thread's following gqa_decode_attn* calls
 * record `before` on their stream right before the split kernel and `after`
 * right after it (events created by the caller with hipEventCreate), so
 * hipEventElapsedTime(before, after) is that kernel's duration. NULL, NULL
 * turns it off. Host-only; returns GQA_OK or GQA_ERR_INVALID_ARG if only one
 * event is given.
 */
int gqa_decode_set_split_events(hipEvent_t before, hipEvent_t after);

/* Static description of a status code. */
const char* gqa_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
