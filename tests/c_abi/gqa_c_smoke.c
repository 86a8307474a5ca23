/*
 * The C boundary used from plain C, without Python or PyTorch: device memory
 * from hipMalloc, a stream from hipStreamCreate, the library's entry points
 * straight from include/gqa_decode.h.
 *
 *   gqa_c_smoke <inputs.bin> <out.bin>
 *
 * inputs.bin (little-endian): int32 B, h_q, h_kv, d_head, n_splits (0: the
 * library's heuristic), T (token rows of the packed cache); float32 scale;
 * then q [B, h_q, d] bf16 bits, k and v [T, h_kv, d] bf16 bits, seq_lens [B]
 * int32. out.bin receives out [B, h_q, d] fp32 of gqa_decode_attn_ex (caller
 * workspace, caller stream).
 *
 * Also checks, and fails with a message otherwise: gqa_decode_attn (default
 * stream, library workspace, same split count, no length hint) gives the same
 * bytes as gqa_decode_attn_ex without a hint; an
 * unsupported head size is refused on the host with GQA_ERR_UNSUPPORTED and a
 * message; gqa_decode_workspace_bytes is positive.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gqa_decode.h"

#define HIP_OK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s inputs.bin out.bin\n", argv[0]);
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[6];
  float scale;
  if (read_all(f, hdr, sizeof hdr) || read_all(f, &scale, sizeof scale)) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int B = hdr[0], h_q = hdr[1], h_kv = hdr[2], d = hdr[3], n_splits_in = hdr[4], T = hdr[5];
  if (B < 1 || h_q < 1 || h_kv < 1 || d < 1 || T < 0) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  const size_t nq = (size_t)B * h_q * d, nkv = (size_t)T * h_kv * d;
  uint16_t* q = malloc(nq * 2);
  uint16_t* k = malloc(nkv * 2 + 2);
  uint16_t* v = malloc(nkv * 2 + 2);
  int32_t* lens = malloc((size_t)B * 4);
  float* out1 = malloc(nq * 4);
  float* out2 = malloc(nq * 4);
  if (!q || !k || !v || !lens || !out1 || !out2) return 1;
  if (read_all(f, q, nq * 2) || read_all(f, k, nkv * 2) || read_all(f, v, nkv * 2) ||
      read_all(f, lens, (size_t)B * 4)) {
    fprintf(stderr, "short body\n");
    return 1;
  }
  fclose(f);
  int64_t s_max = 0;
  for (int b = 0; b < B; ++b) s_max = lens[b] > s_max ? lens[b] : s_max;

  void *dq, *dk, *dv, *dlens, *dout, *dout2, *dws;
  HIP_OK(hipMalloc(&dq, nq * 2));
  HIP_OK(hipMalloc(&dk, nkv * 2 + 16));
  HIP_OK(hipMalloc(&dv, nkv * 2 + 16));
  HIP_OK(hipMalloc(&dlens, (size_t)B * 4));
  HIP_OK(hipMalloc(&dout, nq * 4));
  HIP_OK(hipMalloc(&dout2, nq * 4));
  HIP_OK(hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, k, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, (size_t)B * 4, hipMemcpyHostToDevice));

  const int ns = n_splits_in > 0 ? n_splits_in : gqa_decode_pick_splits_d(B, h_kv, d, s_max, 0);
  if (ns < 1) {
    fprintf(stderr, "gqa_decode_pick_splits_d: %d (%s)\n", ns, gqa_last_error());
    return 3;
  }
  const size_t ws_bytes = gqa_decode_workspace_bytes(B, h_q, d, ns);
  if (ws_bytes == 0) {
    fprintf(stderr, "gqa_decode_workspace_bytes returned 0\n");
    return 3;
  }
  HIP_OK(hipMalloc(&dws, ws_bytes));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  int r = gqa_decode_attn_ex(dq, dk, dv, (const int32_t*)dlens, NULL, dout, B, h_q, h_kv, d, scale, ns,
                             GQA_DTYPE_BF16, GQA_DTYPE_F32, s_max, dws, ws_bytes, st, 0);
  if (r != GQA_OK) {
    fprintf(stderr, "gqa_decode_attn_ex: %s (%s)\n", gqa_status_string(r), gqa_last_error());
    return 3;
  }
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(out1, dout, nq * 4, hipMemcpyDeviceToHost));
  /* without the hint, as the base entry point has none (a hint may choose another
     workgroup form, whose results differ in rounding) */
  r = gqa_decode_attn_ex(dq, dk, dv, (const int32_t*)dlens, NULL, dout, B, h_q, h_kv, d, scale, ns,
                         GQA_DTYPE_BF16, GQA_DTYPE_F32, 0, dws, ws_bytes, st, 0);
  if (r != GQA_OK) {
    fprintf(stderr, "gqa_decode_attn_ex (no hint): %s (%s)\n", gqa_status_string(r), gqa_last_error());
    return 3;
  }
  HIP_OK(hipStreamSynchronize(st));
  r = gqa_decode_attn(dq, dk, dv, (const int32_t*)dlens, dout2, B, h_q, h_kv, d, scale, ns);
  if (r != GQA_OK) {
    fprintf(stderr, "gqa_decode_attn: %s (%s)\n", gqa_status_string(r), gqa_last_error());
    return 3;
  }
  HIP_OK(hipDeviceSynchronize());
  float* out3 = malloc(nq * 4);
  if (!out3) return 1;
  HIP_OK(hipMemcpy(out3, dout, nq * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out2, dout2, nq * 4, hipMemcpyDeviceToHost));
  if (memcmp(out3, out2, nq * 4) != 0) {
    fprintf(stderr, "gqa_decode_attn and gqa_decode_attn_ex differ\n");
    return 4;
  }
  r = gqa_decode_attn_ex(dq, dk, dv, (const int32_t*)dlens, NULL, dout, B, h_q, h_kv, 96, scale, ns,
                         GQA_DTYPE_BF16, GQA_DTYPE_F32, s_max, dws, ws_bytes, st, 0);
  if (r != GQA_ERR_UNSUPPORTED || !gqa_status_string(r) || gqa_last_error()[0] == '\0') {
    fprintf(stderr, "d_head = 96 gave %d, expected GQA_ERR_UNSUPPORTED with a message\n", r);
    return 5;
  }

  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(out1, 4, nq, o) != nq) {
    perror(argv[2]);
    return 1;
  }
  fclose(o);
  printf("gqa_c_smoke: B=%d h_q=%d h_kv=%d d=%d n_splits=%d ok\n", B, h_q, h_kv, d, ns);
  HIP_OK(hipStreamDestroy(st));
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dlens); hipFree(dout); hipFree(dout2); hipFree(dws);
  free(q); free(k); free(v); free(lens); free(out1); free(out2); free(out3);
  return 0;
}
