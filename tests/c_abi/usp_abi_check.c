/*
 * A plain C consumer of libusp (include/usp.h) with the HIP runtime and no
 * other framework in the process: it checks that the boundary is usable as a
 * C ABI on its own; every entry point of usp.h is called. Numerical parity
 * against the oracle is the Python tests' job; this program checks what needs
 * no reference: the stated range splits (host and device), the pack -> unpack
 * and scatter -> gather round trips bit for bit, an exact reduce-scatter of
 * equal integer partials, the attention entry points that must agree bit for
 * bit (default, workspace, head-chunked with and without a workspace, grouped
 * heads against block attention with equal lengths), a result merged with
 * itself, finite outputs, and error codes with their messages. Exit status 0
 * when every check holds.
 */
#define _DEFAULT_SOURCE /* setenv, unsetenv */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "usp.h"

static int failures = 0;

#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "FAILED: " __VA_ARGS__);  \
      fprintf(stderr, "\n");                    \
      ++failures;                               \
    }                                           \
  } while (0)

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at %s\n", hipGetErrorString(e_), #call); \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

/* deterministic bf16 bits of values in [-1, 1) (xorshift, truncating fp32) */
static void fill_bf16(uint16_t* x, size_t n, uint32_t seed) {
  uint32_t s = seed * 2654435761u + 1u;
  for (size_t i = 0; i < n; ++i) {
    s ^= s << 13;
    s ^= s >> 17;
    s ^= s << 5;
    float f = (float)(s >> 8) / 8388608.0f - 1.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    x[i] = (uint16_t)(u >> 16);
  }
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes));
  return p;
}

static void check_ranges(void) {
  int64_t b[5];
  CHECK(usp_balanced_ranges(257, 3, b) == USP_OK && b[0] == 0 && b[1] == 86 && b[2] == 172 &&
            b[3] == 257, "257 tokens over 3 ranks");
  CHECK(usp_balanced_ranges(577, 4, b) == USP_OK && b[1] == 145 && b[2] == 289 && b[3] == 433 &&
            b[4] == 577, "577 tokens over 4 ranks");
  CHECK(usp_balanced_ranges(65537, 4, b) == USP_OK && b[1] == 16385 && b[4] == 65537,
        "65537 tokens over 4 ranks");
  int32_t c[4];
  CHECK(usp_head_chunk_ranges(8, 3, c) == USP_OK && c[1] == 3 && c[2] == 6 && c[3] == 8,
        "8 heads in 3 chunks");
  CHECK(usp_balanced_ranges(2, 3, b) == USP_EINVAL && strlen(usp_last_error()) > 0,
        "fewer items than parts is rejected with a message");
}

static void check_relayout(void) {
  const int64_t B = 2, S = 301;
  const int32_t H = 6, D = 64, P = 4;
  const size_t n = (size_t)B * S * H * D;
  uint16_t* host = (uint16_t*)malloc(n * 2);
  uint16_t* back = (uint16_t*)malloc(n * 2);
  fill_bf16(host, n, 7);
  int64_t hb[P + 1];
  CHECK(usp_balanced_ranges(H, P, hb) == USP_OK, "head ranges");
  void* seq = dev_alloc(n * 2);
  void* out = dev_alloc(n * 2);
  void* blk[P];
  for (int j = 0; j < P; ++j) blk[j] = dev_alloc((size_t)B * S * (hb[j + 1] - hb[j]) * D * 2);
  HIP_OK(hipMemcpy(seq, host, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(out, 0xff, n * 2));
  CHECK(usp_pack_seq_to_heads(seq, blk, USP_BF16, B, S, H, D, P, -1, NULL) == USP_OK, "pack");
  CHECK(usp_unpack_heads_to_seq((const void* const*)blk, out, USP_BF16, B, S, H, D, P, -1, NULL) ==
            USP_OK, "unpack");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(back, out, n * 2, hipMemcpyDeviceToHost));
  CHECK(memcmp(host, back, n * 2) == 0, "unpack(pack(x)) == x bit for bit");
  /* block 1 holds heads [2, 4): spot-check one element against the closed form */
  uint16_t e;
  const int64_t bb = 1, s = 17, i = 1, d = 5;
  HIP_OK(hipMemcpy(&e, (char*)blk[1] + ((((size_t)bb * S + s) * (hb[2] - hb[1]) + i) * D + d) * 2,
                   2, hipMemcpyDeviceToHost));
  CHECK(e == host[(((size_t)bb * S + s) * H + hb[1] + i) * D + d], "block element in place");
  for (int j = 0; j < P; ++j) HIP_OK(hipFree(blk[j]));
  HIP_OK(hipFree(seq));
  HIP_OK(hipFree(out));
  free(host);
  free(back);
}

/* Two tensors of one shape in one launch (the q, k, v form): the blocks the
 * planes call writes equal those of one single-tensor call per tensor, and
 * its unpack of rank 1's rows rebuilds rank 1's shards of both tensors. */
static void check_relayout_planes(void) {
  enum { T = 2, P = 3 };
  const int64_t B = 1, S = 257;
  const int32_t H = 6, D = 128;
  const size_t n = (size_t)B * S * H * D;
  int64_t hb[P + 1], tb[P + 1];
  CHECK(usp_balanced_ranges(H, P, hb) == USP_OK && usp_balanced_ranges(S, P, tb) == USP_OK,
        "plane ranges");
  uint16_t* host = (uint16_t*)malloc(n * 2 * T);
  fill_bf16(host, n, 11);
  fill_bf16(host + n, n, 12);
  void* seq[T];
  void* blk[T * P];
  void* ref[P];
  size_t bn[P];
  for (int t = 0; t < T; ++t) {
    seq[t] = dev_alloc(n * 2);
    HIP_OK(hipMemcpy(seq[t], host + t * n, n * 2, hipMemcpyHostToDevice));
  }
  for (int j = 0; j < P; ++j) {
    bn[j] = (size_t)B * S * (hb[j + 1] - hb[j]) * D;
    ref[j] = dev_alloc(bn[j] * 2);
    for (int t = 0; t < T; ++t) blk[t * P + j] = dev_alloc(bn[j] * 2);
  }
  CHECK(usp_pack_seq_to_heads_planes(T, (const void* const*)seq, blk, USP_BF16, B, S, H, D, P, -1, 0,
                                     0, NULL) == USP_OK,
        "planes pack");
  uint16_t* a = (uint16_t*)malloc(n * 2);
  uint16_t* r = (uint16_t*)malloc(n * 2);
  for (int t = 0; t < T; ++t) {
    CHECK(usp_pack_seq_to_heads(seq[t], ref, USP_BF16, B, S, H, D, P, -1, NULL) == USP_OK,
          "single-tensor pack");
    HIP_OK(hipDeviceSynchronize());
    for (int j = 0; j < P; ++j) {
      HIP_OK(hipMemcpy(a, blk[t * P + j], bn[j] * 2, hipMemcpyDeviceToHost));
      HIP_OK(hipMemcpy(r, ref[j], bn[j] * 2, hipMemcpyDeviceToHost));
      CHECK(memcmp(a, r, bn[j] * 2) == 0, "planes pack equals the single-tensor pack (tensor %d, block %d)",
            t, j);
    }
  }
  const int64_t len1 = tb[2] - tb[1];
  const size_t ns = (size_t)B * len1 * H * D;
  void* sh[T];
  for (int t = 0; t < T; ++t) {
    sh[t] = dev_alloc(ns * 2);
    HIP_OK(hipMemset(sh[t], 0xff, ns * 2));
  }
  CHECK(usp_unpack_heads_to_seq_planes(T, (const void* const*)blk, sh, USP_BF16, B, S, H, D, P, 1, 0, 0,
                                       NULL) == USP_OK,
        "planes unpack of rank 1's rows");
  HIP_OK(hipDeviceSynchronize());
  for (int t = 0; t < T; ++t) {
    HIP_OK(hipMemcpy(a, sh[t], ns * 2, hipMemcpyDeviceToHost));
    CHECK(memcmp(a, host + t * n + (size_t)tb[1] * H * D, ns * 2) == 0,
          "rank 1's shard of tensor %d bit for bit", t);
    HIP_OK(hipFree(sh[t]));
    HIP_OK(hipFree(seq[t]));
  }
  for (int j = 0; j < P; ++j) {
    HIP_OK(hipFree(ref[j]));
    for (int t = 0; t < T; ++t) HIP_OK(hipFree(blk[t * P + j]));
  }
  free(host);
  free(a);
  free(r);
}

/* The two-phase exchange: pack and unpack one head chunk at a time (equal
 * head groups of 3 heads, plan 2/1) rebuild the tensor bit for bit, and each
 * pack phase leaves the other heads of a block as they were. */
static void check_relayout_chunks(void) {
  const int64_t B = 2, S = 203;
  const int32_t H = 12, D = 64, P = 4, h = H / P;
  const size_t n = (size_t)B * S * H * D, nb = (size_t)B * S * h * D;
  uint16_t* host = (uint16_t*)malloc(n * 2);
  uint16_t* back = (uint16_t*)malloc(n * 2);
  uint16_t* hblk = (uint16_t*)malloc(nb * 2);
  fill_bf16(host, n, 11);
  int32_t kc[3];
  CHECK(usp_head_chunk_ranges(h, 2, kc) == USP_OK && kc[1] == 2 && kc[2] == 3, "chunk plan 2/1");
  void* seq = dev_alloc(n * 2);
  void* out = dev_alloc(n * 2);
  void* blk[P];
  for (int j = 0; j < P; ++j) {
    blk[j] = dev_alloc(nb * 2);
    HIP_OK(hipMemset(blk[j], 0xff, nb * 2));
  }
  HIP_OK(hipMemcpy(seq, host, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(out, 0xff, n * 2));
  CHECK(usp_pack_seq_to_heads_chunk(seq, blk, USP_BF16, B, S, H, D, P, -1, kc[0], kc[1], NULL) ==
            USP_OK, "pack chunk 0");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hblk, blk[3], nb * 2, hipMemcpyDeviceToHost));
  int ok_first = 1;
  for (size_t row = 0; row < (size_t)B * S; ++row)
    for (int i = 0; i < h; ++i)
      for (int d = 0; d < D; ++d) {
        const uint16_t got = hblk[(row * h + i) * D + d];
        const uint16_t want = i < kc[1] ? host[(row * H + 3 * h + i) * D + d] : 0xffff;
        ok_first &= got == want;
      }
  CHECK(ok_first, "first phase: its heads moved, the others untouched");
  CHECK(usp_pack_seq_to_heads_chunk(seq, blk, USP_BF16, B, S, H, D, P, -1, kc[1], kc[2], NULL) ==
            USP_OK, "pack chunk 1");
  for (int c = 0; c < 2; ++c)
    CHECK(usp_unpack_heads_to_seq_chunk((const void* const*)blk, out, USP_BF16, B, S, H, D, P, -1,
                                        kc[c], kc[c + 1], NULL) == USP_OK, "unpack chunk");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(back, out, n * 2, hipMemcpyDeviceToHost));
  CHECK(memcmp(host, back, n * 2) == 0, "chunk phases: unpack(pack(x)) == x bit for bit");
  CHECK(usp_pack_seq_to_heads_chunk(seq, blk, USP_BF16, B, S, 10, D, P, -1, 0, 1, NULL) ==
            USP_EINVAL && strlen(usp_last_error()) > 0, "ragged head groups rejected");
  for (int j = 0; j < P; ++j) HIP_OK(hipFree(blk[j]));
  HIP_OK(hipFree(seq));
  HIP_OK(hipFree(out));
  free(host);
  free(back);
  free(hblk);
}

static void check_attention(void) {
  const int64_t B = 1, S = 700;
  const int32_t h = 3, D = 128;
  const size_t n = (size_t)B * S * h * D;
  uint16_t* host = (uint16_t*)malloc(n * 2);
  void* qkv[3];
  for (int t = 0; t < 3; ++t) {
    fill_bf16(host, n, 11 + t);
    qkv[t] = dev_alloc(n * 2);
    HIP_OK(hipMemcpy(qkv[t], host, n * 2, hipMemcpyHostToDevice));
  }
  float* o[3];
  float* lse[3];
  for (int r = 0; r < 3; ++r) {
    o[r] = (float*)dev_alloc(n * 4);
    lse[r] = (float*)dev_alloc((size_t)B * h * S * 4);
  }
  size_t ws_bytes = 0;
  CHECK(usp_attention_workspace_bytes(USP_BF16, B, S, h, D, &ws_bytes) == USP_OK && ws_bytes > 0,
        "workspace size");
  void* ws = dev_alloc(ws_bytes);
  CHECK(usp_attention_fwd(qkv[0], qkv[1], qkv[2], o[0], USP_BF16, USP_F32, B, S, h, D, 0, h, 0.0f,
                          lse[0], NULL) == USP_OK, "usp_attention_fwd");
  CHECK(usp_attention_fwd_ws(qkv[0], qkv[1], qkv[2], o[1], USP_BF16, USP_F32, B, S, h, D, 0, h,
                             0.0f, lse[1], ws, ws_bytes, NULL) == USP_OK, "usp_attention_fwd_ws");
  CHECK(usp_attention_fwd_chunked(qkv[0], qkv[1], qkv[2], o[2], USP_BF16, USP_F32, B, S, h, D, 0.0f,
                                  lse[2], 2, NULL) == USP_OK, "usp_attention_fwd_chunked");
  HIP_OK(hipDeviceSynchronize());
  float* chunked_ws_out = (float*)dev_alloc(n * 4);
  CHECK(usp_attention_fwd_chunked_ws(qkv[0], qkv[1], qkv[2], chunked_ws_out, USP_BF16, USP_F32, B, S,
                                     h, D, 0.0f, NULL, 2, ws, ws_bytes, NULL) == USP_OK,
        "usp_attention_fwd_chunked_ws");
  HIP_OK(hipDeviceSynchronize());
  float* a = (float*)malloc(n * 4);
  float* b = (float*)malloc(n * 4);
  HIP_OK(hipMemcpy(a, o[0], n * 4, hipMemcpyDeviceToHost));
  int finite = 1;
  for (size_t i = 0; i < n; ++i) finite &= isfinite(a[i]) && fabsf(a[i]) <= 1.0f;
  CHECK(finite, "outputs finite and within the range of V");
  for (int r = 1; r < 3; ++r) {
    HIP_OK(hipMemcpy(b, o[r], n * 4, hipMemcpyDeviceToHost));
    CHECK(memcmp(a, b, n * 4) == 0, "attention path %d equals the default bit for bit", r);
  }
  HIP_OK(hipMemcpy(b, chunked_ws_out, n * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, n * 4) == 0, "chunked attention with a workspace equals the default bit for bit");
  /* the no-allocation form reuses chunked_ws_out: its scratch is the library's */
  CHECK(usp_attention_fwd_noalloc(qkv[0], qkv[1], qkv[2], chunked_ws_out, USP_BF16, USP_F32, B, S, h,
                                  D, 0, h, 0.0f, NULL, NULL) == USP_OK, "usp_attention_fwd_noalloc");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(b, chunked_ws_out, n * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, n * 4) == 0, "attention without allocation equals the default bit for bit");
  /* with the library's workspace pool switched off, the default call runs the
   * key-group kernel (700 keys split in halves at D = 128): the same bits */
  setenv("USP_ATTENTION_POOL", "0", 1);
  CHECK(usp_attention_fwd(qkv[0], qkv[1], qkv[2], chunked_ws_out, USP_BF16, USP_F32, B, S, h, D, 0, h,
                          0.0f, NULL, NULL) == USP_OK, "usp_attention_fwd without the pool");
  unsetenv("USP_ATTENTION_POOL");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(b, chunked_ws_out, n * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, n * 4) == 0, "the key-group kernel equals the default bit for bit");
  CHECK(usp_attention_fwd_noalloc(qkv[0], qkv[1], qkv[2], chunked_ws_out, USP_BF16, USP_F32, 2, 16384,
                                  8, D, 0, 8, 0.0f, NULL, NULL) == USP_EINVAL &&
            strstr(usp_last_error(), "scratch") != NULL,
        "a call beyond the static scratch is rejected");
  HIP_OK(hipFree(chunked_ws_out));
  const size_t nl = (size_t)B * h * S;
  HIP_OK(hipMemcpy(a, lse[0], nl * 4, hipMemcpyDeviceToHost));
  for (int r = 1; r < 3; ++r) {
    HIP_OK(hipMemcpy(b, lse[r], nl * 4, hipMemcpyDeviceToHost));
    CHECK(memcmp(a, b, nl * 4) == 0, "lse of path %d equals the default bit for bit", r);
  }
  CHECK(usp_attention_fwd(qkv[0], qkv[1], qkv[2], o[0], USP_BF16, USP_F32, B, S, h, 96, 0, h, 0.0f,
                          NULL, NULL) == USP_ENOSYS && strlen(usp_last_error()) > 0,
        "unsupported head dim rejected with a message");
  CHECK(usp_attention_fwd_ws(qkv[0], qkv[1], qkv[2], o[1], USP_BF16, USP_F32, B, S, h, D, 0, h,
                             0.0f, NULL, ws, ws_bytes - 1, NULL) == USP_EINVAL,
        "a workspace one byte short is rejected");
  for (int t = 0; t < 3; ++t) HIP_OK(hipFree(qkv[t]));
  for (int r = 0; r < 3; ++r) {
    HIP_OK(hipFree(o[r]));
    HIP_OK(hipFree(lse[r]));
  }
  HIP_OK(hipFree(ws));
  free(host);
  free(a);
  free(b);
}

static void check_device_ranges(void) {
  int64_t* d = (int64_t*)dev_alloc(5 * 8);
  int64_t h[5];
  CHECK(usp_balanced_ranges_device(577, 4, d, NULL) == USP_OK, "device ranges");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(h, d, 5 * 8, hipMemcpyDeviceToHost));
  CHECK(h[0] == 0 && h[1] == 145 && h[2] == 289 && h[3] == 433 && h[4] == 577,
        "device ranges equal the host ones");
  HIP_OK(hipFree(d));
}

/* small integers as fp32: sums of a few of them are exact */
static void fill_small_ints(float* x, size_t n, uint32_t seed) {
  uint32_t s = seed * 2654435761u + 7u;
  for (size_t i = 0; i < n; ++i) {
    s = s * 1664525u + 1013904223u;
    x[i] = (float)((int)(s >> 27) - 16);
  }
}

static void check_rows(void) {
  enum { P = 3 };
  const int64_t B = 2, S = 101, W = 64;
  const size_t n = (size_t)B * S * W;
  int64_t tb[P + 1];
  CHECK(usp_balanced_ranges(S, P, tb) == USP_OK, "row ranges");
  float* host = (float*)malloc(n * 4);
  float* back = (float*)malloc(n * 4);
  fill_small_ints(host, n, 3);
  float* full = (float*)dev_alloc(n * 4);
  float* full2 = (float*)dev_alloc(n * 4);
  void* sh[P];
  void* red[P];
  const void* parts[P];
  for (int r = 0; r < P; ++r) {
    sh[r] = dev_alloc((size_t)B * (tb[r + 1] - tb[r]) * W * 4);
    red[r] = dev_alloc((size_t)B * (tb[r + 1] - tb[r]) * W * 4);
    parts[r] = full;  /* P copies of the same partial */
  }
  HIP_OK(hipMemcpy(full, host, n * 4, hipMemcpyHostToDevice));
  CHECK(usp_scatter_rows(full, sh, USP_F32, B, S, W, P, -1, NULL) == USP_OK, "scatter");
  CHECK(usp_gather_rows((const void* const*)sh, full2, USP_F32, B, S, W, P, NULL) == USP_OK, "gather");
  CHECK(usp_reduce_scatter_rows(parts, red, USP_F32, B, S, W, P, -1, NULL) == USP_OK,
        "reduce-scatter");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(back, full2, n * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(host, back, n * 4) == 0, "gather(scatter(x)) == x bit for bit");
  int rs_ok = 1;
  for (int r = 0; r < P; ++r) {
    const int64_t len = tb[r + 1] - tb[r];
    float* got = (float*)malloc((size_t)B * len * W * 4);
    HIP_OK(hipMemcpy(got, red[r], (size_t)B * len * W * 4, hipMemcpyDeviceToHost));
    for (int64_t b = 0; b < B; ++b)
      for (int64_t i = 0; i < len * W; ++i)
        rs_ok &= got[b * len * W + i] == (float)P * host[(b * S + tb[r]) * W + i];
    free(got);
  }
  CHECK(rs_ok, "reduce-scatter of P equal integer partials is P times the rows, exactly");
  for (int r = 0; r < P; ++r) {
    HIP_OK(hipFree(sh[r]));
    HIP_OK(hipFree(red[r]));
  }
  HIP_OK(hipFree(full));
  HIP_OK(hipFree(full2));
  free(host);
  free(back);
}

static void check_block_and_merge(void) {
  const int64_t B = 1, S = 300;
  const int32_t h = 4, hkv = 2, D = 64;
  const size_t nq = (size_t)B * S * h * D, nk = (size_t)B * S * hkv * D, nl = (size_t)B * h * S;
  uint16_t* host = (uint16_t*)malloc(nq * 2);
  void *q = dev_alloc(nq * 2), *k = dev_alloc(nk * 2), *v = dev_alloc(nk * 2);
  fill_bf16(host, nq, 21);
  HIP_OK(hipMemcpy(q, host, nq * 2, hipMemcpyHostToDevice));
  fill_bf16(host, nk, 22);
  HIP_OK(hipMemcpy(k, host, nk * 2, hipMemcpyHostToDevice));
  fill_bf16(host, nk, 23);
  HIP_OK(hipMemcpy(v, host, nk * 2, hipMemcpyHostToDevice));
  float *o1 = (float*)dev_alloc(nq * 4), *o2 = (float*)dev_alloc(nq * 4), *o3 = (float*)dev_alloc(nq * 4);
  float *l1 = (float*)dev_alloc(nl * 4), *l2 = (float*)dev_alloc(nl * 4), *l3 = (float*)dev_alloc(nl * 4);
  CHECK(usp_attention_fwd_gqa(q, k, v, o1, USP_BF16, USP_F32, B, S, h, hkv, D, 0, h, 0.0f, l1, NULL,
                              0, NULL) == USP_OK, "usp_attention_fwd_gqa");
  CHECK(usp_attention_fwd_block(q, k, v, o2, USP_BF16, USP_F32, B, S, S, h, hkv, D, 0, h, 0.0f, l2,
                                NULL, 0, NULL) == USP_OK, "usp_attention_fwd_block");
  /* a result merged with itself: weights 1/2 each, so O comes back exactly */
  CHECK(usp_attention_merge(o2, l2, o2, l2, o3, l3, USP_F32, B, S, h, D, 0, h, NULL) == USP_OK,
        "usp_attention_merge");
  HIP_OK(hipDeviceSynchronize());
  float* a = (float*)malloc(nq * 4);
  float* b = (float*)malloc(nq * 4);
  HIP_OK(hipMemcpy(a, o1, nq * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b, o2, nq * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, nq * 4) == 0, "block attention with Sq = Sk equals the grouped call bit for bit");
  HIP_OK(hipMemcpy(a, o3, nq * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, nq * 4) == 0, "merging a result with itself returns it exactly");
  HIP_OK(hipMemcpy(a, l2, nl * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b, l3, nl * 4, hipMemcpyDeviceToHost));
  int lse_ok = 1;
  for (size_t i = 0; i < nl; ++i) lse_ok &= fabsf(b[i] - (a[i] + 0.69314718f)) <= 2e-6f * (1.0f + fabsf(a[i]));
  CHECK(lse_ok, "merging a result with itself adds log 2 to lse");
  /* 300 keys at D = 64 are too few to split: whole walks give the same bits */
  CHECK(usp_attention_fwd_block_whole(q, k, v, o3, USP_BF16, USP_F32, B, S, S, h, hkv, D, 0, h, 0.0f,
                                      l3, NULL) == USP_OK, "usp_attention_fwd_block_whole");
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(a, o2, nq * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b, o3, nq * 4, hipMemcpyDeviceToHost));
  CHECK(memcmp(a, b, nq * 4) == 0, "whole walks over a block too short to split equal the block call");
  void* pq = q;
  HIP_OK(hipFree(pq));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(o1));
  HIP_OK(hipFree(o2));
  HIP_OK(hipFree(o3));
  HIP_OK(hipFree(l1));
  HIP_OK(hipFree(l2));
  HIP_OK(hipFree(l3));
  free(host);
  free(a);
  free(b);
}

int main(void) {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    fprintf(stderr, "no HIP device\n");
    return 2;
  }
  printf("%s\n", usp_version());
  check_ranges();
  check_device_ranges();
  check_relayout();
  check_relayout_planes();
  check_relayout_chunks();
  check_rows();
  check_attention();
  check_block_and_merge();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("usp C ABI check: ok\n");
  return 0;
}
