/*
 * Host-side checks of libusp that need no GPU: the range splits, the
 * head-chunk plan, the workspace size, and the rejection of invalid calls
 * (every call below fails its argument checks before any HIP call). Pointer
 * arrays are heap blocks of exactly the documented length, so a build of the
 * library with the host AddressSanitizer reports any read or write past
 * them. Built by ulysses_sequence_attention_amd/build.py (build_host_check)
 * against an ASan-instrumented libusp; run by tests/test_host_asan.py.
 * Exit status 0 and the line "usp host check: ok" mean every check passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "usp.h"

static int failures = 0;

#define EXPECT(cond, ...)                                          \
  do {                                                             \
    if (!(cond)) {                                                 \
      ++failures;                                                  \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);         \
      fprintf(stderr, __VA_ARGS__);                                \
      fputc('\n', stderr);                                         \
    }                                                              \
  } while (0)

/* A status and a non-empty message for it. */
#define EXPECT_ERR(call, code)                                                         \
  do {                                                                                 \
    const int st_ = (call);                                                            \
    EXPECT(st_ == (code), "%s returned %d, expected %d", #call, st_, (int)(code));     \
    EXPECT(strlen(usp_last_error()) > 0, "%s left no message", #call);                 \
  } while (0)

/* Stand-ins for device pointers: 16-byte aligned, never dereferenced. */
static void* fake(int i) { return (void*)(uintptr_t)(0x100000u + 16u * (unsigned)i); }

/* A heap array of exactly n stand-in pointers, entry `null_at` NULL. */
static void** fakes(int n, int null_at) {
  void** a = (void**)malloc(sizeof(void*) * (size_t)n);
  for (int i = 0; i < n; ++i) a[i] = i == null_at ? NULL : fake(i + 1);
  return a;
}

static void check_ranges(void) {
  for (int64_t total = 1; total <= 260; ++total) {
    for (int32_t parts = 1; parts <= 70 && parts <= total; ++parts) {
      int64_t* b = (int64_t*)malloc(sizeof(int64_t) * (size_t)(parts + 1));
      const int st = usp_balanced_ranges(total, parts, b);
      EXPECT(st == USP_OK, "usp_balanced_ranges(%lld, %d) = %d", (long long)total, parts, st);
      if (st == USP_OK) {
        EXPECT(usp_last_error()[0] == '\0', "message left after success");
        const int64_t base = total / parts, extra = total % parts;
        EXPECT(b[0] == 0 && b[parts] == total, "ends of %lld / %d", (long long)total, parts);
        for (int32_t r = 0; r < parts; ++r)
          EXPECT(b[r + 1] - b[r] == base + (r < extra ? 1 : 0), "range %d of %lld / %d", r,
                 (long long)total, parts);
      }
      free(b);
    }
  }
  int64_t* b = (int64_t*)malloc(sizeof(int64_t) * 4);
  EXPECT_ERR(usp_balanced_ranges(2, 3, b), USP_EINVAL);
  EXPECT_ERR(usp_balanced_ranges(5, 0, b), USP_EINVAL);
  EXPECT_ERR(usp_balanced_ranges(5, 3, NULL), USP_EINVAL);
  free(b);
}

static void check_head_chunks(void) {
  for (int32_t heads = 1; heads <= 80; ++heads) {
    for (int32_t chunks = 1; chunks <= heads; ++chunks) {
      int32_t* b = (int32_t*)malloc(sizeof(int32_t) * (size_t)(chunks + 1));
      const int32_t c = (heads + chunks - 1) / chunks;
      const int valid = (int64_t)(chunks - 1) * c < heads;
      const int st = usp_head_chunk_ranges(heads, chunks, b);
      if (valid) {
        EXPECT(st == USP_OK, "usp_head_chunk_ranges(%d, %d) = %d", heads, chunks, st);
        if (st == USP_OK)
          for (int32_t i = 0; i <= chunks; ++i)
            EXPECT(b[i] == (i * c < heads ? i * c : heads), "bound %d of %d / %d", i, heads, chunks);
      } else {
        EXPECT(st == USP_EINVAL, "usp_head_chunk_ranges(%d, %d) = %d, expected a rejection", heads,
               chunks, st);
      }
      free(b);
    }
  }
  int32_t b[4];
  EXPECT_ERR(usp_head_chunk_ranges(0, 1, b), USP_EINVAL);
  EXPECT_ERR(usp_head_chunk_ranges(3, 4, b), USP_EINVAL);
  EXPECT_ERR(usp_head_chunk_ranges(3, 1, NULL), USP_EINVAL);
}

static void check_workspace(void) {
  size_t n = 1;
  EXPECT(usp_attention_workspace_bytes(USP_F32, 1, 1000, 4, 64, &n) == USP_OK && n == 0, "fp32 size");
  EXPECT(usp_attention_workspace_bytes(USP_BF16, 1, 32760, 5, 128, &n) == USP_OK &&
             n == (size_t)128 * 5 * 2 * 256 * 131 * 4,
         "video-DiT share size %zu", n);
  EXPECT(usp_attention_workspace_bytes(USP_BF16, 2, 257, 3, 64, &n) == USP_OK &&
             n == (size_t)2 * 3 * 2 * 2 * 256 * 67 * 4,
         "ragged size %zu", n);
  EXPECT_ERR(usp_attention_workspace_bytes(USP_BF16, 1, 16, 2, 64, NULL), USP_EINVAL);
  EXPECT_ERR(usp_attention_workspace_bytes(USP_BF16, 0, 16, 2, 64, &n), USP_ESHAPE);
  EXPECT_ERR(usp_attention_workspace_bytes((usp_dtype)7, 1, 16, 2, 64, &n), USP_EDTYPE);
}

static void check_relayout_rejections(void) {
  const int P = 8;
  void** blk = fakes(P, -1);
  void** blk_null = fakes(P, P - 1);
  void** blk65 = fakes(USP_MAX_PARTS + 1, -1);
  void* seq = fake(0);
  void* odd = (void*)((uintptr_t)fake(0) + 8);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk65, USP_BF16, 1, 640, 128, 64, USP_MAX_PARTS + 1, -1, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk_null, USP_BF16, 1, 64, 40, 128, P, -1, NULL), USP_EINVAL);
  EXPECT_ERR(usp_unpack_heads_to_seq((const void* const*)blk_null, seq, USP_BF16, 1, 64, 40, 128, P, 0,
                                     NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads(odd, blk, USP_BF16, 1, 64, 40, 128, P, -1, NULL), USP_EALIGN);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk, (usp_dtype)7, 1, 64, 40, 128, P, -1, NULL), USP_EDTYPE);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk, USP_BF16, 1, 64, 40, 4, P, -1, NULL), USP_EALIGN);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk, USP_BF16, 1, 64, 40, 128, P, P, NULL), USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk, USP_BF16, 1, 7, 40, 128, P, -1, NULL), USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, blk, USP_BF16, 0, 64, 40, 128, P, -1, NULL), USP_ESHAPE);
  EXPECT_ERR(usp_pack_seq_to_heads(seq, NULL, USP_BF16, 1, 64, 40, 128, P, -1, NULL), USP_EINVAL);
  /* head-chunk phases: ragged groups, an empty or outside chunk */
  EXPECT_ERR(usp_pack_seq_to_heads_chunk(seq, blk, USP_BF16, 1, 64, 42, 128, P, -1, 0, 2, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads_chunk(seq, blk, USP_BF16, 1, 64, 40, 128, P, -1, 2, 2, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_unpack_heads_to_seq_chunk((const void* const*)blk, seq, USP_BF16, 1, 64, 40, 128, P,
                                           -1, 4, 6, NULL),
             USP_EINVAL);
  /* several tensors in one launch: too many, a NULL in the last plane */
  void** seqs3 = fakes(3, -1);
  void** seqs3_null = fakes(3, 2);
  void** blk3 = fakes(3 * P, -1);
  void** blk3_null = fakes(3 * P, 3 * P - 1);
  void** seqs5 = fakes(USP_MAX_PLANES + 1, -1);
  void** blk5 = fakes((USP_MAX_PLANES + 1) * P, -1);
  EXPECT_ERR(usp_pack_seq_to_heads_planes(USP_MAX_PLANES + 1, (const void* const*)seqs5, blk5, USP_BF16,
                                          1, 64, 40, 128, P, -1, 0, 0, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads_planes(3, (const void* const*)seqs3, blk3_null, USP_BF16, 1, 64, 40,
                                          128, P, -1, 0, 0, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_unpack_heads_to_seq_planes(3, (const void* const*)blk3, seqs3_null, USP_BF16, 1, 64,
                                            40, 128, P, 0, 0, 0, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_pack_seq_to_heads_planes(0, (const void* const*)seqs3, blk3, USP_BF16, 1, 64, 40, 128,
                                          P, -1, 0, 0, NULL),
             USP_EINVAL);
  free(blk); free(blk_null); free(blk65); free(seqs3); free(seqs3_null); free(blk3); free(blk3_null);
  free(seqs5); free(blk5);
}

static void check_rows_rejections(void) {
  const int P = 4;
  void** sh = fakes(P, -1);
  void** sh_null = fakes(P, P - 1);
  void** sh65 = fakes(USP_MAX_PARTS + 1, -1);
  void* full = fake(0);
  EXPECT_ERR(usp_scatter_rows(full, sh_null, USP_BF16, 1, 100, 5120, P, -1, NULL), USP_EINVAL);
  EXPECT_ERR(usp_gather_rows((const void* const*)sh_null, full, USP_BF16, 1, 100, 5120, P, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_reduce_scatter_rows((const void* const*)sh_null, sh, USP_BF16, 1, 100, 5120, P, -1, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_scatter_rows(full, sh65, USP_BF16, 1, 100, 5120, USP_MAX_PARTS + 1, -1, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_gather_rows((const void* const*)sh, full, USP_BF16, 1, 3, 5120, P, NULL), USP_EINVAL);
  EXPECT_ERR(usp_scatter_rows(full, sh, USP_BF16, 1, 100, 4, P, -1, NULL), USP_EALIGN);
  EXPECT_ERR(usp_scatter_rows(full, sh, (usp_dtype)5, 1, 100, 5120, P, -1, NULL), USP_EDTYPE);
  free(sh); free(sh_null); free(sh65);
}

static void check_attention_rejections(void) {
  void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4), *ws = fake(5);
  void* odd = (void*)((uintptr_t)fake(6) + 4);
  size_t need = 0;
  EXPECT(usp_attention_workspace_bytes(USP_BF16, 1, 1000, 4, 128, &need) == USP_OK, "size");
  EXPECT_ERR(usp_attention_fwd(NULL, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0, 4, 0.f, NULL, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 2, 2, 0.f, NULL, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd(q, k, v, o, USP_BF16, USP_F32, 0, 1000, 4, 128, 0, 4, 0.f, NULL, NULL),
             USP_ESHAPE);
  EXPECT_ERR(usp_attention_fwd(q, k, v, o, USP_F32, USP_BF16, 1, 1000, 4, 64, 0, 4, 0.f, NULL, NULL),
             USP_EDTYPE);
  EXPECT_ERR(usp_attention_fwd(q, k, v, odd, USP_BF16, USP_F32, 1, 1000, 4, 128, 0, 4, 0.f, NULL, NULL),
             USP_EALIGN);
  EXPECT_ERR(usp_attention_fwd_ws(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0, 4, 0.f, NULL, NULL,
                                  need, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_ws(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0, 4, 0.f, NULL, ws,
                                  need - 1, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_ws(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0, 4, 0.f, NULL, odd,
                                  need, NULL),
             USP_EALIGN);
  /* the static scratch holds 192 MiB: 40 heads of the video-DiT shape do not fit */
  EXPECT_ERR(usp_attention_fwd_noalloc(q, k, v, o, USP_BF16, USP_BF16, 1, 32760, 40, 128, 0, 40, 0.f,
                                       NULL, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_gqa(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 6, 4, 128, 0, 6, 0.f, NULL,
                                   NULL, 0, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_block(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 0, 4, 4, 128, 0, 4, 0.f,
                                     NULL, NULL, 0, NULL),
             USP_ESHAPE);
  EXPECT_ERR(usp_attention_fwd_block_whole(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 0, 4, 4, 128, 0, 4,
                                           0.f, NULL, NULL),
             USP_ESHAPE);
  EXPECT_ERR(usp_attention_fwd_block_whole(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 500, 6, 4, 128, 0, 6,
                                           0.f, NULL, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_block_whole(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 500, 4, 4, 96, 0, 4,
                                           0.f, NULL, NULL),
             USP_ENOSYS);
  EXPECT_ERR(usp_attention_merge((const float*)q, (const float*)k, (const float*)q, (const float*)k, q,
                                 NULL, USP_BF16, 1, 100, 4, 128, 0, 4, NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_chunked(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0.f, NULL, 5,
                                       NULL),
             USP_EINVAL);
  EXPECT_ERR(usp_attention_fwd_chunked_ws(q, k, v, o, USP_BF16, USP_F32, 1, 1000, 4, 128, 0.f, NULL, 2,
                                          NULL, 0, NULL),
             USP_EINVAL);
}

int main(void) {
  EXPECT(usp_version() && strlen(usp_version()) > 0, "version string");
  check_ranges();
  check_head_chunks();
  check_workspace();
  check_relayout_rejections();
  check_rows_rejections();
  check_attention_rejections();
  if (failures) {
    fprintf(stderr, "usp host check: %d failure(s)\n", failures);
    return 1;
  }
  printf("usp host check: ok\n");
  return 0;
}
