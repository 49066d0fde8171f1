// libusp C ABI: argument validation, error reporting, host-side ranges and
// dispatch to the HIP kernels. See include/usp.h for the contract of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "usp_internal.h"

namespace usp {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return USP_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(USP_EHIP, "%s: %s", what, hipGetErrorString(e));
  return USP_OK;
}

// Balanced contiguous ranges (h3-blackwell-runtime distributed.py,
// balanced_ranges): base = total / parts, the first total % parts ranges take
// one extra item.
static int check_ranges(int64_t total, int32_t parts) {
  if (parts < 1) return fail(USP_EINVAL, "need at least one range (got %d)", parts);
  if (total < parts)
    return fail(USP_EINVAL, "%lld items are too few for %d ranges of one item or more",
                (long long)total, parts);
  return USP_OK;
}

static void host_bounds(int64_t total, int32_t parts, int64_t* bounds) {
  const int64_t base = total / parts, extra = total % parts;
  for (int32_t r = 0; r <= parts; ++r) bounds[r] = r * base + (r < extra ? r : extra);
}

static int esize_of(usp_dtype dt) { return dt == USP_F32 ? 4 : dt == USP_BF16 ? 2 : 0; }

// Overflow-checked product of non-negative int64 factors.
static bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

static int check_relayout(const void* seq, const void* const* blk, usp_dtype dt, int64_t B,
                          int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank) {
  if (P < 1 || P > USP_MAX_PARTS)
    return fail(USP_EINVAL, "P must be in [1, %d] (got %d)", USP_MAX_PARTS, P);
  if (S < P) return fail(USP_EINVAL, "cannot split %lld tokens over %d ranks", (long long)S, P);
  if (H < P) return fail(USP_EINVAL, "cannot split %d heads over %d ranks", H, P);
  if (rank >= P) return fail(USP_EINVAL, "rank %d out of range for P = %d", rank, P);
  if (B < 1 || D < 1) return fail(USP_ESHAPE, "B and D must be positive");
  const int es = esize_of(dt);
  if (!es) return fail(USP_EDTYPE, "unsupported dtype %d", (int)dt);
  if ((int64_t(D) * es) % 16)
    return fail(USP_EALIGN, "D * element size (%d bytes) must be a multiple of 16", D * es);
  int64_t n;
  if (!mul_ok(B, S, &n) || !mul_ok(n, H, &n) || !mul_ok(n, D, &n) || !mul_ok(n, es, &n))
    return fail(USP_ESHAPE, "tensor size overflows");
  if (!seq || !blk) return fail(USP_EINVAL, "null seq or block array");
  if (!aligned16(seq)) return fail(USP_EALIGN, "seq pointer is not 16-byte aligned");
  for (int32_t j = 0; j < P; ++j) {
    if (!blk[j]) return fail(USP_EINVAL, "block pointer %d is null", j);
    if (!aligned16(blk[j])) return fail(USP_EALIGN, "block pointer %d is not 16-byte aligned", j);
  }
  return USP_OK;
}

// One phase of the head-chunked exchange: equal head groups and a non-empty
// chunk inside a group.
static int check_chunk(int32_t H, int32_t P, int32_t head_lo, int32_t head_hi) {
  if (H % P)
    return fail(USP_EINVAL, "head-chunk relayouts need equal head groups (%d heads over %d ranks)", H, P);
  if (head_lo < 0 || head_hi > H / P || head_lo >= head_hi)
    return fail(USP_EINVAL, "head chunk [%d, %d) is empty or outside a group of %d heads", head_lo,
                head_hi, H / P);
  return USP_OK;
}

// Arguments of the row movements; `ptrs` are the P shard/partial/output
// pointers, of which only ptrs[rank] must be set when rank >= 0 and the
// array is written per rank (scatter, reduce-scatter outputs).
static int check_rows(const void* full, bool need_full, const void* const* ptrs, bool all_ptrs,
                      const void* const* ptrs2, usp_dtype dt, int64_t B, int64_t S, int64_t W,
                      int32_t P, int32_t rank) {
  if (P < 1 || P > USP_MAX_PARTS)
    return fail(USP_EINVAL, "P must be in [1, %d] (got %d)", USP_MAX_PARTS, P);
  if (S < P) return fail(USP_EINVAL, "cannot split %lld rows over %d ranks", (long long)S, P);
  if (rank >= P) return fail(USP_EINVAL, "rank %d out of range for P = %d", rank, P);
  if (B < 1 || W < 1) return fail(USP_ESHAPE, "B and W must be positive");
  const int es = esize_of(dt);
  if (!es) return fail(USP_EDTYPE, "unsupported dtype %d", (int)dt);
  if ((W * es) % 16)
    return fail(USP_EALIGN, "W * element size (%lld bytes) must be a multiple of 16",
                (long long)(W * es));
  int64_t n;
  if (!mul_ok(B, S, &n) || !mul_ok(n, W, &n) || !mul_ok(n, es, &n))
    return fail(USP_ESHAPE, "tensor size overflows");
  if (need_full) {
    if (!full) return fail(USP_EINVAL, "null full tensor");
    if (!aligned16(full)) return fail(USP_EALIGN, "full tensor is not 16-byte aligned");
  }
  for (const void* const* arr : {ptrs, ptrs2}) {
    if (!arr) continue;
    const bool all = arr == ptrs ? all_ptrs : true;
    for (int32_t j = 0; j < P; ++j) {
      if (!all && j != rank) continue;
      if (!arr[j]) return fail(USP_EINVAL, "pointer %d is null", j);
      if (!aligned16(arr[j])) return fail(USP_EALIGN, "pointer %d is not 16-byte aligned", j);
    }
  }
  return USP_OK;
}

static int check_attention(const AttnArgs& a) {
  if (!a.q || !a.k || !a.v || !a.o) return fail(USP_EINVAL, "null q, k, v or o");
  if (a.h < 1) return fail(USP_EINVAL, "h must be positive");
  if (a.h_kv < 1 || a.h_kv > a.h || a.h % a.h_kv)
    return fail(USP_EINVAL, "%d query heads cannot share %d key/value heads evenly", a.h, a.h_kv);
  if (a.head_lo < 0 || a.head_hi > a.h || a.head_lo >= a.head_hi)
    return fail(USP_EINVAL, "head range [%d, %d) is empty or outside [0, %d)", a.head_lo,
                a.head_hi, a.h);
  if (a.B < 1 || a.S < 1 || a.Sk < 1) return fail(USP_ESHAPE, "B, S and Sk must be positive");
  const int es = esize_of(a.in_dt);
  if (!es) return fail(USP_EDTYPE, "unsupported input dtype %d", (int)a.in_dt);
  if (a.out_dt != USP_F32 && a.out_dt != USP_BF16)
    return fail(USP_EDTYPE, "unsupported output dtype %d", (int)a.out_dt);
  if (a.in_dt == USP_F32 && a.out_dt != USP_F32)
    return fail(USP_EDTYPE, "fp32 inputs require an fp32 output");
  if (a.in_dt == USP_BF16 && a.D != 64 && a.D != 128)
    return fail(USP_ENOSYS, "bf16 attention supports D in {64, 128} (got %d)", a.D);
  if (a.in_dt == USP_F32 && a.D != 32 && a.D != 64 && a.D != 128)
    return fail(USP_ENOSYS, "fp32 attention supports D in {32, 64, 128} (got %d)", a.D);
  int64_t n;
  if (!mul_ok(a.B, a.S, &n) || !mul_ok(n, a.h, &n) || !mul_ok(n, a.D, &n) ||
      !mul_ok(n, 4, &n) || !mul_ok(a.B, a.Sk, &n) || !mul_ok(n, a.h_kv, &n) ||
      !mul_ok(n, a.D, &n) || !mul_ok(n, 4, &n))
    return fail(USP_ESHAPE, "tensor size overflows");
  if (a.S > (int64_t(1) << 31) - 1024 || a.Sk > (int64_t(1) << 31) - 1024 ||
      a.B * a.h > (int64_t(1) << 31) - 1)
    return fail(USP_ESHAPE, "S, Sk or B * h too large for one launch");
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.o))
    return fail(USP_EALIGN, "q, k, v and o must be 16-byte aligned");
  if (a.lse && (reinterpret_cast<uintptr_t>(a.lse) & 3u))
    return fail(USP_EALIGN, "lse must be 4-byte aligned");
  return USP_OK;
}

// ---- the workspace pool of the calls given no workspace --------------------
// A bf16 call whose keys split in halves and that brings no workspace takes
// one from a stream-ordered memory pool the library keeps per device (the
// key-half kernels and their merge, then hipFreeAsync on the same stream), so
// it runs the same kernels as the workspace form, with the same bits. The pool
// keeps freed memory for the next call (release threshold at its maximum):
// after the first calls an allocation is a pool lookup. Where the pool cannot
// be used — the stream is being captured into a graph, the allocation fails,
// or the environment sets USP_ATTENTION_POOL=0 — the call runs the key-group
// kernel, which needs no workspace and gives the same bits.
constexpr int kMaxPoolDevices = 64;
static std::mutex g_pool_mu;
static hipMemPool_t g_pool[kMaxPoolDevices];

static bool pool_allowed(hipStream_t s) {
  const char* e = getenv("USP_ATTENTION_POOL");
  if (e && e[0] == '0') return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs == hipStreamCaptureStatusNone;
}

// The pool of the device that runs `s`, created on first use; nullptr if
// the runtime refuses (the caller then runs without a workspace).
static hipMemPool_t device_pool(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxPoolDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof props);
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess || !pool) return nullptr;
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    g_pool[dev] = pool;
  }
  return g_pool[dev];
}

static int run_attention(const AttnArgs& a, hipStream_t s) {
  if (a.in_dt == USP_F32) return launch_attention_f32(a, s);
  if (!a.ws && !a.whole && attention_bf16_splits(a.Sk, a.D) && pool_allowed(s)) {
    const size_t need = attention_bf16_ws_bytes(a.B, a.S, a.head_hi - a.head_lo, a.D);
    hipMemPool_t pool = device_pool(s);
    void* ws = nullptr;
    if (pool && hipMallocFromPoolAsync(&ws, need, pool, s) == hipSuccess && ws) {
      AttnArgs b = a;
      b.ws = ws;
      b.ws_bytes = need;
      const int st = launch_attention_bf16(b, s);
      if (hipFreeAsync(ws, s) != hipSuccess && st == USP_OK)
        return fail(USP_EHIP, "hipFreeAsync of the attention workspace failed");
      return st;
    }
    (void)hipGetLastError();  // the pool could not serve: run without a workspace
  }
  return launch_attention_bf16(a, s);
}

}  // namespace usp

using namespace usp;

extern "C" {

const char* usp_last_error(void) { return g_last_error.c_str(); }

const char* usp_version(void) { return "usp 0.1.0 gfx950"; }

int usp_balanced_ranges(int64_t total, int32_t parts, int64_t* bounds) {
  if (int st = check_ranges(total, parts)) return st;
  if (!bounds) return fail(USP_EINVAL, "bounds is null");
  host_bounds(total, parts, bounds);
  return ok();
}

int usp_balanced_ranges_device(int64_t total, int32_t parts, int64_t* d_bounds, void* stream) {
  if (int st = check_ranges(total, parts)) return st;
  if (!d_bounds) return fail(USP_EINVAL, "d_bounds is null");
  if (reinterpret_cast<uintptr_t>(d_bounds) & 7u) return fail(USP_EALIGN, "d_bounds misaligned");
  if (int st = launch_ranges_device(total, parts, d_bounds, (hipStream_t)stream)) return st;
  return ok();
}

int usp_head_chunk_ranges(int32_t heads, int32_t chunks, int32_t* bounds) {
  if (heads < 1) return fail(USP_EINVAL, "heads must be positive (got %d)", heads);
  if (chunks < 1) return fail(USP_EINVAL, "chunks must be positive (got %d)", chunks);
  if (chunks > heads)
    return fail(USP_EINVAL, "cannot run %d heads in %d non-empty chunks", heads, chunks);
  if (!bounds) return fail(USP_EINVAL, "bounds is null");
  const int32_t size = (heads + chunks - 1) / chunks;
  // every chunk non-empty <=> (chunks - 1) * size < heads
  if (int64_t(chunks - 1) * size >= heads)
    return fail(USP_EINVAL, "%d chunks of %d heads leave a chunk empty for %d heads", chunks,
                size, heads);
  for (int32_t c = 0; c < chunks; ++c) bounds[c] = c * size;
  bounds[chunks] = heads;
  return ok();
}

}  // extern "C"

namespace usp {
// n planes of one relayout (one launch): the per-plane checks of the
// single-plane calls, plus the plane count and, for a head-chunk phase
// (head_hi > 0), equal head groups and a chunk inside a group.
static int relayout_planes(int32_t n, const void* const* seq, const void* const* blk, bool pack,
                           usp_dtype dtype, int64_t B, int64_t S, int32_t H, int32_t D, int32_t P,
                           int32_t rank, int32_t head_lo, int32_t head_hi, hipStream_t stream) {
  if (n < 1 || n > USP_MAX_PLANES)
    return fail(USP_EINVAL, "plane count must be in [1, %d] (got %d)", USP_MAX_PLANES, n);
  if (!seq || !blk) return fail(USP_EINVAL, "null seq or block array");
  for (int32_t t = 0; t < n; ++t)
    if (int st = check_relayout(seq[t], blk + size_t(t) * (P > 0 ? P : 0), dtype, B, S, H, D, P, rank))
      return st;
  if (head_hi > 0 || head_lo != 0)
    if (int st = check_chunk(H, P, head_lo, head_hi)) return st;
  RelayoutArgs a{n, seq, blk, B, S, H, D, P, rank < 0 ? -1 : rank, esize_of(dtype), head_lo,
                 head_hi};
  if (int st = launch_relayout(a, pack, stream)) return st;
  return ok();
}
}  // namespace usp

extern "C" {

int usp_pack_seq_to_heads(const void* seq, void* const* blk, usp_dtype dtype, int64_t B,
                          int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                          void* stream) {
  return relayout_planes(1, &seq, (const void* const*)blk, true, dtype, B, S, H, D, P, rank, 0, 0,
                         (hipStream_t)stream);
}

int usp_unpack_heads_to_seq(const void* const* blk, void* seq, usp_dtype dtype, int64_t B,
                            int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                            void* stream) {
  const void* s = seq;
  return relayout_planes(1, &s, blk, false, dtype, B, S, H, D, P, rank, 0, 0, (hipStream_t)stream);
}

int usp_pack_seq_to_heads_chunk(const void* seq, void* const* blk, usp_dtype dtype, int64_t B,
                                int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                                int32_t head_lo, int32_t head_hi, void* stream) {
  if (head_hi <= 0) return fail(USP_EINVAL, "head chunk [%d, %d) is empty", head_lo, head_hi);
  return relayout_planes(1, &seq, (const void* const*)blk, true, dtype, B, S, H, D, P, rank,
                         head_lo, head_hi, (hipStream_t)stream);
}

int usp_unpack_heads_to_seq_chunk(const void* const* blk, void* seq, usp_dtype dtype, int64_t B,
                                  int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                                  int32_t head_lo, int32_t head_hi, void* stream) {
  if (head_hi <= 0) return fail(USP_EINVAL, "head chunk [%d, %d) is empty", head_lo, head_hi);
  const void* s = seq;
  return relayout_planes(1, &s, blk, false, dtype, B, S, H, D, P, rank, head_lo, head_hi,
                         (hipStream_t)stream);
}

int usp_pack_seq_to_heads_planes(int32_t n, const void* const* seq, void* const* blk,
                                 usp_dtype dtype, int64_t B, int64_t S, int32_t H, int32_t D,
                                 int32_t P, int32_t rank, int32_t head_lo, int32_t head_hi,
                                 void* stream) {
  return relayout_planes(n, seq, (const void* const*)blk, true, dtype, B, S, H, D, P, rank,
                         head_lo, head_hi, (hipStream_t)stream);
}

int usp_unpack_heads_to_seq_planes(int32_t n, const void* const* blk, void* const* seq,
                                   usp_dtype dtype, int64_t B, int64_t S, int32_t H, int32_t D,
                                   int32_t P, int32_t rank, int32_t head_lo, int32_t head_hi,
                                   void* stream) {
  return relayout_planes(n, (const void* const*)seq, blk, false, dtype, B, S, H, D, P, rank,
                         head_lo, head_hi, (hipStream_t)stream);
}

int usp_scatter_rows(const void* full, void* const* shards, usp_dtype dtype, int64_t B, int64_t S,
                     int64_t W, int32_t P, int32_t rank, void* stream) {
  if (!shards) return fail(USP_EINVAL, "null shard array");
  if (int st = check_rows(full, true, shards, rank < 0, nullptr, dtype, B, S, W, P, rank)) return st;
  RowArgs a{const_cast<void*>(full), nullptr, shards, B, S, W, P, rank < 0 ? -1 : rank,
            esize_of(dtype)};
  if (int st = launch_rows(a, RowOp::kScatter, (hipStream_t)stream)) return st;
  return ok();
}

int usp_gather_rows(const void* const* shards, void* full, usp_dtype dtype, int64_t B, int64_t S,
                    int64_t W, int32_t P, void* stream) {
  if (!shards) return fail(USP_EINVAL, "null shard array");
  if (int st = check_rows(full, true, shards, true, nullptr, dtype, B, S, W, P, -1)) return st;
  RowArgs a{full, shards, nullptr, B, S, W, P, -1, esize_of(dtype)};
  if (int st = launch_rows(a, RowOp::kGather, (hipStream_t)stream)) return st;
  return ok();
}

int usp_reduce_scatter_rows(const void* const* partials, void* const* out, usp_dtype dtype,
                            int64_t B, int64_t S, int64_t W, int32_t P, int32_t rank,
                            void* stream) {
  if (!partials || !out) return fail(USP_EINVAL, "null partial or output array");
  if (int st = check_rows(nullptr, false, out, rank < 0, partials, dtype, B, S, W, P, rank))
    return st;
  RowArgs a{nullptr, partials, out, B, S, W, P, rank < 0 ? -1 : rank, esize_of(dtype)};
  if (int st = launch_rows(a, RowOp::kReduceScatter, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_fwd(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                      usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t D,
                      int32_t head_lo, int32_t head_hi, float scale, float* lse, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, head_lo, head_hi, scale, in_dt, out_dt, nullptr, 0, h};
  if (int st = check_attention(a)) return st;
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_workspace_bytes(usp_dtype in_dt, int64_t B, int64_t S, int32_t heads,
                                  int32_t D, size_t* bytes) {
  if (!bytes) return fail(USP_EINVAL, "bytes is null");
  if (B < 1 || S < 1 || heads < 1 || D < 1) return fail(USP_ESHAPE, "B, S, heads and D must be positive");
  if (in_dt == USP_F32) {
    *bytes = 0;
    return ok();
  }
  if (in_dt != USP_BF16) return fail(USP_EDTYPE, "unsupported input dtype %d", (int)in_dt);
  if (S > (int64_t(1) << 31) - 1024 || B * heads > (int64_t(1) << 31) - 1)
    return fail(USP_ESHAPE, "S or B * heads too large for one launch");
  *bytes = attention_bf16_ws_bytes(B, S, heads, D);
  return ok();
}

int usp_attention_fwd_ws(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                         usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t D,
                         int32_t head_lo, int32_t head_hi, float scale, float* lse, void* ws,
                         size_t ws_bytes, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, head_lo, head_hi, scale, in_dt, out_dt, ws, ws_bytes, h};
  if (int st = check_attention(a)) return st;
  if (in_dt == USP_BF16) {
    if (!ws) return fail(USP_EINVAL, "workspace is null");
    if (!aligned16(ws)) return fail(USP_EALIGN, "workspace is not 16-byte aligned");
  } else {
    a.ws = nullptr;  // the fp32 path needs none
  }
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

// ---- usp_attention_fwd_noalloc: the key-half workspace in a static array ----
namespace usp {
namespace {

// Device memory the library reserves on every GPU it runs on, for callers
// that cannot allocate (graph capture, tight serving loops). In host code
// the array's name is a host-side stand-in, not a device address: host code
// only ever uses the per-device address from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = size_t(USP_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The scratch address on the device that runs `stream`, looked up once per
// device with that device current.
int scratch_address(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(USP_EHIP, "hipGetDevice failed");
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess)
    return fail(USP_EHIP, "hipStreamGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(USP_EINVAL, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return fail(USP_EHIP, "hipSetDevice(%d) failed", dev);
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p)
      return fail(USP_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return USP_OK;
}

}  // namespace
}  // namespace usp

int usp_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                              usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S, int32_t h,
                              int32_t D, int32_t head_lo, int32_t head_hi, float scale, float* lse,
                              void* stream) {
  using namespace usp;
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, head_lo, head_hi, scale, in_dt, out_dt, nullptr, 0, h};
  if (int st = check_attention(a)) return st;
  if (in_dt == USP_BF16) {
    const size_t need = attention_bf16_ws_bytes(B, S, head_hi - head_lo, D);
    if (need > kScratchBytes)
      return fail(USP_EINVAL, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                  need, kScratchBytes);
    if (int st = scratch_address((hipStream_t)stream, &a.ws)) return st;
    a.ws_bytes = kScratchBytes;
  }
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_fwd_gqa(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                          usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t h_kv,
                          int32_t D, int32_t head_lo, int32_t head_hi, float scale, float* lse,
                          void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, head_lo, head_hi, scale, in_dt, out_dt, ws, ws_bytes, h_kv};
  if (int st = check_attention(a)) return st;
  if (in_dt != USP_BF16) a.ws = nullptr;
  if (a.ws && !aligned16(a.ws)) return fail(USP_EALIGN, "workspace is not 16-byte aligned");
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_fwd_block(const void* q, const void* k, const void* v, void* o,
                            usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t Sq, int64_t Sk,
                            int32_t h, int32_t h_kv, int32_t D, int32_t head_lo, int32_t head_hi,
                            float scale, float* lse, void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, Sq, Sk, h, D, head_lo, head_hi, scale, in_dt, out_dt, ws, ws_bytes,
             h_kv};
  if (int st = check_attention(a)) return st;
  if (in_dt != USP_BF16) a.ws = nullptr;
  if (a.ws && !aligned16(a.ws)) return fail(USP_EALIGN, "workspace is not 16-byte aligned");
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_fwd_block_whole(const void* q, const void* k, const void* v, void* o,
                                  usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t Sq,
                                  int64_t Sk, int32_t h, int32_t h_kv, int32_t D, int32_t head_lo,
                                  int32_t head_hi, float scale, float* lse, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, Sq, Sk, h, D, head_lo, head_hi, scale, in_dt, out_dt, nullptr, 0,
             h_kv};
  a.whole = true;
  if (int st = check_attention(a)) return st;
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)D);
  if (int st = run_attention(a, (hipStream_t)stream)) return st;
  return ok();
}

int usp_attention_merge(const float* o_a, const float* lse_a, const float* o_b,
                        const float* lse_b, void* o, float* lse, usp_dtype out_dt, int64_t B,
                        int64_t S, int32_t h, int32_t D, int32_t head_lo, int32_t head_hi,
                        void* stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return fail(USP_EINVAL, "null o_a, lse_a, o_b, lse_b or o");
  if (h < 1) return fail(USP_EINVAL, "h must be positive");
  if (head_lo < 0 || head_hi > h || head_lo >= head_hi)
    return fail(USP_EINVAL, "head range [%d, %d) is empty or outside [0, %d)", head_lo, head_hi, h);
  if (B < 1 || S < 1) return fail(USP_ESHAPE, "B and S must be positive");
  if (out_dt != USP_F32 && out_dt != USP_BF16)
    return fail(USP_EDTYPE, "unsupported output dtype %d", (int)out_dt);
  if (D != 32 && D != 64 && D != 128)
    return fail(USP_ENOSYS, "attention merge supports D in {32, 64, 128} (got %d)", D);
  if (out_dt == USP_BF16 && (o == static_cast<const void*>(o_a) || o == static_cast<const void*>(o_b)))
    return fail(USP_EINVAL, "a bf16 output cannot overwrite an fp32 input");
  int64_t n;
  if (!mul_ok(B, S, &n) || !mul_ok(n, h, &n) || !mul_ok(n, D, &n) || !mul_ok(n, 4, &n))
    return fail(USP_ESHAPE, "tensor size overflows");
  if (n / 16 > (int64_t(1) << 31) - 1) return fail(USP_ESHAPE, "tensor too large for one launch");
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o))
    return fail(USP_EALIGN, "o_a, o_b and o must be 16-byte aligned");
  for (const float* p : {lse_a, lse_b, static_cast<const float*>(lse)})
    if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(USP_EALIGN, "lse arrays must be 4-byte aligned");
  MergeArgs a{o_a, lse_a, o_b, lse_b, o, lse, B, S, h, D, head_lo, head_hi, out_dt};
  if (int st = launch_attention_merge(a, (hipStream_t)stream)) return st;
  return ok();
}

// head-chunk passes of a (validated) attention call over all a.h heads; with
// a workspace, the first (largest) chunk's size check covers every pass
static int run_chunked(AttnArgs a, int32_t chunks, hipStream_t stream) {
  const int32_t h = a.h;
  if (chunks < 1 || chunks > h)
    return fail(USP_EINVAL, "cannot run %d heads in %d non-empty chunks", h, chunks);
  int32_t bounds[USP_MAX_PARTS + 1];
  int32_t* hb = bounds;
  std::string heap;  // large chunk counts: bounds on the heap
  if (chunks > USP_MAX_PARTS) {
    heap.resize(sizeof(int32_t) * (chunks + 1));
    hb = reinterpret_cast<int32_t*>(&heap[0]);
  }
  if (int st = usp_head_chunk_ranges(h, chunks, hb)) return st;
  if (!(a.scale > 0.0f)) a.scale = 1.0f / sqrtf((float)a.D);
  for (int32_t c = 0; c < chunks; ++c) {
    a.head_lo = hb[c];
    a.head_hi = hb[c + 1];
    if (int st = run_attention(a, stream)) return st;
  }
  return ok();
}

int usp_attention_fwd_chunked(const void* q, const void* k, const void* v, void* o,
                              usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S,
                              int32_t h, int32_t D, float scale, float* lse, int32_t chunks,
                              void* stream) {
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, 0, h, scale, in_dt, out_dt, nullptr, 0, h};
  if (int st = check_attention(a)) return st;
  return run_chunked(a, chunks, (hipStream_t)stream);
}

int usp_attention_fwd_chunked_ws(const void* q, const void* k, const void* v, void* o,
                                 usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S,
                                 int32_t h, int32_t D, float scale, float* lse, int32_t chunks,
                                 void* ws, size_t ws_bytes, void* stream) {
  AttnArgs a{q, k, v, o, lse, B, S, S, h, D, 0, h, scale, in_dt, out_dt, ws, ws_bytes, h};
  if (int st = check_attention(a)) return st;
  if (in_dt == USP_BF16) {
    if (!ws) return fail(USP_EINVAL, "workspace is null");
    if (!aligned16(ws)) return fail(USP_EALIGN, "workspace is not 16-byte aligned");
  } else {
    a.ws = nullptr;  // the fp32 path needs none
  }
  return run_chunked(a, chunks, (hipStream_t)stream);
}

}  // extern "C"
