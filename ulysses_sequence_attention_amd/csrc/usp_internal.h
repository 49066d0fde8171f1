// Internal helpers of libusp (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "usp.h"  // include/ is on the include path

namespace usp {

// Record a status and message for usp_last_error(); returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's message and return USP_OK.
int ok();
// Translate the last HIP launch status into USP_EHIP (or USP_OK).
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Unsigned division by a run-time invariant d >= 1 for dividends n < 2^31,
// as a multiply-high and a shift (Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, round-up variant):
// shift = ceil(log2 d), mul = floor(2^32 (2^shift - d) / d) + 1,
// n / d = (mulhi(n, mul) + n) >> shift.
struct FastDiv {
  uint32_t d, mul, shift;
  FastDiv() : d(1), mul(1), shift(0) {}
  explicit FastDiv(uint32_t divisor) : d(divisor) {
    shift = 0;
    while ((1ull << shift) < divisor) ++shift;
    mul = (uint32_t)(((1ull << 32) * ((1ull << shift) - divisor)) / divisor + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, mul) + n) >> shift;
  }
};

// Kernel launchers (one per translation unit).
int launch_ranges_device(int64_t total, int32_t parts, int64_t* d_bounds, hipStream_t s);

struct RelayoutArgs {
  // n planes (tensors of one shape, e.g. q, k, v) moved by one launch
  int32_t n;
  const void* const* seq;   // n sequence-side tensors (pack: sources; unpack: destinations)
  const void* const* blk;   // n * P head blocks, plane-major: blk[t * P + j]
  int64_t B, S;
  int32_t H, D, P, rank, esize;
  // one phase of the head-chunked exchange: heads [head_lo, head_hi) of each
  // of the P equal groups (head_hi = 0: whole groups, ragged allowed)
  int32_t head_lo, head_hi;
};
int launch_relayout(const RelayoutArgs& a, bool pack, hipStream_t s);

// Ragged token rows of [B][S][W] tensors over P balanced ranges.
enum class RowOp { kScatter, kGather, kReduceScatter };
struct RowArgs {
  void* full;                 // scatter: source; gather: destination; else unused
  const void* const* in;      // gather: P shards; reduce-scatter: P partials
  void* const* out;           // scatter: P shards; reduce-scatter: P outputs
  int64_t B, S, W;
  int32_t P, rank, esize;     // rank < 0: every rank's rows
};
int launch_rows(const RowArgs& a, RowOp op, hipStream_t s);

struct AttnArgs {
  const void *q, *k, *v;
  void* o;
  float* lse;
  int64_t B, S;      // S: query rows (q, o, lse) per batch row
  int64_t Sk;        // keys (k, v) per batch row
  int32_t h, D, head_lo, head_hi;
  float scale;
  usp_dtype in_dt, out_dt;
  void* ws;         // bf16 path: key-half workspace, or nullptr for the key-group kernel
  size_t ws_bytes;
  int32_t h_kv;     // heads of k and v (h for plain multi-head attention); divides h
  bool whole = false;  // bf16 path: walk every row's keys in one pass (never split them)
};
int launch_attention_f32(const AttnArgs& a, hipStream_t s);
// Log-sum-exp merge of two attention results (fp32 o and lse) for heads
// [head_lo, head_hi) of [B][S][h][D] tensors.
struct MergeArgs {
  const float *o_a, *lse_a, *o_b, *lse_b;
  void* o;
  float* lse;       // may be nullptr
  int64_t B, S;
  int32_t h, D, head_lo, head_hi;
  usp_dtype out_dt;
};
int launch_attention_merge(const MergeArgs& a, hipStream_t s);
int launch_attention_bf16(const AttnArgs& a, hipStream_t s);
// Workspace bytes the bf16 key-half path needs for B x heads x S rows.
size_t attention_bf16_ws_bytes(int64_t B, int64_t S, int32_t heads, int32_t D);
// Whether bf16 attention over Sk keys at head dim D splits each row's keys in
// halves (the form that takes a workspace, or the key-group kernel without).
bool attention_bf16_splits(int64_t Sk, int32_t D);

}  // namespace usp
