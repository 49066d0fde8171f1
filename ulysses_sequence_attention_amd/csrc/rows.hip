// Ragged token-row movements at the model boundary, without padding:
//   scatter  m-star scatter_sequence: rank r's contiguous window
//            [t_r, t_{r+1}) of a sequence-replicated [B][S][W] tensor;
//   gather   m-star gather_sequence / h3-blackwell-runtime all_gather_rows:
//            the rank shards [B][len_r][W] concatenated in rank order;
//   reduce-scatter  h3-blackwell-runtime reduce_scatter_rows: rank r's rows
//            of the sum of P partials of the full sequence, added in rank
//            order.
// Rows split over P ranks by the balanced ranges (the first S mod P ranks
// hold one extra row). W * esize is a multiple of 16, so a row is a whole number of
// 16-byte chunks and no chunk straddles two rows.
//
// Both kernels walk one side linearly in 16-byte chunks (fully coalesced)
// and compute the other side's address per chunk; for a fixed batch row a
// rank's rows are contiguous on both sides, so the other side is read or
// written in long runs too. The reduce-scatter reads the P partials at the
// same offset, sums them in fp32 in rank order and rounds once (RNE for
// bf16 outputs). All divisions are multiply-high by host magic numbers.
#include "usp_internal.h"

namespace usp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Ptrs {
  u32x4* p[USP_MAX_PARTS];
};

struct RowParams {
  uint32_t n_chunks;        // chunks of this launch
  uint32_t row0;            // first walked row of this launch
  uint32_t cpr;             // chunks per row
  uint32_t S;               // rows per batch row of the full tensor
  uint32_t len;             // walked rows per batch row (S, or len_r for one rank)
  uint32_t t0;              // first full-tensor row of the walked range (0 or t_r)
  uint32_t base, extra, xb;  // ranges of S: base = S / P, extra = S % P, xb = extra * (base + 1)
  int32_t rank;             // walked rank, or -1 for every rank
  uint32_t P;
  FastDiv fd_cpr, fd_len, fd_base, fd_base1;
};

constexpr int kThreads = 256;
// one 16-byte chunk per thread: 13-21 VGPRs, so that these waves also fit
// beside the attention kernel's workgroups on a CU (measured faster alone
// too than four chunks per thread at 64 VGPRs)
constexpr int kUnroll = 1;

// full-tensor row s (within a batch row) -> (rank r, index within its shard, shard length)
__device__ __forceinline__ void rank_of(const RowParams& p, uint32_t s, uint32_t& r, uint32_t& i,
                                        uint32_t& len) {
  if (s < p.xb) {
    r = p.fd_base1.div(s);
    i = s - r * (p.base + 1);
    len = p.base + 1;
  } else {
    const uint32_t g = p.fd_base.div(s - p.xb);
    r = p.extra + g;
    i = s - p.xb - g * p.base;
    len = p.base;
  }
}

// Walks the full tensor's rows [t0, t0 + len) of every batch row; kScatter
// copies full -> shards, else shards -> full.
template <bool kScatter>
__global__ __launch_bounds__(kThreads) void row_copy_kernel(RowParams p, u32x4* full, Ptrs shard) {
  const uint32_t first = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  u32x4 val[kUnroll];
  const u32x4* src[kUnroll];
  u32x4* dst[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t idx = first + u * kThreads;
    dst[u] = nullptr;
    if (idx < p.n_chunks) {
      const uint32_t wrow = p.row0 + p.fd_cpr.div(idx);  // walked row: b * len + (s - t0)
      const uint32_t c = idx - (wrow - p.row0) * p.cpr;
      const uint32_t b = p.fd_len.div(wrow);
      const uint32_t s = p.t0 + (wrow - b * p.len);
      uint32_t r, i, lr;
      rank_of(p, s, r, i, lr);
      const uint64_t foff = (uint64_t(b) * p.S + s) * p.cpr + c;
      const uint64_t soff = (uint64_t(b) * lr + i) * p.cpr + c;
      if (kScatter) {
        src[u] = full + foff;
        dst[u] = shard.p[r] + soff;
      } else {
        src[u] = shard.p[r] + soff;
        dst[u] = full + foff;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst[u]) val[u] = __builtin_nontemporal_load(src[u]);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (dst[u]) __builtin_nontemporal_store(val[u], dst[u]);
}

__device__ __forceinline__ void add_chunk(f32x4 (&acc)[2], u32x4 x, bool bf16) {
  if (bf16) {
    // bf16 element e of the chunk is the high half of fp32 (x >> 16 for odd e)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[w >> 1][2 * (w & 1)] += __uint_as_float(x[w] << 16);
      acc[w >> 1][2 * (w & 1) + 1] += __uint_as_float(x[w] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) acc[0][w] += __uint_as_float(x[w]);
  }
}

// bf16 round-to-nearest-even of a finite fp32 value
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// out[r][b][i] = sum_j partial[j][b][t_r + i] over j = 0 .. P - 1 in order,
// for the walked rows.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void reduce_scatter_kernel(RowParams p, Ptrs part, Ptrs out) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= p.n_chunks) return;
  const uint32_t wrow = p.row0 + p.fd_cpr.div(idx);
  const uint32_t c = idx - (wrow - p.row0) * p.cpr;
  const uint32_t b = p.fd_len.div(wrow);
  const uint32_t s = p.t0 + (wrow - b * p.len);
  uint32_t r, i, lr;
  rank_of(p, s, r, i, lr);
  const uint64_t foff = (uint64_t(b) * p.S + s) * p.cpr + c;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // loads of several partials in flight before their adds
  uint32_t j = 0;
  for (; j + 4 <= p.P; j += 4) {
    const u32x4 x0 = __builtin_nontemporal_load(part.p[j] + foff);
    const u32x4 x1 = __builtin_nontemporal_load(part.p[j + 1] + foff);
    const u32x4 x2 = __builtin_nontemporal_load(part.p[j + 2] + foff);
    const u32x4 x3 = __builtin_nontemporal_load(part.p[j + 3] + foff);
    add_chunk(acc, x0, kBf16);
    add_chunk(acc, x1, kBf16);
    add_chunk(acc, x2, kBf16);
    add_chunk(acc, x3, kBf16);
  }
  for (; j < p.P; ++j) add_chunk(acc, __builtin_nontemporal_load(part.p[j] + foff), kBf16);
  u32x4 y;
  if (kBf16) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      y[w] = bf16_rne(acc[w >> 1][2 * (w & 1)]) | (bf16_rne(acc[w >> 1][2 * (w & 1) + 1]) << 16);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) y[w] = __float_as_uint(acc[0][w]);
  }
  __builtin_nontemporal_store(y, out.p[r] + (uint64_t(b) * lr + i) * p.cpr + c);
}

}  // namespace

int launch_rows(const RowArgs& a, RowOp op, hipStream_t s) {
  const uint64_t cpr = uint64_t(a.W) * a.esize / 16;
  const int64_t base = a.S / a.P, extra = a.S % a.P;
  int64_t len = a.S, t0 = 0;
  if (a.rank >= 0) {
    t0 = a.rank * base + (a.rank < extra ? a.rank : extra);
    len = base + (a.rank < extra ? 1 : 0);
  }
  const uint64_t rows = uint64_t(a.B) * len;
  if (cpr >= (1u << 30) || a.S >= (int64_t(1) << 31) || rows >= (1ull << 31))
    return fail(USP_ESHAPE, "row sizes exceed the 32-bit index range of one row walk");

  RowParams p;
  p.cpr = uint32_t(cpr);
  p.S = uint32_t(a.S);
  p.len = uint32_t(len);
  p.t0 = uint32_t(t0);
  p.base = uint32_t(base);
  p.extra = uint32_t(extra);
  p.xb = uint32_t(extra * (base + 1));
  p.rank = a.rank;
  p.P = uint32_t(a.P);
  p.fd_cpr = FastDiv(p.cpr);
  p.fd_len = FastDiv(p.len);
  p.fd_base = FastDiv(p.base);
  p.fd_base1 = FastDiv(p.base + 1);

  // inputs (gather, reduce-scatter) and outputs (scatter, reduce-scatter);
  // each array is present only for the operations that use it
  Ptrs x{}, y{};
  for (int j = 0; j < a.P; ++j) {
    if (a.in) x.p[j] = const_cast<u32x4*>(static_cast<const u32x4*>(a.in[j]));
    if (a.out) y.p[j] = static_cast<u32x4*>(a.out[j]);
  }
  u32x4* full = static_cast<u32x4*>(a.full);

  // Keep every flat chunk index of a launch below 2^31: split the row walk.
  const uint64_t per = op == RowOp::kReduceScatter ? kThreads : uint64_t(kThreads) * kUnroll;
  const uint64_t max_rows = ((1ull << 31) - per) / cpr;
  for (uint64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const uint64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    p.row0 = uint32_t(r0);
    p.n_chunks = uint32_t(nr * cpr);
    const unsigned grid = unsigned((p.n_chunks + per - 1) / per);
    switch (op) {
      case RowOp::kScatter:
        row_copy_kernel<true><<<grid, kThreads, 0, s>>>(p, full, y);
        break;
      case RowOp::kGather:
        row_copy_kernel<false><<<grid, kThreads, 0, s>>>(p, full, x);
        break;
      case RowOp::kReduceScatter:
        if (a.esize == 2)
          reduce_scatter_kernel<true><<<grid, kThreads, 0, s>>>(p, x, y);
        else
          reduce_scatter_kernel<false><<<grid, kThreads, 0, s>>>(p, x, y);
        break;
    }
    if (int st = check_launch("rows kernel")) return st;
  }
  return USP_OK;
}

}  // namespace usp
