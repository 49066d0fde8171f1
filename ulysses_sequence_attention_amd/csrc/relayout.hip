// Sequence-sharded <-> head-sharded relayouts (the local data movement on
// either side of the Ulysses all-to-alls: h3-blackwell-runtime distributed.py,
// SequenceParallelContext.seq_to_heads / heads_to_seq) and the device twin of
// the balanced ranges.
//
// Both directions are a permutation of whole 16-byte chunks: a head's D-vector
// is D*esize bytes, a multiple of 16, so no chunk straddles two heads. The
// kernel walks the sequence-side tensor linearly (fully coalesced 128-bit
// accesses) and computes, for every chunk, where it lives on the head side:
//
//   seq row R = (b, s)      chunk c within the row = (head, dc)
//   head -> group j, index i within the group (closed form of the balanced
//   head ranges), block j row = b * S + t_r + s
//   block offset = ((row_j * h_j) + i) * chunks_per_head + dc
//
// Consecutive chunks of a row go to a few contiguous runs of h_j * D * esize
// bytes (>= 384 B at every supported shape), so the scattered side is also
// written or read in long contiguous runs. All divisions are multiply-high
// by host-computed magic numbers.
#include "usp_internal.h"

namespace usp {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

// per plane: the sequence-side tensor and its P head blocks
struct Ptrs {
  u32x4* seq[USP_MAX_PLANES];
  u32x4* p[USP_MAX_PLANES][USP_MAX_PARTS];
};

struct RelayoutParams {
  uint32_t n_chunks;   // chunks handled by this launch per plane (seq side, < 2^31)
  uint32_t row0;       // first seq row of this launch
  uint32_t cpr;        // chunks per seq row = H * cph
  uint32_t cph;        // chunks per head = D * esize / 16
  uint32_t base, extra, xb;  // head ranges: base = H / P, extra = H % P, xb = extra*(base+1)
  uint32_t len;        // seq rows per batch row on the seq side (S or len_r)
  uint32_t S;          // rows per batch row on the head side
  uint32_t t0;         // first token row of this rank (0 in world mode)
  FastDiv fd_cpr, fd_cph, fd_base, fd_base1, fd_len;
};

constexpr int kThreads = 256;
// one 16-byte chunk per thread: 13-21 VGPRs, so that these waves also fit
// beside the attention kernel's workgroups on a CU (measured faster alone
// too than four chunks per thread at 64 VGPRs)
constexpr int kUnroll = 1;

template <bool kPack>
__global__ __launch_bounds__(kThreads) void relayout_kernel(RelayoutParams p, Ptrs ptr) {
  const uint32_t first = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  const int t = blockIdx.y;  // plane
  u32x4* const seq = ptr.seq[t];
  u32x4 val[kUnroll];
  u32x4* dst[kUnroll];
  const u32x4* src[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t idx = first + u * kThreads;
    dst[u] = nullptr;
    if (idx < p.n_chunks) {
      const uint32_t lrow = p.fd_cpr.div(idx);
      const uint32_t c = idx - lrow * p.cpr;
      const uint32_t row = p.row0 + lrow;
      const uint32_t head = p.fd_cph.div(c);
      const uint32_t dc = c - head * p.cph;
      uint32_t j, i, hj;
      if (head < p.xb) {
        j = p.fd_base1.div(head);
        i = head - j * (p.base + 1);
        hj = p.base + 1;
      } else {
        const uint32_t rest = head - p.xb;
        const uint32_t g = p.fd_base.div(rest);
        j = p.extra + g;
        i = rest - g * p.base;
        hj = p.base;
      }
      const uint32_t b = p.fd_len.div(row);
      const uint32_t s = row - b * p.len;
      const uint64_t hrow = uint64_t(b) * p.S + p.t0 + s;
      const uint64_t hoff = (hrow * hj + i) * p.cph + dc;
      const uint64_t soff = uint64_t(row) * p.cpr + c;
      if (kPack) {
        src[u] = seq + soff;
        dst[u] = ptr.p[t][j] + hoff;
      } else {
        src[u] = ptr.p[t][j] + hoff;
        dst[u] = seq + soff;
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

// One phase of the head-chunked exchange (maxdiffusion PR #428, two-phase
// all-to-all): only heads [lo, lo + hc) of each of the P equal groups of h
// heads move. Per seq row these are P runs of hc * cph chunks, at head
// offset j * h + lo on the seq side and at head lo of row (b, t0 + s) in
// block j; within a run the chunk index r is the same on both sides, so a
// chunk's two addresses are the run bases plus r and no head division is
// needed. Both sides are read and written in runs of hc * D * esize bytes.
struct ChunkParams {
  uint32_t n_chunks;  // chunks moved by this launch per plane (< 2^31)
  uint32_t row0;      // first seq row of this launch
  uint32_t cpr;       // chunks per seq row = H * cph
  uint32_t cph;       // chunks per head
  uint32_t h, lo;     // heads per group; first head of the phase in a group
  uint32_t crow;      // chunks moved per seq row = P * cgrp
  uint32_t cgrp;      // chunks moved per group and row = hc * cph
  uint32_t len, S, t0;
  FastDiv fd_crow, fd_cgrp, fd_len;
};

template <bool kPack>
__global__ __launch_bounds__(kThreads) void relayout_chunk_kernel(ChunkParams p, Ptrs ptr) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= p.n_chunks) return;
  const int t = blockIdx.y;  // plane
  u32x4* const seq = ptr.seq[t];
  const uint32_t lrow = p.fd_crow.div(idx);
  const uint32_t c = idx - lrow * p.crow;
  const uint32_t j = p.fd_cgrp.div(c);
  const uint32_t r = c - j * p.cgrp;
  const uint32_t row = p.row0 + lrow;
  const uint32_t b = p.fd_len.div(row);
  const uint32_t s = row - b * p.len;
  const uint64_t hrow = uint64_t(b) * p.S + p.t0 + s;
  const uint64_t hoff = (hrow * p.h + p.lo) * p.cph + r;
  const uint64_t soff = uint64_t(row) * p.cpr + (uint64_t(j) * p.h + p.lo) * p.cph + r;
  if (kPack)
    __builtin_nontemporal_store(__builtin_nontemporal_load(seq + soff), ptr.p[t][j] + hoff);
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load(ptr.p[t][j] + hoff), seq + soff);
}

__global__ void ranges_kernel(int64_t total, int32_t parts, int64_t* bounds) {
  const int32_t r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r > parts) return;
  const int64_t base = total / parts, extra = total % parts;
  bounds[r] = r * base + (r < extra ? int64_t(r) : extra);
}

}  // namespace

int launch_ranges_device(int64_t total, int32_t parts, int64_t* d_bounds, hipStream_t s) {
  const int threads = 256;
  const int blocks = (parts + 1 + threads - 1) / threads;
  ranges_kernel<<<blocks, threads, 0, s>>>(total, parts, d_bounds);
  return check_launch("ranges_kernel");
}

int launch_relayout(const RelayoutArgs& a, bool pack, hipStream_t s) {
  const uint32_t cph = uint32_t(a.D) * a.esize / 16;
  const uint64_t cpr = uint64_t(a.H) * cph;
  const int64_t base = a.H / a.P, extra = a.H % a.P;
  int64_t len = a.S, t0 = 0;
  if (a.rank >= 0) {
    const int64_t sb = a.S / a.P, se = a.S % a.P;
    t0 = a.rank * sb + (a.rank < se ? a.rank : se);
    len = sb + (a.rank < se ? 1 : 0);
  }
  const uint64_t rows = uint64_t(a.B) * len;
  if (cpr >= (1u << 30) || a.S >= (int64_t(1) << 31) || rows >= (1ull << 31))
    return fail(USP_ESHAPE, "relayout sizes exceed the 32-bit index range of one row walk");

  Ptrs ptr{};
  for (int t = 0; t < a.n; ++t) {
    ptr.seq[t] = const_cast<u32x4*>(static_cast<const u32x4*>(a.seq[t]));
    for (int j = 0; j < a.P; ++j)
      ptr.p[t][j] = const_cast<u32x4*>(static_cast<const u32x4*>(a.blk[size_t(t) * a.P + j]));
  }

  if (a.head_hi > 0) {  // one head-chunk phase (equal groups, checked by the caller)
    ChunkParams p;
    p.cpr = uint32_t(cpr);
    p.cph = cph;
    p.h = uint32_t(a.H / a.P);
    p.lo = uint32_t(a.head_lo);
    p.cgrp = uint32_t(a.head_hi - a.head_lo) * cph;
    p.crow = p.cgrp * uint32_t(a.P);  // <= cpr < 2^30
    p.len = uint32_t(len);
    p.S = uint32_t(a.S);
    p.t0 = uint32_t(t0);
    p.fd_crow = FastDiv(p.crow);
    p.fd_cgrp = FastDiv(p.cgrp);
    p.fd_len = FastDiv(p.len);
    const uint64_t max_rows = ((1ull << 31) - 1) / p.crow;
    for (uint64_t r0 = 0; r0 < rows; r0 += max_rows) {
      const uint64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
      p.row0 = uint32_t(r0);
      p.n_chunks = uint32_t(nr * p.crow);
      const dim3 grid((p.n_chunks + kThreads - 1) / kThreads, a.n);
      if (pack)
        relayout_chunk_kernel<true><<<grid, kThreads, 0, s>>>(p, ptr);
      else
        relayout_chunk_kernel<false><<<grid, kThreads, 0, s>>>(p, ptr);
      if (int st = check_launch(pack ? "head-chunk pack kernel" : "head-chunk unpack kernel"))
        return st;
    }
    return USP_OK;
  }

  RelayoutParams p;
  p.cpr = uint32_t(cpr);
  p.cph = cph;
  p.base = uint32_t(base);
  p.extra = uint32_t(extra);
  p.xb = uint32_t(extra * (base + 1));
  p.len = uint32_t(len);
  p.S = uint32_t(a.S);
  p.t0 = uint32_t(t0);
  p.fd_cpr = FastDiv(p.cpr);
  p.fd_cph = FastDiv(cph);
  p.fd_base = FastDiv(p.base);
  p.fd_base1 = FastDiv(p.base + 1);
  p.fd_len = FastDiv(p.len);

  // Keep every flat chunk index of a launch below 2^31: split the row walk.
  const uint64_t max_rows = ((1ull << 31) - 1) / cpr;
  for (uint64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const uint64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    p.row0 = uint32_t(r0);
    p.n_chunks = uint32_t(nr * cpr);
    const uint32_t per_block = kThreads * kUnroll;
    const dim3 grid((p.n_chunks + per_block - 1) / per_block, a.n);
    if (pack)
      relayout_kernel<true><<<grid, kThreads, 0, s>>>(p, ptr);
    else
      relayout_kernel<false><<<grid, kThreads, 0, s>>>(p, ptr);
    if (int st = check_launch(pack ? "pack kernel" : "unpack kernel")) return st;
  }
  return USP_OK;
}

}  // namespace usp
