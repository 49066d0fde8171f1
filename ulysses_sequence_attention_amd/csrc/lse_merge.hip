// Log-sum-exp merge of two attention results over disjoint key blocks (the
// fold of a ring step in Ulysses+Ring attention, maxdiffusion PR #428
// description: the head-chunked passes also run under Ulysses+Ring).
//
// Softmax over the union of two key sets: with per-block outputs O_a, O_b
// (each normalised over its own keys) and natural-log normalisers lse_a,
// lse_b of a query row,
//   lse = log(e^lse_a + e^lse_b),  O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.
// Evaluated as M = max(lse_a, lse_b), e_x = exp(lse_x - M) (one of them is
// 1), lse = M + log(e_a + e_b), O = f_a O_a + f_b O_b with f_x = e_x / (e_a +
// e_b). A block with lse = -inf (no keys) gets weight 0; if both are -inf
// the row has no keys and O = 0, lse = -inf.
//
// HBM-bound: one thread per 4 head-dim elements of a row (16-byte loads of
// O_a and O_b, one 16- or 8-byte store); the D / 4 threads of a
// (batch, row, head) are consecutive lanes of one wave, so they read lse_a
// and lse_b in one load before the one lane that writes lse stores it. That
// is what lets o and lse be updated in place (o == o_a, lse == lse_a).
#include "usp_internal.h"

namespace usp {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

struct MergeParams {
  const float* o_a;
  const float* lse_a;
  const float* o_b;
  const float* lse_b;
  void* o;
  float* lse;
  uint32_t n;        // threads: B * S * nheads * D / 4
  uint32_t S, h, head_lo, nheads;
  FastDiv fd_nh, fd_S;
};

template <int D, bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(MergeParams p) {
  constexpr uint32_t CH = D / 4;  // threads per (batch, row, head); divides 64
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= p.n) return;
  const uint32_t t = idx / CH, ch = idx % CH;  // t = (b * S + row) * nheads + head_i
  const uint32_t bs = p.fd_nh.div(t);
  const uint32_t head = p.head_lo + (t - bs * p.nheads);
  const uint32_t b = p.fd_S.div(bs), row = bs - b * p.S;
  const size_t li = (size_t(b) * p.h + head) * p.S + row;
  const size_t oi = (size_t(bs) * p.h + head) * D + ch * 4;

  const float la = p.lse_a[li], lb = p.lse_b[li];
  const f32x4 x = *reinterpret_cast<const f32x4*>(p.o_a + oi);
  const f32x4 y = *reinterpret_cast<const f32x4*>(p.o_b + oi);
  const float m = fmaxf(la, lb);
  float fa = 0.0f, fb = 0.0f, lse = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);
    const float den = ea + eb;
    const float inv = 1.0f / den;
    fa = ea * inv;
    fb = eb * inv;
    lse = m + logf(den);
  }
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = fmaf(fa, x[e], fb * y[e]);
  if (kBf16)
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + oi) = __builtin_convertvector(r, bf16x4);
  else
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + oi) = r;
  if (p.lse && ch == 0) p.lse[li] = lse;
}

template <int D>
int launch_d(const MergeParams& p, bool bf16, hipStream_t s) {
  const unsigned grid = unsigned((uint64_t(p.n) + kThreads - 1) / kThreads);
  if (bf16)
    lse_merge_kernel<D, true><<<grid, kThreads, 0, s>>>(p);
  else
    lse_merge_kernel<D, false><<<grid, kThreads, 0, s>>>(p);
  return check_launch("lse_merge_kernel");
}

}  // namespace

int launch_attention_merge(const MergeArgs& a, hipStream_t s) {
  const int32_t nheads = a.head_hi - a.head_lo;
  const uint64_t n = uint64_t(a.B) * a.S * nheads * (a.D / 4);
  if (n >= (1ull << 31) || uint64_t(a.B) * a.S >= (1ull << 31))
    return fail(USP_ESHAPE, "merge of %llu elements exceeds one launch",
                (unsigned long long)(n * 4));
  MergeParams p;
  p.o_a = a.o_a;
  p.lse_a = a.lse_a;
  p.o_b = a.o_b;
  p.lse_b = a.lse_b;
  p.o = a.o;
  p.lse = a.lse;
  p.n = uint32_t(n);
  p.S = uint32_t(a.S);
  p.h = uint32_t(a.h);
  p.head_lo = uint32_t(a.head_lo);
  p.nheads = uint32_t(nheads);
  p.fd_nh = FastDiv(p.nheads);
  p.fd_S = FastDiv(p.S);
  const bool bf16 = a.out_dt == USP_BF16;
  switch (a.D) {
    case 32:
      return launch_d<32>(p, bf16, s);
    case 64:
      return launch_d<64>(p, bf16, s);
    case 128:
      return launch_d<128>(p, bf16, s);
    default:
      return fail(USP_ENOSYS, "attention merge: unsupported D %d", a.D);
  }
}

}  // namespace usp
