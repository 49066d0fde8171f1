// Plain fp32 non-causal attention (the fp32 path of usp_attention_fwd).
//
// What it computes: per head n, O[s] = sum_t softmax_t(scale * <Q[s], K[t]>) V[t]
// (m-star ulysses_attention: each rank runs the unchanged attention kernel on
// the full sequence of its head group). One thread owns one query row; a
// wave walks the keys in tiles staged through LDS and keeps an online softmax
// (running maximum and sum, rescaled per tile) in fp32. Scores are kept in the
// base-2 domain (Q is pre-multiplied by scale * log2(e)) so each weight is a
// single exp2. With grouped K/V heads (h_kv < h, m-star ulysses_attention)
// query head n reads K/V head n / (h / h_kv). The query rows (Sq) and the
// keys (Sk) may be different sequence blocks.
#include "usp_internal.h"

namespace usp {

namespace {

constexpr int kRows = 64;  // queries per block (one wave)
constexpr int kKeys = 16;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int S, int Sk, int h, int h_kv, int head_lo,
    int nheads, int n_qtiles, float c_log2, float scale) {
  __shared__ float4 ks[kKeys][D / 4];
  __shared__ float4 vs[kKeys][D / 4];

  int bid = blockIdx.x;
  const int qt = bid % n_qtiles;
  bid /= n_qtiles;
  const int head = head_lo + bid % nheads;
  const int b = bid / nheads;
  const int row = qt * kRows + threadIdx.x;
  const bool live = row < S;
  const size_t rs = size_t(h) * D;  // q / o row stride in elements
  const size_t base = size_t(b) * S * rs + size_t(head) * D;
  const size_t rsk = size_t(h_kv) * D;  // k / v row stride
  const size_t basek = size_t(b) * Sk * rsk + size_t(head / (h / h_kv)) * D;

  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    float4 x = live ? *reinterpret_cast<const float4*>(q + base + row * rs + d)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    qr[d] = x.x * c_log2;
    qr[d + 1] = x.y * c_log2;
    qr[d + 2] = x.z * c_log2;
    qr[d + 3] = x.w * c_log2;
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < Sk; t0 += kKeys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeys * (D / 4); e += kRows) {
      const int t = e / (D / 4), dc = e % (D / 4);
      const bool in = t0 + t < Sk;
      const size_t off = basek + size_t(t0 + t) * rsk + dc * 4;
      ks[t][dc] = in ? *reinterpret_cast<const float4*>(k + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      vs[t][dc] = in ? *reinterpret_cast<const float4*>(v + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    const int nk = Sk - t0 < kKeys ? Sk - t0 : kKeys;
    float sc[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < kKeys; ++t) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D / 4; ++d) {
        const float4 kk = ks[t][d];
        dot = fmaf(qr[4 * d], kk.x, dot);
        dot = fmaf(qr[4 * d + 1], kk.y, dot);
        dot = fmaf(qr[4 * d + 2], kk.z, dot);
        dot = fmaf(qr[4 * d + 3], kk.w, dot);
      }
      sc[t] = t < nk ? dot : -INFINITY;
      mt = fmaxf(mt, sc[t]);
    }
    const float mn = fmaxf(m, mt);
    const float alpha = exp2f(m - mn);  // 0 on the first tile (m = -inf)
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int t = 0; t < kKeys; ++t) {
      const float p = exp2f(sc[t] - mn);
      l += p;
#pragma unroll
      for (int d = 0; d < D / 4; ++d) {
        const float4 vv = vs[t][d];
        acc[4 * d] = fmaf(p, vv.x, acc[4 * d]);
        acc[4 * d + 1] = fmaf(p, vv.y, acc[4 * d + 1]);
        acc[4 * d + 2] = fmaf(p, vv.z, acc[4 * d + 2]);
        acc[4 * d + 3] = fmaf(p, vv.w, acc[4 * d + 3]);
      }
    }
    m = mn;
  }
  if (!live) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *reinterpret_cast<float4*>(o + base + row * rs + d) =
        make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
  if (lse) {
    // m is log2-domain: log(sum exp(scale * dot)) = m * ln 2 + log(l)
    lse[(size_t(b) * h + head) * S + row] = m * 0.69314718055994531f + logf(l);
  }
  (void)scale;
}

}  // namespace

int launch_attention_f32(const AttnArgs& a, hipStream_t s) {
  const int S = int(a.S), nheads = a.head_hi - a.head_lo;
  const int n_qtiles = (S + kRows - 1) / kRows;
  const int64_t grid = int64_t(n_qtiles) * nheads * a.B;
  if (grid > 0x7fffffff) return fail(USP_ESHAPE, "attention grid too large");
  const float c = a.scale * 1.4426950408889634f;
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* v = static_cast<const float*>(a.v);
  float* o = static_cast<float*>(a.o);
  switch (a.D) {
    case 32:
      attn_f32_kernel<32><<<unsigned(grid), kRows, 0, s>>>(q, k, v, o, a.lse, S, int(a.Sk), a.h, a.h_kv, a.head_lo,
                                                          nheads, n_qtiles, c, a.scale);
      break;
    case 64:
      attn_f32_kernel<64><<<unsigned(grid), kRows, 0, s>>>(q, k, v, o, a.lse, S, int(a.Sk), a.h, a.h_kv, a.head_lo,
                                                          nheads, n_qtiles, c, a.scale);
      break;
    case 128:
      attn_f32_kernel<128><<<unsigned(grid), kRows, 0, s>>>(q, k, v, o, a.lse, S, int(a.Sk), a.h, a.h_kv,
                                                           a.head_lo, nheads, n_qtiles, c,
                                                           a.scale);
      break;
    default:
      return fail(USP_ENOSYS, "fp32 attention: unsupported D %d", a.D);
  }
  return check_launch("attn_f32_kernel");
}

}  // namespace usp
