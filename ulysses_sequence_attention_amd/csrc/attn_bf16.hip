// Flash-style non-causal attention for bf16 Q/K/V on CDNA4 matrix cores
// (gfx950 v_mfma_f32_32x32x16_bf16), fp32 scores, softmax and accumulation.
//
// What it computes (m-star ulysses_attention: the unchanged attention kernel
// run on the full sequence of the rank's head group): per head n,
//   O[s] = sum_t softmax_t(scale * <Q[s], K[t]>) V[t].
//
// Work decomposition. A workgroup of 4 waves owns BM = 4 * 64 query rows of
// one (batch, head); each wave owns 64 rows as two 32-row MFMA blocks. The
// keys are walked in tiles of BN rows (64 for D = 128, 128 for D = 64), each
// tile staged in LDS (K row-major, V transposed), double buffered: the next
// tile's global loads are issued before the current tile's math and written
// to the other LDS buffer after it, with one barrier per tile.
//
// Layout trick. The score block is computed transposed, S^T = K Q^T (A = K,
// B = Q^T), so a lane of the 32x32 accumulator holds 16 keys of ONE query
// (the other 16 keys of that 32-key block sit in lane ^ 32): the row maximum
// is an in-lane reduction plus one cross-half exchange. The A operand's row
// rho is fed with K row pi(rho), where for rho = 8a + 4g + c (a < 4, g < 2,
// c < 4) pi(rho) = 16(a / 2) + 8g + 4(a % 2) + c. With it, accumulator
// register r (< 16) of a lane in half g holds key 16(r / 8) + 8g + (r % 8):
// registers 0..7 and 8..15 are each 8 consecutive keys, which is exactly the
// B operand layout of the second product O^T = V^T P^T (A = V^T). So P^T
// goes from accumulators to bf16 operands without any lane exchange, and
// V^T fragments are single 16-byte LDS reads of 8 consecutive keys.
//
// Online softmax (base 2: weights are exp2(c * s - c * m), c = scale *
// log2(e)) with lazy rescaling: the reference maximum m of a row is only
// moved when a tile's maximum exceeds it by more than a factor 2 in weight,
// so flat rows almost never rescale their O accumulators, while a row whose
// maximum jumps (a dominant key arriving) rescales and gives that key the
// weight exp2(0) = 1, exact in bf16. Weights are rounded to bf16 once for the
// P V product, and the row sum is taken over those same rounded weights
// (v_dot2c_f32_bf16 against (1, 1)), so the rounding of a dominant weight
// cancels between numerator and denominator. Every decision depends on one
// (batch, head, query) row only, so a head's result does not depend on which
// other heads share the launch.
//
// Block -> tile order is XCD aware: the hardware deals workgroup ids round
// robin over the 8 XCDs, so ids are remapped to give each XCD a contiguous
// range of (batch, head, query tile) work, keeping one head's K/V stream in
// one XCD's L2.
#include "usp_internal.h"

namespace usp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 1.0f;  // lazy-rescale threshold, log2 units

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int S, h, head_lo, nheads, n_qtiles;
  float c;      // scale * log2(e)
  float scale;  // softmax scale (for the natural-log normaliser)
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint32_t half16(const uint4& u, int j) {
  const uint32_t w = (j >> 1) == 0 ? u.x : (j >> 1) == 1 ? u.y : (j >> 1) == 2 ? u.z : u.w;
  return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int D, int QB, int BN, bool kOutBf16>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(Params p) {
  constexpr int BM = kWaves * QB * 32;
  constexpr int NKB = BN / 32;           // 32-key blocks per tile
  constexpr int KS = D / 16;             // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;            // 32-wide blocks of the output head dim
  constexpr int KLD = D + 8;             // K tile row stride (elements)
  constexpr int VLD = BN + 8;            // V^T tile row stride (elements)
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int NKL = BN * CPR / kThreads;        // K chunks per thread per tile
  constexpr int NVP = (BN / 4) * CPR / kThreads;  // V (4-key x chunk) groups per thread
  static_assert(NKL * kThreads == BN * CPR, "K tile must split evenly over the block");
  static_assert(NVP * kThreads == (BN / 4) * CPR, "V tile must split evenly over the block");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][D * VLD];

  // ---- XCD-aware workgroup -> (batch, head, query tile) -------------------
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = bid & 7;
  const int lid = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (bid >> 3);
  const int qt = lid % p.n_qtiles;
  const int bh = lid / p.n_qtiles;
  const int head = p.head_lo + bh % p.nheads;
  const int b = bh / p.nheads;

  const int S = p.S;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const size_t rs = size_t(p.h) * D;                             // token row stride
  const size_t hb = size_t(b) * S * rs + size_t(head) * D;       // (b, token 0, head)
  const int qrow0 = qt * BM + w * (QB * 32);

  // ---- Q^T fragments (B operand), resident for the whole key walk --------
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < S) x = *reinterpret_cast<const uint4*>(p.q + hb + size_t(row) * rs + s * 16 + g * 8);
      qf[qb][s] = as_bf16x8(x);
    }
  }

  // ---- K/V tile staging ---------------------------------------------------
  uint4 kreg[NKL];
  uint4 vreg[NVP][4];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / CPR, ch = idx % CPR;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (t0 + r < S)
        kreg[i] = *reinterpret_cast<const uint4*>(p.k + hb + size_t(t0 + r) * rs + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + i * kThreads;
      const int kq = idx % (BN / 4), ch = idx / (BN / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = t0 + 4 * kq + e;
        vreg[i][e] = make_uint4(0, 0, 0, 0);
        if (key < S)
          vreg[i][e] = *reinterpret_cast<const uint4*>(p.v + hb + size_t(key) * rs + ch * 8);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(&ks[buf][r * KLD + ch * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i) {
      const int idx = tid + i * kThreads;
      const int kq = idx % (BN / 4), ch = idx / (BN / 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint2 x;
        x.x = half16(vreg[i][0], j) | (half16(vreg[i][1], j) << 16);
        x.y = half16(vreg[i][2], j) | (half16(vreg[i][3], j) << 16);
        *reinterpret_cast<uint2*>(&vt[buf][(ch * 8 + j) * VLD + 4 * kq]) = x;
      }
    }
  };

  // K row fed to A-operand row l32 (see the layout note above)
  const int a4 = l32 >> 3, g4 = (l32 >> 2) & 1, c4 = l32 & 3;
  const int pi = 16 * (a4 >> 1) + 8 * g4 + 4 * (a4 & 1) + c4;

  f32x16 oacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float mrow[QB], lrow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrow[qb] = -INFINITY;
    lrow[qb] = 0.f;
  }

  const int nkt = (S + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const bool has_next = kt + 1 < nkt;
    if (has_next) load_tile((kt + 1) * BN);

    // ---- S^T = K Q^T ------------------------------------------------------
    f32x16 sacc[NKB][QB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][qb][r] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf =
            as_bf16x8(*reinterpret_cast<const uint4*>(&ks[buf][(kb * 32 + pi) * KLD + s * 16 + g * 8]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][s], sacc[kb][qb], 0, 0, 0);
      }
    }

    // ---- mask keys past the end (last tile only) ---------------------------
    if ((kt + 1) * BN > S) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * BN + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
          if (key >= S) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb][r] = -INFINITY;
          }
        }
    }

    // ---- online softmax ------------------------------------------------------
    float mnew[QB];
    bool need[QB];
    bool any_need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mnew[qb] = fmaxf(mrow[qb], mx);
      need[qb] = (mnew[qb] - mrow[qb]) * p.c > kTau;
      any_need |= need[qb];
    }
    if (__any(any_need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mu = need[qb] ? mnew[qb] : mrow[qb];
        const float alpha = __builtin_amdgcn_exp2f((mrow[qb] - mu) * p.c);
        lrow[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
        mrow[qb] = mu;
      }
    }
    bf16x8 pf[QB][NKB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = mrow[qb] * p.c;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 pv;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][8 * h2 + j], p.c, -mc));
          const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
          pf[qb][kb][h2] = pb;
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one, ls, false);
        }
      }
      lrow[qb] += ls;
    }

    // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4*>(
              &vt[buf][(db * 32 + l32) * VLD + kb * 32 + h2 * 16 + g * 8]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][h2], oacc[qb][db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store ------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lrow[qb] + __shfl_xor(lrow[qb], 32);
    const float inv = 1.0f / lt;
    const int row = qrow0 + qb * 32 + l32;
    if (row < S) {
      const size_t ob = hb + size_t(row) * rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = db * 32 + 8 * a + 4 * g;
          f32x4 x;
          x[0] = oacc[qb][db][4 * a + 0] * inv;
          x[1] = oacc[qb][db][4 * a + 1] * inv;
          x[2] = oacc[qb][db][4 * a + 2] * inv;
          x[3] = oacc[qb][db][4 * a + 3] * inv;
          if (kOutBf16) {
            const bf16x4 y = __builtin_convertvector(x, bf16x4);
            *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + ob + d) = y;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + ob + d) = x;
          }
        }
      }
      if (p.lse && g == 0)
        p.lse[(size_t(b) * p.h + head) * S + row] = mrow[qb] * p.scale + logf(lt);
    }
  }
}

template <int D, int QB, int BN>
int launch(const AttnArgs& a, hipStream_t s) {
  constexpr int BM = kWaves * QB * 32;
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.S = int(a.S);
  p.h = a.h;
  p.head_lo = a.head_lo;
  p.nheads = a.head_hi - a.head_lo;
  p.n_qtiles = int((a.S + BM - 1) / BM);
  p.c = a.scale * 1.4426950408889634f;
  p.scale = a.scale;
  const int64_t grid = int64_t(p.n_qtiles) * p.nheads * a.B;
  if (grid > 0x7fffffff) return fail(USP_ESHAPE, "attention grid too large");
  if (a.out_dt == USP_BF16)
    attn_bf16_kernel<D, QB, BN, true><<<unsigned(grid), kThreads, 0, s>>>(p);
  else
    attn_bf16_kernel<D, QB, BN, false><<<unsigned(grid), kThreads, 0, s>>>(p);
  return check_launch("attn_bf16_kernel");
}

}  // namespace

int launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  switch (a.D) {
    case 128:
      return launch<128, 2, 64>(a, s);
    case 64:
      return launch<64, 2, 128>(a, s);
    default:
      return fail(USP_ENOSYS, "bf16 attention: unsupported D %d", a.D);
  }
}

}  // namespace usp
