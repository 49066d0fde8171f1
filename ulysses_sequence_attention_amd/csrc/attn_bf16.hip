// Flash-style non-causal attention for bf16 Q/K/V on CDNA4 matrix cores
// (gfx950 v_mfma_f32_32x32x16_bf16), fp32 scores, softmax and accumulation.
//
// What it computes (m-star ulysses_attention: the unchanged attention kernel
// run on the full sequence of the rank's head group): per head n,
//   O[s] = sum_t softmax_t(scale * <Q[s], K[t]>) V[t],
// with K and V of head n / grp when grp query heads share each K/V head.
// The Sq query rows and the Sk keys may be different sequence blocks (a
// ring step of Ulysses+Ring attends a query block to another rank's keys).
//
// Work decomposition. A workgroup of NW waves owns BM = NW * QB * 32 query
// rows of one (batch, head); each wave owns QB blocks of 32 rows (one MFMA
// column block each). Keys are walked in tiles of BN rows staged in LDS,
// both row-major. With 8 waves of 32 rows, two waves share each SIMD.
//
// Software pipeline. K is staged one tile ahead of V: while iteration j
// turns the scores of tile j into weights (exp2, VALU), the same basic block
// computes the scores of tile j + 1 (MFMA), so the matrix pipe and the VALU
// work at once inside one wave; then the weights of tile j multiply V_j.
// LDS holds two K tiles and two V tiles; iteration j issues the direct
// global-to-LDS loads of K_{j+2} and V_{j+1} at its top and ends with one
// barrier. The last (possibly partial) tile is peeled off the loop so the
// steady-state body carries no key mask.
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
// goes from accumulators to bf16 operands without any lane exchange; the
// V^T fragments (8 consecutive keys of one head-dim column) come from the
// row-major V tile through two transposing LDS reads.
//
// Online softmax (base 2: weights are exp2(c * s - c * m), c = scale *
// log2(e)) with lazy rescaling: the reference maximum m of a row is only
// moved when a tile's maximum exceeds it by more than a factor 2 in weight,
// so flat rows almost never rescale their O accumulators, while a row whose
// maximum jumps (a dominant key arriving) rescales and gives that key the
// weight exp2(0) = 1, exact in bf16. Weights are rounded to bf16 once for the
// P V product, and the row sum is taken over those same rounded weights
// (v_dot2c_f32_bf16 against (1, 1)), so the rounding of a dominant weight
// cancels between numerator and denominator.
//
// Key halves. For walks of 8 to 1024 key tiles (nkt = ceil(Sk / BN)) every
// row's key range is split once, at key tile floor(nkt / 2), into two walks
// whose softmax states (reference maximum m, row sum l, unnormalised O) are
// merged at the end with weights 2^(c (m_i - M)), M the larger maximum.
// Whether and where a walk splits depends on Sk and D only, so a row's bits
// never depend on the launch (its head range, batch, the query block it sits
// in or the device). Splitting gives 2x as many work units, which keeps the
// last round of a launch from running half empty (a workgroup fills a CU,
// and at S = 32760, 128 tiles of 256 rows per head, a head is exactly one
// round of 256 half-walks); an even split, since the longer half sets every
// CU's finish time. Shorter and longer walks run whole (at D = 64 a short
// walk runs in 4-wave workgroups of 128 rows with 64-key tiles, three per
// CU). Callers that run several launches at once (the key blocks of a ring
// step on separate streams) may ask for whole walks at every length: the
// launches then fill each other's last rounds and no state is merged. Two
// forms of the split:
//   * key groups (usp_attention_fwd): a workgroup of 8 waves is two groups
//     of 4 waves that walk the two halves for the same 128 rows, each with
//     its own K/V buffers, and merge through LDS;
//   * key-half parts (usp_attention_fwd_ws): 8-wave workgroups of 256 rows
//     walk one half each and leave their state in a caller workspace, and
//     attn_merge_halves merges them with the same arithmetic. Half as much
//     K/V staging per row; same bits.
//
// Block -> tile order is XCD aware: the hardware deals workgroup ids round
// robin over the 8 XCDs, so ids are remapped to give each XCD a contiguous
// range of (batch, head, query tile) work, keeping one head's K/V stream in
// one XCD's L2.
#include <type_traits>

#include "usp_internal.h"

namespace usp {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Keys per K/V tile, per head dim.
#ifndef USP_D128_BN
#define USP_D128_BN 64
#endif
#ifndef USP_D64_BN
#define USP_D64_BN 128
#endif

constexpr float kTau = 1.0f;  // lazy-rescale threshold, log2 units
constexpr int kTileRows = 256;  // query rows of a tile (an 8-wave workgroup)

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int Sq, Sk;  // query rows (q, o, lse) and keys (k, v) per batch row
  int h, head_lo, nheads, n_qtiles;
  int h_kv, grp;  // heads of k and v; query heads per K/V head (h = grp * h_kv)
  float c;      // scale * log2(e)
  float scale;  // softmax scale (for the natural-log normaliser)
  // key-half walks (PARTS = 2): unit (part, tile) = part * n_tiles + tile
  // leaves its unnormalised O rows in ws_o [unit][256][D], reference maxima
  // in ws_m [unit][256] and the two lane-half row sums in ws_l [unit][256][2]
  int n_tiles;
  float* ws_o;
  float* ws_m;
  float* ws_l;
};

// workgroup id (< n) -> logical work id, giving each of the 8 XCDs (which
// are dealt ids round robin) a contiguous range of logical ids
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = n >> 3, rem = n & 7, xcd = id & 7;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + (id >> 3);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// max / sum of a value with the same value in lane ^ 32 (v_permlane32_swap:
// with both operands x it returns (x of lanes 0-31, x of lanes 32-63) in
// both halves)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS
// (buffer_load_dwordx4 ... lds): lane i reads resource base + soff + voff
// (soff a wave-uniform byte offset in a scalar register, voff the lane's
// 32-bit byte offset; raw buffer, stride 0, no range clamp in practice since
// offsets stay inside the tensor) and its bytes land at lds_addr + 16 i,
// lds_addr uniform over the wave (M0). Per-lane addressing is a fixed 32-bit
// offset and the resource is built once, so a load costs no per-lane and
// almost no scalar address arithmetic.
//
// Written as inline assembly on purpose: issued through the compiler's
// builtin, the load counts as an LDS write of unknown address, and the
// compiler then makes the next LDS read of any buffer wait for every such
// load to land (s_waitcnt vmcnt(0) in front of the step's first fragment
// read), which serialises each tile load with the step that issues it
// (measured: 4-5% of the kernel's time). The kernel waits for its own loads
// (loads_done) before the barrier that publishes them. The instruction has
// no register result. The host pass sees an empty body.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource at `addr` (bytes, wave-uniform) covering 2^31 - 1 bytes.
__device__ __forceinline__ i32x4 buffer_rsrc(uint64_t addr) {
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(addr)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(addr >> 32) & 0xffffu));
  r[2] = 0x7fffffff;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + soff + voff (soff wave-uniform) straight into
// LDS at lds_addr + 16 lane (lds_addr wave-uniform, an LDS byte address).
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t soff, uint32_t voff,
                                           uint32_t lds_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int m0 = __builtin_amdgcn_readfirstlane(int(lds_addr));
  const int so = __builtin_amdgcn_readfirstlane(int(soff));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(so)
               : "memory", "m0");
#endif
}

// KG key groups of NW / KG waves share a workgroup; PARTS = 2 makes each
// workgroup walk one key half and leave its state in the workspace. NW = 4
// (short walks at D = 64: 128-row workgroups, 64-key tiles) asks for three
// workgroups per CU, i.e. at most 168 VGPRs per lane.
template <int D, int NW, int KG, int PARTS, int BN, bool kOutBf16>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 3 : 1) void attn_bf16_kernel(Params p) {
  constexpr int QB = 1;                         // 32-row query blocks per wave
  constexpr int GW = NW / KG;                   // waves per key group
  static_assert(GW * KG == NW && KG <= 2, "one or two key groups of equal size");
  static_assert(PARTS == 1 || (PARTS == 2 && KG == 1), "key halves in groups or in parts");
  constexpr int BM = GW * QB * 32;              // query rows of the workgroup
  constexpr int SUB = kTileRows / BM;           // workgroups per tile
  static_assert(SUB * BM == kTileRows, "a tile must split evenly into workgroups");
  constexpr int NKB = BN / 32;           // 32-key blocks per tile
  constexpr int KS = D / 16;             // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;            // 32-wide blocks of the output head dim
  constexpr int ROWB = 2 * D;            // bytes per K/V row
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int RPL = 256 / ROWB;        // rows per 256-byte line of the 64 LDS banks
  constexpr int RPI = 1024 / ROWB;       // rows per direct load (64 lanes x 16 bytes)
  constexpr int NQ = BN * ROWB / 1024;   // direct loads per tile
  constexpr int NI = NQ / GW;            // direct loads per wave per tile (K and V each)
  static_assert(NI * GW == NQ, "a tile must split evenly into the group's direct loads");
  constexpr int TB = BN * ROWB;          // bytes per K or V tile

  // LDS: per key group K tiles in buffers 0, 1, then V tiles in buffers 0,
  // 1; rows unpadded. After the key walk the space holds the second group's
  // partial results for the merge.
  constexpr int MERGE_B = GW * 64 * (NDB * 16 + 2) * 4;
  static_assert(KG == 1 || MERGE_B <= KG * 4 * TB, "merge area must fit the tile buffers");
  __shared__ __attribute__((aligned(16))) char lds[KG * 4 * TB];

  // ---- XCD-aware workgroup -> (batch, head, query tile, sub-tile[, part])
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  // key halves: part-major ids, so that the workgroups an XCD runs at once
  // walk the same key half of one head (one K/V stream per L2; with the two
  // halves of a tile side by side the K/V bytes fetched per call rose from
  // 420 to 713 MB)
  const int part = PARTS == 2 ? u / p.n_tiles : 0;
  const int lid = PARTS == 2 ? u % p.n_tiles : u / SUB, sub = PARTS == 2 ? 0 : u % SUB;
  const int qt = lid % p.n_qtiles;
  const int bh = lid / p.n_qtiles;
  const int head = p.head_lo + bh % p.nheads;
  const int b = bh / p.nheads;

  const int Sq = p.Sq, Sk = p.Sk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int grp = wid / GW, w = wid % GW;                    // key group, wave within it
  const int l32 = lane & 31, g = lane >> 5;
  char* const glds = lds + grp * 4 * TB;  // this group's tile buffers
  const size_t rs = size_t(p.h) * D;                             // q / o token row stride
  const size_t hb = size_t(b) * Sq * rs + size_t(head) * D;       // (b, token 0, head)
  // K/V: query head n reads K/V head n / grp (grouped K/V heads)
  const size_t rsk = size_t(p.h_kv) * D;
  const size_t hbk = size_t(b) * Sk * rsk + size_t(head / p.grp) * D;
  const int qrow0 = qt * kTileRows + sub * BM + w * (QB * 32);
  const float c = p.c;

  // ---- Q^T fragments (B operand), resident for the whole key walk --------
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (row < Sq) x = *reinterpret_cast<const uint4*>(p.q + hb + size_t(row) * rs + s * 16 + g * 8);
      qf[qb][s] = as_bf16x8(x);
    }
  }

  // ---- K/V tile staging (global -> LDS directly) ---------------------------
  // A direct load (buffer_load_dwordx4 ... lds) writes lane i's 16 bytes to
  // LDS base + 16 i, so one load fills RPI whole rows and rows cannot be
  // padded. Instead the 16-byte chunks of a row are stored at XOR-swizzled
  // positions (lane i fetches the chunk whose swizzled position is i mod CPR):
  //   K: chunk c of row r at position c ^ ((r / RPL) mod CPR), so the 16 rows
  //      of a fragment read fall on 16 distinct bank quads;
  //   V: chunk c of row r at position c ^ 4((r / RPL) mod (CPR / 4)), so the
  //      4 rows x 4 chunks of a transposed read are distinct bank quads.
  // Wave w of a group issues loads q = w + GW i of each of the group's tiles
  // (rows [q RPI, q RPI + RPI)).
  auto swz_k = [](int r) { return (r / RPL) % CPR; };
  auto swz_v = [](int r) { return 4 * ((r / RPL) % (CPR / 4)); };
  // Load i of wave w covers rows (w + GW i) RPI .. + RPI. Both swizzles
  // repeat every 16 rows (K: RPL * CPR, V: RPL * CPR / 4 divides it) and
  // GW * RPI is a multiple of 16, so a lane's swizzled chunk is the same in
  // every load: one per-lane offset serves all of them, and load i adds the
  // wave-uniform GW * RPI * i rows to the tile's base address.
  static_assert((GW * RPI) % (RPL * CPR) == 0, "loads must start on a swizzle period");
  const int lr0 = w * RPI + lane / CPR, lpos = lane % CPR;  // row and chunk of load 0
  const uint32_t kgo = uint32_t((lr0 * rsk + (lpos ^ swz_k(lr0)) * 8) * 2);
  const uint32_t vgo = uint32_t((lr0 * rsk + (lpos ^ swz_v(lr0)) * 8) * 2);
  // A tile that runs past Sk loads key row Sk - 1 in place of the missing rows:
  // finite data whose scores the mask sets to -inf (weight 0).
  //
  // Addressing: one buffer resource per tensor at (batch b, key 0, K/V head)
  // for the whole walk, the tile's first key row and the load's row block as
  // the scalar offset, the lane's chunk as the vector offset. Where one
  // (batch, head) slab spans 2^31 bytes or more (the range of a resource and
  // of its offsets) the resource is rebuilt at every tile's first key row.
  const uint32_t rsk2 = uint32_t(rsk * 2);  // K/V token row stride, bytes
  const bool rebase = uint64_t(Sk) * rsk2 >= 0x7fffffffull;
  const uint64_t kaddr = reinterpret_cast<uint64_t>(p.k + hbk);
  const uint64_t vaddr = reinterpret_cast<uint64_t>(p.v + hbk);
  const i32x4 krs = buffer_rsrc(kaddr), vrs = buffer_rsrc(vaddr);
  const uint32_t lds_grp =
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds)) +
      uint32_t(grp * 4 * TB) + uint32_t(w * 1024);
  auto issue = [&](const i32x4& rs0, uint64_t addr, uint32_t go, int lbase, int t0, bool guard,
                   bool is_v) {
    i32x4 rs = rs0;
    uint32_t s0 = uint32_t(t0) * rsk2;
    if (rebase) {
      rs = buffer_rsrc(addr + uint64_t(t0) * rsk2);
      s0 = 0;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t soff = s0, off;
      if (guard) {  // rows are clamped relative to the tile's first row (< Sk)
        const int r = GW * RPI * i + lr0, rc = min(r, Sk - 1 - t0);
        off = uint32_t((rc * rsk + (lpos ^ (is_v ? swz_v(r) : swz_k(r))) * 8) * 2);
      } else {
        soff += uint32_t(GW * RPI * i) * rsk2;
        off = go;
      }
      load_lds16(rs, soff, off, lds_grp + uint32_t(lbase + GW * i * 1024));
    }
  };
  auto load_k = [&](int buf, int t0, bool guard) { issue(krs, kaddr, kgo, buf * TB, t0, guard, false); };
  auto load_v = [&](int buf, int t0, bool guard) {
    issue(vrs, vaddr, vgo, (2 + buf) * TB, t0, guard, true);
  };
  // the wave's direct loads have landed in LDS (a barrier then publishes them)
  auto loads_done = []() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // K row fed to A-operand row l32 (see the layout note above)
  const int a4 = l32 >> 3, g4 = (l32 >> 2) & 1, c4 = l32 & 3;
  const int pi = 16 * (a4 >> 1) + 8 * g4 + 4 * (a4 & 1) + c4;
  // per-lane byte offsets of the fragment reads within a K tile (k-step s,
  // key block 0) and a V tile (head-dim block db, key row 0); key blocks
  // and rows add uniform offsets, the swizzles depend on the lane only
  uint32_t kad[KS], vad[NDB];
#pragma unroll
  for (int st = 0; st < KS; ++st) kad[st] = uint32_t(pi * ROWB + (((2 * st + g) ^ swz_k(pi)) * 16));
  {
    // ds_read_b64_tr_b16: in each 16-lane group, lane j points at 4 bf16 of
    // row j / 4 (head-dim offset 4 (j mod 4)) and receives element j mod 4
    // of lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4: 4 keys of head
    // dim j. Lane l32 = 16 dh + j of half g covers keys 8 g + 4 half + (0..3).
    const int j = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vad[db] = uint32_t((8 * g + j / 4) * ROWB +
                         (((4 * db + 2 * dh + (j & 3) / 2) ^ swz_v(j / 4)) * 16) + (j & 1) * 8);
  }

  // ---- the per-tile steps ---------------------------------------------------
  // S^T = K Q^T for the K tile in ks[buf]
  auto qk = [&](int buf, f32x16 (&sacc)[NKB][QB]) {
    const f32x16 zero = {};  // first k-step: accumulator operand is the inline constant 0
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = as_bf16x8(
            *reinterpret_cast<const uint4*>(glds + buf * TB + kb * 32 * ROWB + kad[s]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][s],
                                                                  s == 0 ? zero : sacc[kb][qb], 0, 0, 0);
      }
    }
  };

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

  // row maxima of a score tile, moving the reference maxima (and rescaling O
  // and the row sums) where a row's maximum grew by more than kTau
  auto update_max = [&](f32x16 (&sacc)[NKB][QB]) {
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
      mx = max_halves(mx);
      mnew[qb] = fmaxf(mrow[qb], mx);
      need[qb] = (mnew[qb] - mrow[qb]) * c > kTau;
      any_need |= need[qb];
    }
    if (__any(any_need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mu = need[qb] ? mnew[qb] : mrow[qb];
        const float alpha = __builtin_amdgcn_exp2f((mrow[qb] - mu) * c);
        lrow[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
        mrow[qb] = mu;
      }
    }
  };

  // weights exp2(c s - c m) rounded to bf16 (the B operand of the P V
  // product) and their row sums
  auto weights = [&](f32x16 (&sacc)[NKB][QB], bf16x8 (&pf)[QB][NKB][2]) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = mrow[qb] * c;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 pv;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pv[j] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][8 * h2 + j], c, -mc));
          const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
          pf[qb][kb][h2] = pb;
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one, ls, false);
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one, ls, false);
        }
      }
      lrow[qb] += ls;
    }
  };

  // O^T += V^T P^T for the V tile in vt[buf]
  auto pv = [&](int buf, bf16x8 (&pf)[QB][NKB][2]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* vrow = glds + (2 + buf) * TB + (kb * 32 + h2 * 16) * ROWB + vad[db];
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrow));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vrow + 4 * ROWB));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb][h2], oacc[qb][db], 0, 0, 0);
        }
      }
    }
  };

  // keys at or past Sk get score -inf (weight 0); t0 is the tile's first key
  auto mask = [&](f32x16 (&sacc)[NKB][QB], int t0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = t0 + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
        if (key >= Sk) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[kb][qb][r] = -INFINITY;
        }
      }
  };

  // key tiles [kt_lo, kt_lo + nkt) of this group or part: half 0 is the
  // first nkt_all / 2 tiles (rounded down), half 1 the rest; tile indices
  // below are relative to kt_lo, so only the last tile of half 1 can be
  // partial. The halves depend on Sk and BN only.
  const int nkt_all = (Sk + BN - 1) / BN;
  constexpr bool kHalves = KG == 2 || PARTS == 2;
  const int half = KG == 2 ? grp : part;
  const int kt_lo = kHalves ? half * (nkt_all / 2) : 0;
  const int nkt = !kHalves ? nkt_all : half == 0 ? nkt_all / 2 : nkt_all - nkt_all / 2;
  auto key0 = [&](int kt) { return (kt_lo + kt) * BN; };      // first key of tile kt
  auto partial = [&](int kt) { return key0(kt) + BN > Sk; };  // tile runs past Sk

  // ---- the key walk: 2 + (nkt - 1) barriers when nkt > 0 ------------------
  if (nkt > 0) {
  // ---- prologue: K_0, V_0, K_1 in LDS; scores of tile 0 -------------------
  load_k(0, key0(0), partial(0));
  load_v(0, key0(0), partial(0));
  if (nkt > 1) load_k(1, key0(1), partial(1));
  loads_done();
  __syncthreads();

  f32x16 sa[NKB][QB], sb[NKB][QB];
  qk(0, sa);
  __syncthreads();  // every wave has read K_0 before step 0 refills buffer 0 with K_2

  // one steady-state iteration on tile kt (< nkt - 1): `cur` holds the scores
  // of tile kt, `nxt` receives those of tile kt + 1. At its start the step
  // loads K of tile kt + 2 into the K buffer tile kt used (read in the
  // previous step) and V of tile kt + 1 into the V buffer tile kt - 1 used;
  // the barrier at its end publishes both. With `full` true both tiles lie
  // wholly before Sk, so the loads carry no row guards.
  auto step = [&](auto full, int kt, f32x16 (&cur)[NKB][QB], f32x16 (&nxt)[NKB][QB]) {
    constexpr bool kFull = decltype(full)::value;
    if (kFull) {
      load_k(kt & 1, key0(kt + 2), false);
      load_v((kt + 1) & 1, key0(kt + 1), false);
    } else {
      if (kt + 2 < nkt) load_k(kt & 1, key0(kt + 2), partial(kt + 2));
      load_v((kt + 1) & 1, key0(kt + 1), partial(kt + 1));
    }
    update_max(cur);
    bf16x8 pf[QB][NKB][2];
    qk((kt + 1) & 1, nxt);  // MFMA: scores of the next tile ...
    weights(cur, pf);       // ... while the VALU turns this tile into weights
    pv(kt & 1, pf);
    loads_done();
    __syncthreads();
  };
  const std::integral_constant<bool, true> full;
  const std::integral_constant<bool, false> guarded;

  int kt = 0;
  // pairs of steps whose loads all lie before the (possibly partial) last tile
  for (; kt + 5 <= nkt; kt += 2) {
    step(full, kt, sa, sb);
    step(full, kt + 1, sb, sa);
  }
  for (; kt + 2 < nkt; kt += 2) {
    step(guarded, kt, sa, sb);
    step(guarded, kt + 1, sb, sa);
  }
  if (kt + 1 < nkt) {
    step(guarded, kt, sa, sb);
    ++kt;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sa[kb][qb] = sb[kb][qb];
  }

  // ---- last tile -------------------------------------------------------------
  {
    if (partial(kt)) mask(sa, key0(kt));
    update_max(sa);
    bf16x8 pf[QB][NKB][2];
    weights(sa, pf);
    pv(kt & 1, pf);
  }
  }  // nkt > 0

  if constexpr (KG == 2) {
    // the shorter walk (group 0, by at most one tile, or empty for a single
    // tile) matches the other group's barrier count
    const int n1 = nkt_all - nkt_all / 2;
    for (int i = nkt > 0 ? nkt + 1 : 0; i < n1 + 1; ++i) __syncthreads();
    __syncthreads();  // every wave is done with its tile buffers
    // Merge. Group 1 leaves its unnormalised O^T accumulators, reference
    // maxima and (lane-partial) row sums in LDS; wave w of group 0, which
    // owns the same 32 rows, weighs both sides by 2^(c (m_i - M)), M the
    // larger maximum (a group that saw no key has m = -inf, weight 0). The
    // arithmetic is spelled out (fmaf) because attn_merge_halves repeats it
    // bit for bit.
    f32x4* const mo = reinterpret_cast<f32x4*>(lds);
    float* const mm = reinterpret_cast<float*>(lds + GW * 64 * NDB * 16 * 4);
    float* const ml = mm + GW * 64;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = oacc[0][db][4 * a + e];
          mo[((w * NDB + db) * 4 + a) * 64 + lane] = x;
        }
      mm[w * 64 + lane] = mrow[0];
      ml[w * 64 + lane] = lrow[0];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = mm[w * 64 + lane], l1 = ml[w * 64 + lane];
    const float mx = fmaxf(mrow[0], m1);
    const float a0 = __builtin_amdgcn_exp2f((mrow[0] - mx) * c);
    const float a1 = __builtin_amdgcn_exp2f((m1 - mx) * c);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const f32x4 x = mo[((w * NDB + db) * 4 + a) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[0][db][4 * a + e] = fmaf(x[e], a1, oacc[0][db][4 * a + e] * a0);
      }
    lrow[0] = fmaf(l1, a1, lrow[0] * a0);
    mrow[0] = mx;
  }

  // ---- epilogue: normalise and store ------------------------------------------
  if constexpr (PARTS == 2) {
    // a key-half walk: the raw state goes to the workspace (rows past Sq too:
    // the merge skips them)
    const size_t ur = size_t(part) * p.n_tiles + lid;  // unit
    const int rloc = w * 32 + l32;                      // row within the tile
    float* const wo = p.ws_o + (ur * kTileRows + rloc) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[0][db][4 * a + e];
        *reinterpret_cast<f32x4*>(wo + db * 32 + 8 * a + 4 * g) = x;
      }
    if (g == 0) p.ws_m[ur * kTileRows + rloc] = mrow[0];
    p.ws_l[(ur * kTileRows + rloc) * 2 + g] = lrow[0];
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_halves(lrow[qb]);
    const float inv = 1.0f / lt;
    const int row = qrow0 + qb * 32 + l32;
    if (row < Sq) {
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
        p.lse[(size_t(b) * p.h + head) * Sq + row] = fmaf(mrow[qb], p.scale, logf(lt));
    }
  }
}

// Merges the two key-half states of every row left by the PARTS = 2 walks,
// with the arithmetic of the in-workgroup merge of the key-group kernel
// (and its epilogue), so both give the same bits. One thread per 4
// head-dim elements of a row; a row's threads are consecutive.
template <int D, bool kOutBf16>
__global__ __launch_bounds__(256) void attn_merge_halves(Params p) {
  constexpr int CH = D / 4;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(p.n_tiles) * kTileRows * CH) return;
  const int ch = int(idx % CH);
  const int64_t tr = idx / CH;
  const int r = int(tr % kTileRows), lid = int(tr / kTileRows);
  const int qt = lid % p.n_qtiles, bh = lid / p.n_qtiles;
  const int head = p.head_lo + bh % p.nheads, b = bh / p.nheads;
  const int row = qt * kTileRows + r;
  if (row >= p.Sq) return;
  const size_t u0 = size_t(lid) * kTileRows + r, u1 = (size_t(p.n_tiles) + lid) * kTileRows + r;
  const float m0 = p.ws_m[u0], m1 = p.ws_m[u1];
  const float mx = fmaxf(m0, m1);
  const float a0 = __builtin_amdgcn_exp2f((m0 - mx) * p.c);
  const float a1 = __builtin_amdgcn_exp2f((m1 - mx) * p.c);
  const float lg0 = fmaf(p.ws_l[u1 * 2], a1, p.ws_l[u0 * 2] * a0);
  const float lg1 = fmaf(p.ws_l[u1 * 2 + 1], a1, p.ws_l[u0 * 2 + 1] * a0);
  const float lt = lg0 + lg1;
  const float inv = 1.0f / lt;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(p.ws_o + u0 * D + ch * 4);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(p.ws_o + u1 * D + ch * 4);
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = fmaf(x1[e], a1, x0[e] * a0) * inv;
  const size_t ob = ((size_t(b) * p.Sq + row) * p.h + head) * D + ch * 4;
  if (kOutBf16)
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.o) + ob) = __builtin_convertvector(y, bf16x4);
  else
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + ob) = y;
  if (p.lse && ch == 0) p.lse[(size_t(b) * p.h + head) * p.Sq + row] = fmaf(mx, p.scale, logf(lt));
}

// Whether a row's key walk is split into two halves: a function of the key
// count and the tile size only, so every launch form and head range gives a
// row the same arithmetic. Short walks (under 8 tiles) are not split: the
// merge would cost more than the balance gains. Very long ones (over 1024
// tiles) are not either: ceil(S / 256) query tiles then fill at least a
// round of workgroups per head and batch row, so whole walks leave a short
// tail and save the merge.
#ifndef USP_SPLIT_MIN
#define USP_SPLIT_MIN 8
#endif
#ifndef USP_SPLIT_MAX
#define USP_SPLIT_MAX 1024
#endif
bool split_keys(int64_t Sk, int BN) {
  const int64_t nkt = (Sk + BN - 1) / BN;
  return nkt >= USP_SPLIT_MIN && nkt <= USP_SPLIT_MAX;
}

// Bytes of the key-half workspace for `tiles` tiles of 256 rows.
size_t halves_ws_bytes(int64_t tiles, int D) {
  return size_t(tiles) * 2 * kTileRows * (size_t(D) + 3) * sizeof(float);
}

// Short walks at D = 64: fewer than USP_SPLIT_MIN key tiles of BN, walked in
// 64-key tiles by 4-wave workgroups of 128 rows, three per CU (164 VGPRs),
// instead of 8-wave workgroups of 256 rows, one per CU. A short walk is
// mostly the fixed cost of its workgroup; the smaller workgroups pad a
// ragged last query tile less and fill the CUs in fewer rounds (ViT-L/16,
// S = 577: 768 row-slots of 128 in one round against 384 of 256 in one and
// a half; 378 against 307 TF/s). Measured: no gain at longer walks, and
// 64-key tiles in 8-wave workgroups lose 13% at S = 65537.
constexpr int kShortBN = 64;
bool short_walk(int64_t Sk, int D, int BN) {
  return D == 64 && (Sk + BN - 1) / BN < USP_SPLIT_MIN;
}

template <int D, int BN, bool kOutBf16>
int launch_tiles(Params& p, int64_t tiles, void* ws, bool whole, hipStream_t s) {
  if constexpr (D == 64) {
    if (short_walk(p.Sk, D, BN)) {
      // two 128-row workgroups per 256-row tile; no state to merge
      attn_bf16_kernel<D, 4, 1, 1, kShortBN, kOutBf16><<<unsigned(tiles * 2), 256, 0, s>>>(p);
      return check_launch("attn_bf16_kernel (short walks)");
    }
  }
  if (whole || !split_keys(p.Sk, BN)) {
    // whole key walks in 256-row workgroups: no state to merge, no workspace
    attn_bf16_kernel<D, 8, 1, 1, BN, kOutBf16><<<unsigned(tiles), 512, 0, s>>>(p);
    return check_launch("attn_bf16_kernel (whole walks)");
  }
  if (!ws) {
    // key groups: two 128-row workgroups per tile
    attn_bf16_kernel<D, 8, 2, 1, BN, kOutBf16><<<unsigned(tiles * 2), 512, 0, s>>>(p);
    return check_launch("attn_bf16_kernel");
  }
  // key halves in separate 256-row workgroups, then the merge
  p.n_tiles = int(tiles);
  p.ws_o = static_cast<float*>(ws);
  p.ws_m = p.ws_o + size_t(tiles) * 2 * kTileRows * D;
  p.ws_l = p.ws_m + size_t(tiles) * 2 * kTileRows;
  attn_bf16_kernel<D, 8, 1, 2, BN, kOutBf16><<<unsigned(tiles * 2), 512, 0, s>>>(p);
  if (int st = check_launch("attn_bf16_kernel (key halves)")) return st;
  const int64_t threads = tiles * kTileRows * (D / 4);
  attn_merge_halves<D, kOutBf16><<<unsigned((threads + 255) / 256), 256, 0, s>>>(p);
  return check_launch("attn_merge_halves");
}

template <int D, int BN>
int launch(const AttnArgs& a, hipStream_t s) {
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = a.o;
  p.lse = a.lse;
  p.Sq = int(a.S);
  p.Sk = int(a.Sk);
  p.h = a.h;
  p.head_lo = a.head_lo;
  p.nheads = a.head_hi - a.head_lo;
  p.h_kv = a.h_kv;
  p.grp = a.h / a.h_kv;
  p.n_qtiles = int((a.S + kTileRows - 1) / kTileRows);
  p.c = a.scale * 1.4426950408889634f;
  p.scale = a.scale;
  p.n_tiles = 0;
  p.ws_o = p.ws_m = p.ws_l = nullptr;
  const int64_t tiles = int64_t(p.n_qtiles) * p.nheads * a.B;
  if (tiles > 0x3fffffff || (a.ws && tiles * (a.D / 4) > 0x7fffffff))
    return fail(USP_ESHAPE, "attention grid too large");
  if (a.ws && a.ws_bytes < halves_ws_bytes(tiles, a.D))
    return fail(USP_EINVAL, "workspace of %zu bytes is below the %zu this call needs", a.ws_bytes,
                halves_ws_bytes(tiles, a.D));
  return a.out_dt == USP_BF16 ? launch_tiles<D, BN, true>(p, tiles, a.ws, a.whole, s)
                              : launch_tiles<D, BN, false>(p, tiles, a.ws, a.whole, s);
}

}  // namespace

bool attention_bf16_splits(int64_t Sk, int32_t D) {
  switch (D) {
    case 128:
      return split_keys(Sk, USP_D128_BN);
    case 64:
      return split_keys(Sk, USP_D64_BN);
    default:
      return false;
  }
}

size_t attention_bf16_ws_bytes(int64_t B, int64_t S, int32_t heads, int32_t D) {
  return halves_ws_bytes((S + kTileRows - 1) / kTileRows * heads * B, D);
}

int launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  switch (a.D) {
    case 128:
      return launch<128, USP_D128_BN>(a, s);
    case 64:
      return launch<64, USP_D64_BN>(a, s);
    default:
      return fail(USP_ENOSYS, "bf16 attention: unsupported D %d", a.D);
  }
}

}  // namespace usp
