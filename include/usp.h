/*
 * usp.h — C ABI of libusp, the MI355X (gfx950) hot path of Ulysses sequence
 * parallelism: one rank's share of the work, at its real shape.
 *
 * The method (m-star "sequence_parallel" API page, module description):
 * tokens are sharded over an SP group of P ranks; around attention, a first
 * all-to-all turns each rank's sequence shard [seq/P, H, D] into the full
 * sequence over its own head group [seq, H/P, D], attention runs locally per
 * head, and a second all-to-all turns the result back. On one GPU the
 * exchange is replaced by local permutations into "world layouts" that hold
 * every rank's buffers side by side:
 *
 *   sequence-sharded world  seq[B][S][H][D], rank r owns token rows
 *                           [t_r, t_{r+1}) of every batch row;
 *   head-sharded world      P blocks, block j is blk_j[B][S][h_j][D] and holds
 *                           heads [c_j, c_{j+1}) — exactly what rank j holds
 *                           after the first all-to-all.
 *
 * Conventions shared by every call:
 *   - All tensors are dense row-major, element type USP_F32 (4 bytes) or
 *     USP_BF16 (2 bytes, bfloat16). Device pointers must be 16-byte aligned.
 *   - The caller owns every buffer it passes. The library never
 *     synchronizes; device work is enqueued on the caller's stream (a
 *     hipStream_t passed as void*; NULL = the default stream) and the call
 *     returns without waiting for it. The only device memory the library
 *     takes itself: an attention call given no workspace takes one, where
 *     its shape needs one, from a stream-ordered pool the library keeps per
 *     device (allocated and returned on the caller's stream; never during
 *     graph capture), and usp_attention_fwd_noalloc's static scratch array.
 *   - Every call returns USP_OK (0) or a negative status. On error nothing is
 *     launched and no output is written; usp_last_error() gives a message.
 *   - Sizes are validated against overflow; a launch failure reported by the
 *     HIP runtime is returned as USP_EHIP.
 */
#ifndef USP_H
#define USP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum usp_dtype { USP_F32 = 0, USP_BF16 = 1 } usp_dtype;

enum {
  USP_OK = 0,
  USP_EINVAL = -1, /* an argument is out of its domain (counts, ranks, ranges) */
  USP_ESHAPE = -2, /* sizes are inconsistent or overflow */
  USP_EDTYPE = -3, /* element type not supported for this call */
  USP_EALIGN = -4, /* a pointer or row is not 16-byte aligned */
  USP_ENOSYS = -5, /* a valid request the library has no kernel for */
  USP_EHIP = -6    /* the HIP runtime reported an error */
};

/* Largest SP degree the relayout calls accept (block pointers travel as
 * kernel arguments). */
#define USP_MAX_PARTS 64
/* Most tensors one usp_*_planes relayout call moves. */
#define USP_MAX_PLANES 4

/* Message for the last non-zero status returned on the calling thread
 * (thread-local; "" if none). The string stays valid until the next call. */
const char* usp_last_error(void);

/* Library version string, e.g. "usp 0.1.0 gfx950". */
const char* usp_version(void);

/*
 * Balanced contiguous ranges (h3-blackwell-runtime distributed.py,
 * balanced_ranges; m-star sp_seq_split): cut the item indices
 * 0 .. total-1 into `parts` consecutive runs of at least one item; with
 * base = total / parts and
 * extra = total % parts, range r has base + (r < extra) items: the first
 * `extra` ranges hold one item more than the others.
 *   bounds: caller-owned host array of parts + 1 int64; on success
 *           bounds[0] = 0, bounds[parts] = total, range r = [bounds[r],
 *           bounds[r+1]).
 * Errors: parts < 1 or total < parts -> USP_EINVAL; bounds NULL -> USP_EINVAL.
 */
int usp_balanced_ranges(int64_t total, int32_t parts, int64_t* bounds);

/* The same boundaries computed on the device by a kernel on `stream` into the
 * caller-owned device array d_bounds[parts + 1] (8-byte aligned). Same
 * errors as usp_balanced_ranges. */
int usp_balanced_ranges_device(int64_t total, int32_t parts, int64_t* d_bounds,
                               void* stream);

/*
 * Head-chunk plan (maxdiffusion PR #428, two-phase head-chunked Ulysses
 * all-to-all: heads run in `chunks` passes, the final chunk carrying the
 * remainder). Every chunk but the last holds ceil(heads / chunks) heads; the
 * last holds the rest (8 heads in 3 chunks: 3/3/2).
 *   bounds: caller-owned host array of chunks + 1 int32.
 * Errors: heads < 1, chunks < 1, chunks > heads, or a plan that would leave a
 * chunk empty (e.g. 5 heads in 4 chunks) -> USP_EINVAL.
 */
int usp_head_chunk_ranges(int32_t heads, int32_t chunks, int32_t* bounds);

/*
 * Sequence-sharded -> head-sharded relayout (the data movement around the
 * first all-to-all: h3-blackwell-runtime distributed.py,
 * SequenceParallelContext.seq_to_heads; m-star sp_head_slice for the head
 * groups). Token ranges t = balanced(S, P), head ranges c = balanced(H, P).
 *   rank < 0  (world): seq is [B][S][H][D]; for every j, b, s, i, d:
 *             blk[j][b][s][i][d] = seq[b][s][c_j + i][d].
 *   rank = r  (one rank's share): seq is r's compact shard [B][len_r][H][D]
 *             and only rows [t_r, t_{r+1}) of every block are written:
 *             blk[j][b][t_r + s][i][d] = seq[b][s][c_j + i][d].
 *   blk: host array of P device pointers, block j of [B][S][h_j][D]. In a
 *        multi-GPU system these are the peers' receive buffers.
 *   P = 1 copies seq byte for byte. Pure data movement: results are exact.
 * Errors: P < 1, P > USP_MAX_PARTS, S < P, H < P, rank >= P -> USP_EINVAL;
 *   B < 1, D < 1 or byte sizes overflowing int64 -> USP_ESHAPE; dtype not
 *   F32/BF16 -> USP_EDTYPE; D * element size not a multiple of 16 or a
 *   pointer not 16-byte aligned -> USP_EALIGN; seq, blk or blk[j] NULL ->
 *   USP_EINVAL. Buffers must not overlap.
 */
int usp_pack_seq_to_heads(const void* seq, void* const* blk, usp_dtype dtype, int64_t B,
                          int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                          void* stream);

/*
 * Head-sharded -> sequence-sharded relayout (the data movement around the
 * second all-to-all: h3-blackwell-runtime distributed.py,
 * SequenceParallelContext.heads_to_seq). Exact inverse of the pack:
 *   rank < 0: seq[b][s][c_j + i][d] = blk[j][b][s][i][d] for all rows;
 *   rank = r: seq is r's shard [B][len_r][H][D],
 *             seq[b][s][c_j + i][d] = blk[j][b][t_r + s][i][d].
 * Same arguments and errors as usp_pack_seq_to_heads.
 */
int usp_unpack_heads_to_seq(const void* const* blk, void* seq, usp_dtype dtype, int64_t B,
                            int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                            void* stream);

/*
 * One phase of the head-chunked (two-phase) exchange (maxdiffusion PR #428,
 * "two-phase (head-chunked) Ulysses all-to-all", description: the exchange
 * and the attention run once per chunk of every rank's heads, so that one
 * chunk's exchange can overlap another chunk's attention). With P equal head
 * groups of h = H / P heads (c_j = j * h), only heads [head_lo, head_hi) of
 * every group move; the chunk plan over h comes from usp_head_chunk_ranges.
 *   usp_pack_seq_to_heads_chunk, for head_lo <= i < head_hi:
 *     rank < 0: blk[j][b][s][i][d] = seq[b][s][c_j + i][d] for all rows;
 *     rank = r: blk[j][b][t_r + s][i][d] = seq[b][s][c_j + i][d] (seq = r's
 *               shard [B][len_r][H][D]).
 *   usp_unpack_heads_to_seq_chunk: the inverse for the same heads and rows.
 * Nothing outside those heads (and, for rank >= 0, those rows) is read from
 * the source or written to the destination, so a tensor's phases may run in
 * any order or overlap each other's and other chunks' work; over a whole
 * chunk plan they give exactly usp_pack_seq_to_heads / usp_unpack_heads_to_seq.
 * Arguments, layouts and errors as usp_pack_seq_to_heads, plus: H not a
 * multiple of P (ragged head groups), or [head_lo, head_hi) empty or outside
 * [0, H / P) -> USP_EINVAL.
 */
int usp_pack_seq_to_heads_chunk(const void* seq, void* const* blk, usp_dtype dtype, int64_t B,
                                int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                                int32_t head_lo, int32_t head_hi, void* stream);
int usp_unpack_heads_to_seq_chunk(const void* const* blk, void* seq, usp_dtype dtype, int64_t B,
                                  int64_t S, int32_t H, int32_t D, int32_t P, int32_t rank,
                                  int32_t head_lo, int32_t head_hi, void* stream);

/*
 * Several tensors of one shape through the same relayout in one launch
 * (h3-blackwell-runtime distributed.py, SequenceParallelContext.seq_to_heads
 * moves q, k and v of a layer together): plane t of n is
 * usp_pack_seq_to_heads(seq[t], &blk[t * P], ...) (head_lo = head_hi = 0)
 * or usp_pack_seq_to_heads_chunk(seq[t], &blk[t * P], ..., head_lo,
 * head_hi, ...), and the unpack likewise; the planes stay separate tensors.
 *   n:   1 .. USP_MAX_PLANES planes.
 *   seq: host array of n device pointers (pack: sources; unpack:
 *        destinations), each a tensor as in the single-plane call.
 *   blk: host array of n * P device pointers, plane-major: block j of
 *        plane t at blk[t * P + j].
 * The result is bitwise the n single-plane calls'. Errors: n outside
 * [1, USP_MAX_PLANES] or seq/blk NULL -> USP_EINVAL; otherwise those of the
 * single-plane calls for every plane (the head-chunk checks when head_lo or
 * head_hi is non-zero).
 */
int usp_pack_seq_to_heads_planes(int32_t n, const void* const* seq, void* const* blk,
                                 usp_dtype dtype, int64_t B, int64_t S, int32_t H, int32_t D,
                                 int32_t P, int32_t rank, int32_t head_lo, int32_t head_hi,
                                 void* stream);
int usp_unpack_heads_to_seq_planes(int32_t n, const void* const* blk, void* const* seq,
                                   usp_dtype dtype, int64_t B, int64_t S, int32_t H, int32_t D,
                                   int32_t P, int32_t rank, int32_t head_lo, int32_t head_hi,
                                   void* stream);

/*
 * Ragged token rows at the model boundary, without padding. A tensor
 * [B][S][W] (W = elements per token row, e.g. H * D) is split along S into
 * P contiguous balanced ranges [t_r, t_{r+1}) (usp_balanced_ranges(S, P));
 * shard r is [B][len_r][W], row-major, contiguous. All pointers are device
 * pointers owned by the caller, 16-byte aligned, and W * element size must
 * be a multiple of 16. Errors (all three): P outside [1, USP_MAX_PARTS],
 * S < P, rank >= P, null pointers -> USP_EINVAL; B < 1, W < 1 or sizes
 * overflowing -> USP_ESHAPE; unknown dtype -> USP_EDTYPE; misalignment ->
 * USP_EALIGN; a HIP launch error -> USP_EHIP.
 *
 * usp_scatter_rows (m-star scatter_sequence: with the full tensor replicated
 * on every rank, each narrows to its own window, no communication): copies
 * rows [t_r, t_{r+1}) of `full` into shards[r], for every r (rank < 0; all P
 * pointers set) or for r = rank only (only shards[rank] need be set).
 */
int usp_scatter_rows(const void* full, void* const* shards, usp_dtype dtype, int64_t B, int64_t S,
                     int64_t W, int32_t P, int32_t rank, void* stream);

/*
 * usp_gather_rows (m-star gather_sequence, h3-blackwell-runtime
 * SequenceParallelContext.all_gather_rows: the P shards laid end to end in
 * rank order rebuild the unsharded tensor, with no padding rows):
 * full[b][t_r + i] = shards[r][b][i] for every r.
 */
int usp_gather_rows(const void* const* shards, void* full, usp_dtype dtype, int64_t B, int64_t S,
                    int64_t W, int32_t P, void* stream);

/*
 * usp_reduce_scatter_rows (h3-blackwell-runtime
 * SequenceParallelContext.reduce_scatter_rows: every rank holds a partial
 * sum of the full sequence, e.g. a tensor-parallel partial, and receives its
 * own rows of the total): out[r][b][i] = sum_{j=0}^{P-1} partials[j][b][t_r + i]
 * for every r (rank < 0) or r = rank, the P partials [B][S][W] added in
 * rank order in fp32 and rounded once to the dtype (round to nearest even
 * for USP_BF16). Only out[rank] need be set when rank >= 0.
 */
int usp_reduce_scatter_rows(const void* const* partials, void* const* out, usp_dtype dtype,
                            int64_t B, int64_t S, int64_t W, int32_t P, int32_t rank,
                            void* stream);

/*
 * Non-causal multi-head attention over the full sequence for heads
 * [head_lo, head_hi) of one head-group block (m-star ulysses_attention: the
 * rank runs the unchanged attention kernel on [seq, H/P, D]). For each b,
 * head n in range, query s:
 *   O[b][s][n][:] = sum_t softmax_t(scale * <Q[b][s][n][:], K[b][t][n][:]>)
 *                   * V[b][t][n][:]
 *   q, k, v, o: device [B][S][h][D] (h = heads of the block); heads outside
 *               the range are neither read nor written.
 *   in_dt:  USP_BF16 (flash kernel on MFMA; D in {64, 128}) or USP_F32
 *           (plain fp32 kernel; D in {32, 64, 128}).
 *   out_dt: USP_F32 or USP_BF16 for bf16 inputs; USP_F32 for fp32 inputs.
 *   scale:  softmax scale; <= 0 selects 1/sqrt(D).
 *   lse:    NULL, or device fp32 [B][h][S] receiving the natural-log softmax
 *           normaliser log(sum_t exp(scale * <Q, K_t>)) for heads in range.
 * Scores, softmax and accumulation are fp32. The result for a head depends
 * only on that head's inputs, never on [head_lo, head_hi), B or the device:
 * a head computed in any sub-range is bitwise equal to the same head computed
 * single-shot. With bf16 inputs and keys that split in halves (walks of 8 to
 * 1024 key tiles, a rule of S and D only), the call takes the workspace of
 * usp_attention_fwd_ws from a stream-ordered memory pool the library keeps
 * per device (hipMallocFromPoolAsync before the kernels, hipFreeAsync after
 * them, on `stream`; the pool keeps the memory for later calls) and runs the
 * same kernels, with the same bits. While `stream` is being captured into a
 * graph, when the pool cannot serve, or with the environment variable
 * USP_ATTENTION_POOL=0 (read at every call), it allocates nothing and runs a
 * kernel in which two groups of waves walk the two key halves of 128 query
 * rows and merge their softmax states in LDS: the same bits again. Shapes
 * whose keys do not split need no workspace at all.
 * Errors: h < 1, head range empty or outside [0, h) -> USP_EINVAL;
 *   B < 1, S < 1 or sizes overflowing -> USP_ESHAPE; unsupported
 *   in_dt/out_dt pair -> USP_EDTYPE; unsupported D -> USP_ENOSYS; misaligned
 *   pointers -> USP_EALIGN; q, k, v or o NULL -> USP_EINVAL.
 */
int usp_attention_fwd(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                      usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t D,
                      int32_t head_lo, int32_t head_hi, float scale, float* lse, void* stream);

/*
 * Device workspace (bytes) usp_attention_fwd_ws needs for `heads` heads
 * (head_hi - head_lo) of B batches of S tokens: 0 for USP_F32 inputs, else
 * B * heads * ceil(S / 256) * 2 * 256 * (D + 3) * 4 (171.7 MB for B = 1,
 * heads = 5, S = 32760, D = 128). Written to *bytes.
 * Errors: bytes NULL -> USP_EINVAL; a size < 1 or too large for one launch
 *   -> USP_ESHAPE; unknown in_dt -> USP_EDTYPE.
 */
int usp_attention_workspace_bytes(usp_dtype in_dt, int64_t B, int64_t S, int32_t heads, int32_t D,
                                  size_t* bytes);

/*
 * usp_attention_fwd with a caller-provided device workspace (the same
 * operation and result, bitwise, as usp_attention_fwd). With bf16 inputs
 * each tile of 256 query rows is computed by two workgroups, one per key
 * half, that leave their unnormalised softmax state in `ws`; a second
 * kernel merges the halves exactly as usp_attention_fwd's workgroups merge
 * them in LDS. This keeps one K/V stream per workgroup (the key-group kernel,
 * which usp_attention_fwd runs when it cannot take a workspace, streams two
 * per 128 rows) and is the faster path.
 *   ws, ws_bytes: device buffer, 16-byte aligned, of at least
 *                 usp_attention_workspace_bytes(in_dt, B, S, head_hi -
 *                 head_lo, D) bytes, owned by the caller; its contents on
 *                 entry do not matter and are undefined on return. Calls
 *                 that may overlap must not share one. Ignored (may be NULL)
 *                 for USP_F32 inputs.
 * Other arguments, layouts and errors as usp_attention_fwd, plus: bf16
 * inputs with ws NULL or ws_bytes too small -> USP_EINVAL; ws misaligned ->
 * USP_EALIGN.
 */
int usp_attention_fwd_ws(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                         usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t D,
                         int32_t head_lo, int32_t head_hi, float scale, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * usp_attention_fwd_noalloc: usp_attention_fwd_ws with its workspace taken
 * from device memory the library reserves statically, for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It calls no allocating routine; the
 * caller still owns q, k, v, o and lse. The same kernels and the same bits
 * as usp_attention_fwd_ws (and usp_attention_fwd).
 *   Limit: the bf16 path needs usp_attention_workspace_bytes(in_dt, B, S,
 *          head_hi - head_lo, D) bytes of scratch, at most
 *          USP_NOALLOC_SCRATCH_BYTES (192 MiB: the video-DiT share of
 *          B = 1, S = 32760, 5 heads, D = 128 needs 171.7 MB); larger calls
 *          fail with USP_EINVAL before any launch (split them into head
 *          ranges). fp32 inputs need no scratch.
 *   The scratch is one array per GPU, held from the library's first use on
 *   that GPU until the process ends, and shared by every call on it: calls
 *   that may overlap on one GPU (other streams, other threads) race and
 *   must be serialised by the caller. Its contents do not need clearing.
 * Arguments, layouts and other errors as usp_attention_fwd, plus: the
 *   device of `stream` cannot be determined or its scratch address looked
 *   up -> USP_EHIP.
 */
#define USP_NOALLOC_SCRATCH_BYTES (192u << 20)
int usp_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                              usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S, int32_t h,
                              int32_t D, int32_t head_lo, int32_t head_hi, float scale, float* lse,
                              void* stream);

/*
 * Attention with grouped key/value heads (m-star ulysses_attention: q holds
 * Hq heads, k and v Hkv, both divisible by the SP degree, so each rank's head
 * group is [seq, Hq/P, D] against [seq, Hkv/P, D]): as usp_attention_fwd over
 * query heads [head_lo, head_hi) of q and o [B][S][h][D], with k and v
 * [B][S][h_kv][D]; query head n attends with key/value head n / (h / h_kv),
 * i.e. each run of h / h_kv consecutive query heads shares one K/V head.
 * h_kv = h is usp_attention_fwd. The result of a query head depends only on
 * its inputs (bitwise, as for usp_attention_fwd), so a caller may run head
 * chunks over any query-head ranges.
 *   ws, ws_bytes: NULL (the call then takes a workspace from the pool, as
 *                 usp_attention_fwd does), or a workspace as for
 *                 usp_attention_fwd_ws (sized by usp_attention_workspace_bytes
 *                 for head_hi - head_lo heads); all give the same bits.
 * Errors as usp_attention_fwd_ws, plus: h_kv < 1, h_kv > h or h not a
 * multiple of h_kv -> USP_EINVAL.
 */
int usp_attention_fwd_gqa(const void* q, const void* k, const void* v, void* o, usp_dtype in_dt,
                          usp_dtype out_dt, int64_t B, int64_t S, int32_t h, int32_t h_kv,
                          int32_t D, int32_t head_lo, int32_t head_hi, float scale, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Attention of a query block against one key/value block of another length
 * (Ulysses+Ring, maxdiffusion PR #428 description: under a ring over a second
 * sequence axis, rank (r, j) of a U x R grid holds the query rows of ring
 * block r for head group j and attends them to the K/V block of every ring
 * member in turn; the per-block results combine by usp_attention_merge).
 * For each b, query head n in [head_lo, head_hi), query row s < Sq:
 *   O[b][s][n][:] = sum_{t < Sk} softmax_t(scale * <Q[b][s][n][:], K[b][t][m][:]>)
 *                   * V[b][t][m][:],   m = n / (h / h_kv)
 *   q, o: device [B][Sq][h][D];  k, v: device [B][Sk][h_kv][D].
 *   lse:  NULL, or device fp32 [B][h][Sq] receiving the natural-log
 *         normaliser over this block's Sk keys (what the merge needs).
 *   ws, ws_bytes: NULL (a workspace from the pool, as usp_attention_fwd),
 *         or a workspace as for usp_attention_fwd_ws sized by
 *         usp_attention_workspace_bytes(in_dt, B, Sq, head_hi - head_lo, D)
 *         (it depends on the query rows only); all give the same bits.
 * Sq = Sk with the same tensors is usp_attention_fwd_gqa, bit for bit, and a
 * query row's result depends only on its own row and the key block: running
 * a query block as any split of its rows gives the same bits.
 * Other arguments and dtypes as usp_attention_fwd_gqa. Errors as
 * usp_attention_fwd_gqa, plus: Sk < 1 or k/v sizes overflowing ->
 * USP_ESHAPE.
 */
int usp_attention_fwd_block(const void* q, const void* k, const void* v, void* o,
                            usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t Sq, int64_t Sk,
                            int32_t h, int32_t h_kv, int32_t D, int32_t head_lo, int32_t head_hi,
                            float scale, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * usp_attention_fwd_block for the key blocks of a ring pass that run at the
 * same time on separate streams (Ulysses+Ring, maxdiffusion PR #428
 * description; a ring brings the next K/V block while the rank still
 * attends to the current one). It computes the same O and lse, but every query row walks
 * all Sk keys in one pass: no key-half split, so no workspace and no merge
 * of halves. Launches on two streams then fill each other's last rounds of
 * work; a launch alone runs a part-empty last round wherever
 * B * (head_hi - head_lo) * ceil(Sq / 256) is not a multiple of the CU count
 * (usp_attention_fwd_block is the form for one stream).
 * Where usp_attention_fwd_block does not split the keys (fp32 inputs; bf16
 * with fewer than 8 or more than 1024 key tiles of 64 keys at D = 128, of 128
 * at D = 64) both give the same bits; elsewhere they differ by rounding only.
 * A query row's result depends only on its own row and the key block, as for
 * usp_attention_fwd_block. Allocates nothing. Arguments and errors as
 * usp_attention_fwd_block without ws and ws_bytes.
 */
int usp_attention_fwd_block_whole(const void* q, const void* k, const void* v, void* o,
                                  usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t Sq,
                                  int64_t Sk, int32_t h, int32_t h_kv, int32_t D, int32_t head_lo,
                                  int32_t head_hi, float scale, float* lse, void* stream);

/*
 * Log-sum-exp merge of two attention results of the same query rows over
 * disjoint key blocks (the fold of one Ulysses+Ring step; softmax over the
 * union of the two key sets). For heads n in [head_lo, head_hi):
 *   lse = log(exp(lse_a) + exp(lse_b)),
 *   O   = exp(lse_a - lse) * O_a + exp(lse_b - lse) * O_b,
 * computed in fp32 as M = max(lse_a, lse_b), e_x = exp(lse_x - M),
 * lse = M + log(e_a + e_b), O = (e_a / (e_a + e_b)) O_a + (e_b / (e_a + e_b)) O_b.
 * A block with lse = -inf counts with weight 0; rows whose two lse are both
 * -inf get O = 0, lse = -inf.
 *   o_a, o_b: device fp32 [B][S][h][D] (block outputs, normalised per block).
 *   lse_a, lse_b: device fp32 [B][h][S] (their normalisers, as usp_attention_*
 *             write them).
 *   o:        device [B][S][h][D] of out_dt (USP_F32 or USP_BF16, rounded
 *             to nearest even); may be exactly o_a or o_b when out_dt is
 *             USP_F32 (in-place accumulation), else must not overlap them.
 *   lse:      NULL, or device fp32 [B][h][S]; may be exactly lse_a or lse_b,
 *             else must not overlap them.
 * Heads outside the range are neither read nor written. The fold order of
 * several blocks changes the result only by rounding.
 * Errors: a NULL pointer other than lse, h < 1 or an empty/outside head
 *   range, or a bf16 o equal to o_a or o_b -> USP_EINVAL; B < 1, S < 1 or
 *   sizes too large -> USP_ESHAPE; out_dt unknown -> USP_EDTYPE; D not in
 *   {32, 64, 128} -> USP_ENOSYS; o_a, o_b or o not 16-byte aligned, or an
 *   lse pointer not 4-byte aligned -> USP_EALIGN.
 */
int usp_attention_merge(const float* o_a, const float* lse_a, const float* o_b,
                        const float* lse_b, void* o, float* lse, usp_dtype out_dt, int64_t B,
                        int64_t S, int32_t h, int32_t D, int32_t head_lo, int32_t head_hi,
                        void* stream);

/*
 * Head-chunked attention (maxdiffusion PR #428, two-phase Ulysses: attention
 * over head sub-groups in turn, mathematically the single-shot result since
 * heads are independent): runs usp_attention_fwd over each range of
 * usp_head_chunk_ranges(h, chunks) in order on `stream`. Bitwise equal to
 * the single-shot call. Errors: those of usp_head_chunk_ranges and
 * usp_attention_fwd.
 */
int usp_attention_fwd_chunked(const void* q, const void* k, const void* v, void* o,
                              usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S,
                              int32_t h, int32_t D, float scale, float* lse, int32_t chunks,
                              void* stream);

/*
 * usp_attention_fwd_chunked with a caller workspace: each pass runs
 * usp_attention_fwd_ws's kernels. Bitwise equal to usp_attention_fwd_chunked,
 * usp_attention_fwd and usp_attention_fwd_ws.
 *   ws, ws_bytes: device buffer, 16-byte aligned, of at least
 *                 usp_attention_workspace_bytes(in_dt, B, S, c, D) bytes with
 *                 c = ceil(h / chunks) (the largest pass), owned by the
 *                 caller, reused by every pass; contents on entry do not
 *                 matter. Ignored (may be NULL) for USP_F32 inputs.
 * Errors: those of usp_attention_fwd_chunked, plus bf16 inputs with ws NULL
 * or ws_bytes too small -> USP_EINVAL, ws misaligned -> USP_EALIGN.
 */
int usp_attention_fwd_chunked_ws(const void* q, const void* k, const void* v, void* o,
                                 usp_dtype in_dt, usp_dtype out_dt, int64_t B, int64_t S,
                                 int32_t h, int32_t D, float scale, float* lse, int32_t chunks,
                                 void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* USP_H */
