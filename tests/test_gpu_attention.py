"""GPU parity of attention against the float64 oracle.

Tolerances: bf16 inputs graded on the fp32-output epilogue, max-abs <= 1e-2
and relative Frobenius <= 5e-3; the fp32 path <= 1e-5 for both. The bf16
output epilogue is graded per element within max(1e-2, one bf16 ulp of the
reference)."""
import numpy as np
import pytest

import ulysses_sequence_attention_amd as usp
from oracle import attention as A
from oracle import ranges as R
from oracle import relayout as X
from ulysses_sequence_attention_amd import synth

from gpu_util import (BF16_LSE_ABS, BF16_MAX_ABS, BF16_REL_FROB, DEV, F32_MAX_ABS, F32_REL_FROB, bf16_ulp, err,
                      log, no_pool, poisoned, to_dev, to_host, widen)

pytestmark = pytest.mark.gpu
BF, F = synth.BF16, synth.F32


def _run(q, k, v, dtype, out_dtype, lo=0, hi=None, scale=0.0, want_lse=False, chunks=None,
         chunk_ws=False):
    import torch
    B, S, h, D = q.shape
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o = poisoned((B, S, h, D), out_dtype)
    lse = torch.full((B, h, S), float("nan"), device=DEV) if want_lse else None
    if chunks is None:
        usp.usp_attention_fwd(dq, dk, dv, o, head_lo=lo, head_hi=hi, scale=scale, lse=lse)
    elif chunk_ws:
        # workspace for the largest pass, NaN-poisoned, exactly the size asked for
        nb = usp.usp_attention_workspace_bytes(usp.USP_BF16 if dtype == BF else usp.USP_F32, B, S,
                                               -(-h // chunks), D)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), device=DEV)
        usp.usp_attention_fwd_chunked_ws(dq, dk, dv, o, chunks, ws, scale=scale, lse=lse)
    else:
        usp.usp_attention_fwd_chunked(dq, dk, dv, o, chunks, scale=scale, lse=lse)
    torch.cuda.synchronize()
    out = to_host(o)
    return (out, lse.cpu().numpy()) if want_lse else out


def _run_ws(q, k, v, dtype, out_dtype, lo=0, hi=None, want_lse=False):
    """usp_attention_fwd_ws with a NaN-poisoned workspace of exactly the size
    the library asks for."""
    import torch
    B, S, h, D = q.shape
    hi = h if hi is None else hi
    nb = usp.usp_attention_workspace_bytes(usp.USP_BF16 if dtype == BF else usp.USP_F32,
                                           B, S, hi - lo, D)
    ws = torch.full((max(nb, 16) // 4,), float("nan"), device=DEV)
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o = poisoned((B, S, h, D), out_dtype)
    lse = torch.full((B, h, S), float("nan"), device=DEV) if want_lse else None
    usp.usp_attention_fwd_ws(dq, dk, dv, o, ws, head_lo=lo, head_hi=hi, lse=lse)
    torch.cuda.synchronize()
    out = to_host(o)
    return (out, lse.cpu().numpy()) if want_lse else out


SMALL = [  # B, S, h, D : several tiles and ragged tails on both kernels' tilings
    (1, 1, 1, 64), (1, 2, 2, 128), (1, 31, 1, 64), (2, 65, 3, 128), (1, 257, 2, 64),
    (1, 300, 1, 128), (1, 1000, 2, 128), (2, 513, 2, 64), (1, 777, 3, 64), (1, 129, 1, 128),
]


@pytest.mark.parametrize("B,S,h,D", SMALL)
def test_bf16_small_full_compare(B, S, h, D):
    q, k, v = synth.draw_qkv(B, S, h, D, seed=100 + S + D)
    ref, ref_lse = A.attention(*(widen(x, BF) for x in (q, k, v)), return_lse=True)
    log(f"attention bf16->f32 B={B} S={S} h={h} D={D}")
    out, lse = _run(q, k, v, BF, F, want_lse=True)
    ma, rf = err(out, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)
    assert np.max(np.abs(lse - ref_lse)) <= BF16_LSE_ABS
    log(f"attention bf16->bf16 B={B} S={S} h={h} D={D}")
    ob = widen(_run(q, k, v, BF, BF), BF)
    assert np.all(np.abs(ob - ref) <= np.maximum(BF16_MAX_ABS, bf16_ulp(ref)))


@pytest.mark.parametrize("B,S,h,D", [(1, 1, 1, 32), (1, 70, 2, 64), (2, 257, 2, 128),
                                     (1, 100, 3, 32)])
def test_f32_small_full_compare(B, S, h, D):
    q, k, v = synth.draw_qkv(B, S, h, D, seed=7 + S, dtype=F)
    ref, ref_lse = A.attention(q, k, v, return_lse=True)
    log(f"attention f32 B={B} S={S} h={h} D={D}")
    out, lse = _run(q, k, v, F, F, want_lse=True)
    ma, rf = err(out, ref)
    assert ma <= F32_MAX_ABS and rf <= F32_REL_FROB, (ma, rf)
    assert np.max(np.abs(lse - ref_lse)) <= 1e-5


def test_custom_scale_and_head_range_isolation():
    B, S, h, D = 1, 200, 4, 128
    q, k, v = synth.draw_qkv(B, S, h, D, seed=5)
    ref = A.attention(*(widen(x, BF) for x in (q, k, v)), scale=0.3)
    log("attention head range [1, 3) scale 0.3")
    out = _run(q, k, v, BF, F, lo=1, hi=3, scale=0.3)
    ma, rf = err(out[:, :, 1:3], ref[:, :, 1:3])
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB
    assert np.all(np.isnan(out[:, :, 0])) and np.all(np.isnan(out[:, :, 3]))


def test_peaky_softmax_small():
    # 1% of K rows x8: large logits, near one-hot rows
    q, k, v = synth.draw_qkv(1, 2000, 2, 64, seed=9, peaky_frac=0.01)
    ref = A.attention(*(widen(x, BF) for x in (q, k, v)))
    log("attention peaky S=2000")
    ma, rf = err(_run(q, k, v, BF, F), ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


@pytest.mark.parametrize("h,chunks", [(8, 3), (5, 2), (3, 3), (4, 1)])
def test_chunked_bitwise_equals_single_shot_small(h, chunks):
    """Chunked passes equal the single-shot call and the per-range calls,
    bit for bit, and the oracle to the attention tolerance."""
    q, k, v = synth.draw_qkv(1, 333, h, 128, seed=h)
    log(f"attention chunked h={h} chunks={chunks}")
    one = _run(q, k, v, BF, F)
    many = _run(q, k, v, BF, F, chunks=chunks)
    assert one.tobytes() == many.tobytes()
    log(f"attention chunked with workspace h={h} chunks={chunks}")
    assert one.tobytes() == _run(q, k, v, BF, F, chunks=chunks, chunk_ws=True).tobytes()
    cb = usp.usp_head_chunk_ranges(h, chunks)
    by_range = np.concatenate([_run(q, k, v, BF, F, lo=cb[j], hi=cb[j + 1])[:, :, cb[j]:cb[j + 1]]
                               for j in range(chunks)], axis=2)
    assert one.tobytes() == by_range.tobytes()
    ref = A.attention(*(widen(x, BF) for x in (q, k, v)))
    ma, rf = err(one, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


# The key walk's branches. Keys are walked in tiles of BN (64 at D = 128,
# 128 at D = 64), nkt = ceil(S / BN) tiles, split once into halves of
# floor(nkt / 2) and the rest (the second holds the partial last tile); a
# half walks pairs of unguarded steps while every load lies before its last
# tile, then guarded steps, then a single step when its length is even, then
# the masked last tile. Query rows run in tiles of 256 (the last one partial).
EDGE_CASES = [  # B, S, h, D, what the case exercises
    (3, 64, 7, 128, "nkt = 1: the first half is empty, the second one whole tile"),
    (2, 37, 3, 64, "short walk at D = 64: one partial 64-key tile (37 keys), one 128-row "
                   "workgroup with rows and one without"),
    (1, 100, 5, 128, "nkt = 2: one tile per half, the second partial"),
    (1, 257, 6, 128, "nkt = 5 (odd): halves of 2 and 3 tiles, one key past a whole tile"),
    (1, 513, 4, 64, "short walk at D = 64: 9 tiles of 64 keys, the last of 1 key; the sixth "
                    "128-row workgroup of each head holds 1 row"),
    (1, 896, 2, 64, "D = 64 at the short-walk limit: 14 tiles of 64 keys (7 of 128), "
                    "unguarded pairs of steps"),
    (1, 897, 2, 64, "D = 64 just past it: 8 tiles of 128 keys split into halves of 4, "
                    "a 1-key last tile"),
    (1, 1000, 2, 128, "nkt = 16: halves of 8 with unguarded pairs, guarded pairs and a single step"),
    (1, 4157, 3, 128, "nkt = 65: halves of 32 and 33, long unguarded runs, a 61-key last tile"),
]


@pytest.mark.parametrize("B,S,h,D,plan", EDGE_CASES)
def test_key_walk_edge_cases(B, S, h, D, plan):
    q, k, v = synth.draw_qkv(B, S, h, D, seed=11 + S + h)
    qf, kf, vf = (widen(x, BF) for x in (q, k, v))
    ref, ref_lse = A.attention(qf, kf, vf, return_lse=True)
    log(f"attention edge case B={B} S={S} h={h} D={D}: {plan}")
    out, lse = _run(q, k, v, BF, F, want_lse=True)
    with no_pool():  # the key-group kernel where the keys split: the same bits
        out_kg, lse_kg = _run(q, k, v, BF, F, want_lse=True)
    assert out.tobytes() == out_kg.tobytes() and lse.tobytes() == lse_kg.tobytes()
    ma, rf = err(out, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)
    assert np.max(np.abs(lse - ref_lse)) <= BF16_LSE_ABS
    ob = widen(_run(q, k, v, BF, BF), BF)
    assert np.all(np.abs(ob - ref) <= np.maximum(BF16_MAX_ABS, bf16_ulp(ref)))


@pytest.mark.parametrize("D", [128, 64])
def test_rows_bitwise_independent_of_launch(D):
    """A row's arithmetic depends on S, D and its own head only: 40 heads in
    one launch (160 query tiles, 320 key-half workgroups) and four launches
    of 10 heads (80 workgroups each, a different spread over the CUs and XCDs)
    give the same bits."""
    q, k, v = synth.draw_qkv(1, 1000, 40, D, seed=31)
    log(f"attention D={D}: 40 heads in one launch vs four launches of 10 heads")
    one = _run(q, k, v, BF, F)
    parts = np.concatenate([_run(q, k, v, BF, F, lo=lo, hi=lo + 10)[:, :, lo:lo + 10]
                            for lo in range(0, 40, 10)], axis=2)
    assert one.tobytes() == parts.tobytes()
    with no_pool():  # the key-group kernel: the same bits in either spread
        parts = np.concatenate([_run(q, k, v, BF, F, lo=lo, hi=lo + 10)[:, :, lo:lo + 10]
                                for lo in range(0, 40, 10)], axis=2)
        assert one.tobytes() == parts.tobytes() == _run(q, k, v, BF, F).tobytes()
    sub = slice(0, 40, 13)
    ref = A.attention(*(widen(x[:, :, sub], BF) for x in (q, k, v)))
    ma, rf = err(one[:, :, sub], ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


EXACT_CASES = [  # B, S, h, D: lengths that are whole key tiles and whole 256-row tiles
    (1, 256, 2, 128), (1, 512, 1, 64), (2, 4096, 1, 128), (1, 8192, 1, 64), (1, 320, 2, 128),
    (1, 128, 3, 64),
]


@pytest.mark.parametrize("B,S,h,D", EXACT_CASES)
def test_exact_tile_multiples(B, S, h, D):
    """No partial key tile and no partial query tile (the masked last tile is
    never taken; even and odd key-tile counts split into equal or unequal
    halves): both kernels against the oracle, and bitwise against each other."""
    q, k, v = synth.draw_qkv(B, S, h, D, seed=61 + S + D)
    ref, ref_lse = A.attention(*(widen(x, BF) for x in (q, k, v)), return_lse=True)
    log(f"attention exact tiles B={B} S={S} h={h} D={D}")
    out, lse = _run(q, k, v, BF, F, want_lse=True)
    ma, rf = err(out, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)
    assert np.max(np.abs(lse - ref_lse)) <= BF16_LSE_ABS
    out_ws, lse_ws = _run_ws(q, k, v, BF, F, want_lse=True)
    assert out.tobytes() == out_ws.tobytes() and lse.tobytes() == lse_ws.tobytes()
    with no_pool():
        out_kg, lse_kg = _run(q, k, v, BF, F, want_lse=True)
    assert out.tobytes() == out_kg.tobytes() and lse.tobytes() == lse_kg.tobytes()


WS_CASES = [  # B, S, h, D: one key tile (empty first half), odd key-tile counts, both D
    (1, 1, 1, 64), (1, 64, 3, 128), (1, 257, 5, 128), (2, 513, 2, 64), (1, 1000, 2, 128),
    (1, 130, 4, 64), (3, 300, 2, 128),
]


@pytest.mark.parametrize("B,S,h,D", WS_CASES)
def test_workspace_path_bitwise_equals_default(B, S, h, D):
    q, k, v = synth.draw_qkv(B, S, h, D, seed=41 + S)
    log(f"attention with workspace B={B} S={S} h={h} D={D}")
    for out_dtype in (F, BF):
        a, la = _run(q, k, v, BF, out_dtype, want_lse=True)
        b, lb = _run_ws(q, k, v, BF, out_dtype, want_lse=True)
        with no_pool():  # the key-group kernel, where the keys split
            c, lc = _run(q, k, v, BF, out_dtype, want_lse=True)
        assert a.tobytes() == b.tobytes() == c.tobytes()
        assert la.tobytes() == lb.tobytes() == lc.tobytes()
    if h > 1:
        a = _run(q, k, v, BF, F, lo=1, hi=h)
        b = _run_ws(q, k, v, BF, F, lo=1, hi=h)
        with no_pool():
            c = _run(q, k, v, BF, F, lo=1, hi=h)
        assert a.tobytes() == b.tobytes() == c.tobytes()
        assert np.all(np.isnan(b[:, :, 0]))
    ref = A.attention(*(widen(x, BF) for x in (q, k, v)))
    ma, rf = err(_run_ws(q, k, v, BF, F), ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


def test_workspace_path_fp32_inputs():
    q, k, v = synth.draw_qkv(1, 100, 2, 64, seed=3, dtype=F)
    log("attention with workspace, fp32 inputs (no workspace used)")
    assert _run_ws(q, k, v, F, F).tobytes() == _run(q, k, v, F, F).tobytes()


def _run_gqa(q, k, v, dtype, out_dtype, lo=0, hi=None, want_lse=False, use_ws=False):
    import torch
    B, S, h, D = q.shape
    hi = h if hi is None else hi
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o = poisoned((B, S, h, D), out_dtype)
    lse = torch.full((B, h, S), float("nan"), device=DEV) if want_lse else None
    ws = None
    if use_ws:
        nb = usp.usp_attention_workspace_bytes(usp.USP_BF16 if dtype == BF else usp.USP_F32,
                                               B, S, hi - lo, D)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), device=DEV)
    usp.usp_attention_fwd_gqa(dq, dk, dv, o, head_lo=lo, head_hi=hi, lse=lse, ws=ws)
    torch.cuda.synchronize()
    out = to_host(o)
    return (out, lse.cpu().numpy()) if want_lse else out


GQA_CASES = [  # B, S, h, hkv, D
    (1, 300, 4, 2, 128), (2, 257, 6, 1, 64), (1, 1000, 8, 4, 128), (1, 65, 5, 5, 64),
    (3, 130, 4, 1, 128),
]


@pytest.mark.parametrize("B,S,h,hkv,D", GQA_CASES)
def test_gqa_parity_and_bitwise_forms(B, S, h, hkv, D):
    q, k, v = synth.draw_qkv(B, S, h, D, seed=51 + S, hkv=hkv)
    ref, ref_lse = A.attention(*(widen(x, BF) for x in (q, k, v)), return_lse=True)
    log(f"attention gqa B={B} S={S} h={h} hkv={hkv} D={D}")
    out, lse = _run_gqa(q, k, v, BF, F, want_lse=True)
    ma, rf = err(out, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)
    assert np.max(np.abs(lse - ref_lse)) <= BF16_LSE_ABS
    # the workspace form, the key-group kernel, and query-head ranges cutting
    # through a group
    assert _run_gqa(q, k, v, BF, F, use_ws=True).tobytes() == out.tobytes()
    with no_pool():
        assert _run_gqa(q, k, v, BF, F).tobytes() == out.tobytes()
    cut = max(1, h // 2 + (1 if h > 2 else 0))
    parts = np.concatenate([_run_gqa(q, k, v, BF, F, lo=0, hi=cut)[:, :, :cut],
                            _run_gqa(q, k, v, BF, F, lo=cut, hi=h)[:, :, cut:]], axis=2)
    if cut < h:
        assert parts.tobytes() == out.tobytes()
    if hkv == h:
        assert _run(q, k, v, BF, F).tobytes() == out.tobytes()


def test_gqa_fp32_parity():
    q, k, v = synth.draw_qkv(1, 200, 6, 64, seed=57, dtype=F, hkv=2)
    ref = A.attention(q, k, v)
    log("attention gqa fp32 S=200 h=6 hkv=2")
    ma, rf = err(_run_gqa(q, k, v, F, F), ref)
    assert ma <= F32_MAX_ABS and rf <= F32_REL_FROB, (ma, rf)


def test_gqa_small_workload_full():
    """pack q (16 heads) and k, v (4 heads) into 4 head groups -> attention
    per group -> unpack, against the oracle's Ulysses composition."""
    import torch
    from oracle import ulysses as U
    w = synth.WORKLOADS["gqa_small"]
    q, k, v = synth.draw_workload(w)
    B, S, H, Hkv, D, P = w.B, w.S, w.H, w.kv_heads, w.D, w.P
    hq, hk = R.balanced_ranges(H, P), R.balanced_ranges(Hkv, P)
    log("workload gqa_small: pack -> attention x4 -> unpack")
    blocks = []
    for x, hb_ in ((q, hq), (k, hk), (v, hk)):
        bl = [poisoned((B, S, hb_[j + 1] - hb_[j], D), BF) for j in range(P)]
        usp.usp_pack_seq_to_heads(to_dev(x, BF), bl)
        blocks.append(bl)
    ob = [poisoned((B, S, hq[j + 1] - hq[j], D), F) for j in range(P)]
    for j in range(P):
        usp.usp_attention_fwd_gqa(blocks[0][j], blocks[1][j], blocks[2][j], ob[j])
    out = poisoned((B, S, H, D), F)
    usp.usp_unpack_heads_to_seq(ob, out)
    torch.cuda.synchronize()
    ref = U.ulysses_world(*(widen(x, BF) for x in (q, k, v)), P)
    ma, rf = err(to_host(out), ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


def _ulysses_gpu(w: synth.Workload, q, k, v, out_dtype):
    """pack (world) -> attention per head-group block -> unpack, on the GPU."""
    import torch
    B, S, H, D, P = w.B, w.S, w.H, w.D, w.P
    hb = R.balanced_ranges(H, P)
    blocks = []
    for x in (q, k, v):
        bl = [poisoned((B, S, hb[j + 1] - hb[j], D), w.dtype) for j in range(P)]
        usp.usp_pack_seq_to_heads(to_dev(x, w.dtype), bl)
        blocks.append(bl)
    ob = [poisoned((B, S, hb[j + 1] - hb[j], D), out_dtype) for j in range(P)]
    for j in range(P):
        usp.usp_attention_fwd(blocks[0][j], blocks[1][j], blocks[2][j], ob[j])
    out = poisoned((B, S, H, D), out_dtype)
    usp.usp_unpack_heads_to_seq(ob, out)
    torch.cuda.synchronize()
    return to_host(out)


def test_tiny_fp32_workload_full():
    w = synth.WORKLOADS["tiny_fp32"]
    q, k, v = synth.draw_workload(w)
    ref = A.attention(q, k, v)  # single-device attention over all heads
    log("workload tiny_fp32: pack -> attention x3 -> unpack")
    out = _ulysses_gpu(w, q, k, v, F)
    ma, rf = err(out, ref)
    assert ma <= F32_MAX_ABS and rf <= F32_REL_FROB, (ma, rf)


def test_vit_l16_workload_full():
    w = synth.WORKLOADS["vit_l16"]
    q, k, v = synth.draw_workload(w)
    qf, kf, vf = (widen(x, BF) for x in (q, k, v))
    log("workload vit_l16: pack -> attention x4 -> unpack")
    out = _ulysses_gpu(w, q, k, v, F)
    par = A.attention_parallel(qf, kf, vf)
    ref = np.empty(out.shape)
    for (b, hd), (rows, o, _) in par.items():
        ref[b, rows, hd] = o
    ma, rf = err(out, ref)
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)


def _sample_rows(S, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, S - 2, S - 1], rng.choice(S, n, replace=False)]))


def _risky_rows(qf, kf, b, hd, n):
    """Query rows whose softmax is dominated by few keys: the rows with the
    largest scores against the largest-norm keys (the scaled keys of the
    peaky workload), where bf16 rounding of the weights matters most."""
    K = kf[b, :, hd]
    big = np.argsort(np.einsum("sd,sd->s", K, K))[-max(1, K.shape[0] // 100):]
    sc = qf[b, :, hd] @ K[big].T
    top2 = np.sort(np.partition(sc, -2, axis=1)[:, -2:], axis=1)
    # large top score, and a close runner-up (two comparable dominant weights)
    order1 = np.argsort(top2[:, 1])[-n // 2:]
    order2 = np.argsort(top2[:, 1] - 4.0 * np.abs(top2[:, 1] - top2[:, 0]))[-n // 2:]
    return np.unique(np.concatenate([order1, order2]))


def _check_sampled(out, q, k, v, dtype, B, S, rows_per_head, lse=None, out_bf16=None):
    """Compare ``out`` (the fp32-output epilogue) against the oracle on
    ``rows_per_head[(b, head)]``; ``out_bf16`` (the bf16-output epilogue of
    the same call, bf16 bits) is graded per element on the same rows within
    max(1e-2, one bf16 ulp of the reference)."""
    qf, kf, vf = (widen(x, dtype) for x in (q, k, v))
    par = A.attention_parallel(qf, kf, vf, rows_per_head=rows_per_head,
                               workers=min(16, A.host_cores()))
    got, ref, lg, lr, gb = [], [], [], [], []
    for (b, hd), (rows, o, ls) in par.items():
        got.append(out[b, rows, hd]); ref.append(o)
        if out_bf16 is not None:
            gb.append(widen(out_bf16[b, rows, hd], BF))
        if lse is not None:
            lg.append(lse[b, hd, rows]); lr.append(ls)
    if out_bf16 is not None:
        r = np.concatenate(ref)
        d = np.abs(np.concatenate(gb) - r)
        log(f"sampled bf16-output epilogue: max_abs={d.max():.3e}")
        assert np.all(d <= np.maximum(BF16_MAX_ABS, bf16_ulp(r))), float(d.max())
    ma, rf = err(np.concatenate(got), np.concatenate(ref))
    log(f"sampled parity: {sum(len(r) for r in rows_per_head.values())} rows "
        f"max_abs={ma:.3e} rel_frob={rf:.3e}")
    assert ma <= BF16_MAX_ABS and rf <= BF16_REL_FROB, (ma, rf)
    if lse is not None:
        assert np.max(np.abs(np.concatenate(lg) - np.concatenate(lr))) <= BF16_LSE_ABS
    return ma, rf


def test_video_dit_share_full_size():
    import torch
    w = synth.WORKLOADS["video_dit_share"]
    q, k, v = synth.draw_workload(w)
    hb = R.balanced_ranges(w.H, w.P)
    h0 = hb[1] - hb[0]
    # head-group block 0 (rank 0's share) through the GPU pack, attention there
    blocks = []
    for x in (q, k, v):
        bl = [poisoned((w.B, w.S, hb[j + 1] - hb[j], w.D), BF) for j in range(w.P)]
        log("workload video_dit_share: pack world")
        usp.usp_pack_seq_to_heads(to_dev(x, BF), bl)
        blocks.append(bl[0])
        del bl
    o = poisoned((w.B, w.S, h0, w.D), F)
    lse = torch.empty((w.B, h0, w.S), device=DEV)
    log("workload video_dit_share: attention block 0 (h=5, S=32760)")
    usp.usp_attention_fwd(blocks[0], blocks[1], blocks[2], o, lse=lse)
    torch.cuda.synchronize()
    out = to_host(o)
    assert not np.any(np.isnan(out))
    log("workload video_dit_share: attention block 0 with a workspace")
    ws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, w.B, w.S, h0, w.D) // 4,
                     device=DEV)
    o2 = poisoned((w.B, w.S, h0, w.D), F)
    lse2 = torch.empty((w.B, h0, w.S), device=DEV)
    usp.usp_attention_fwd_ws(blocks[0], blocks[1], blocks[2], o2, ws, lse=lse2)
    torch.cuda.synchronize()
    assert to_host(o2).tobytes() == out.tobytes()
    assert lse2.cpu().numpy().tobytes() == lse.cpu().numpy().tobytes()
    # the benched epilogue (bf16 output, workspace): the fp32 result rounded
    # to nearest even, bit for bit, over the whole output
    log("workload video_dit_share: attention block 0, bf16 output, workspace")
    ob = poisoned((w.B, w.S, h0, w.D), BF)
    usp.usp_attention_fwd_ws(blocks[0], blocks[1], blocks[2], ob, ws)
    torch.cuda.synchronize()
    out_b = to_host(ob)
    assert out_b.tobytes() == synth.f32_to_bf16_bits(out).tobytes()
    del ws, o2, lse2, ob
    sl = slice(hb[0], hb[1])
    rows = {(0, hd): _sample_rows(w.S, 256, 30 + hd) for hd in range(h0)}
    _check_sampled(out, q[:, :, sl], k[:, :, sl], v[:, :, sl], BF, w.B, w.S, rows,
                   lse=lse.cpu().numpy(), out_bf16=out_b)


def test_long_chunked_full_size():
    w = synth.WORKLOADS["long_chunked"]
    q, k, v = synth.draw_workload(w)
    log("workload long_chunked: single shot (S=131072, h=8)")
    one = _run(q, k, v, BF, F)
    log("workload long_chunked: 3 head-chunk passes")
    many = _run(q, k, v, BF, F, chunks=w.chunks)
    assert usp.usp_head_chunk_ranges(w.H, w.chunks) == [0, 3, 6, 8]
    assert one.tobytes() == many.tobytes()
    log("workload long_chunked: 3 head-chunk passes with a workspace")
    assert one.tobytes() == _run(q, k, v, BF, F, chunks=w.chunks, chunk_ws=True).tobytes()
    assert not np.any(np.isnan(one))
    rows = {(0, hd): _sample_rows(w.S, 64, 40 + hd) for hd in range(w.H)}
    _check_sampled(one, q, k, v, BF, w.B, w.S, rows)


def test_indivisible_long_full_size():
    w = synth.WORKLOADS["indivisible_long"]
    q, k, v = synth.draw_workload(w)
    log("workload indivisible_long: pack -> attention x4 -> unpack (S=65537)")
    out = _ulysses_gpu(w, q, k, v, F)
    assert not np.any(np.isnan(out))
    log("workload indivisible_long: the same with bf16 output")
    out_b = _ulysses_gpu(w, q, k, v, BF)
    # the bf16-output epilogue is the fp32 result rounded to nearest even, everywhere
    assert out_b.tobytes() == synth.f32_to_bf16_bits(out).tobytes()
    kf = widen(k, BF)
    qf = widen(q, BF)
    rows = {}
    for b in range(w.B):
        for hd in range(w.H):
            r = _sample_rows(w.S, 48, 50 + 31 * b + hd)
            if hd % 4 == 0:   # the riskiest rows of a third of the heads
                r = np.unique(np.concatenate([r, _risky_rows(qf, kf, b, hd, 400)]))
            rows[(b, hd)] = r
    del kf, qf
    _check_sampled(out, q, k, v, BF, w.B, w.S, rows, out_bf16=out_b)


def test_gqa_video_share_full_size():
    """Rank 0's share of the grouped video-DiT workload: 5 query heads over
    one K/V head at S = 32760, sampled rows against the oracle."""
    import torch
    w = synth.WORKLOADS["gqa_video_share"]
    q, k, v = synth.draw_workload(w)
    hq, hk = R.balanced_ranges(w.H, w.P), R.balanced_ranges(w.kv_heads, w.P)
    qs = q[:, :, hq[0]:hq[1]]
    ks, vs = (x[:, :, hk[0]:hk[1]] for x in (k, v))
    log("workload gqa_video_share: attention on head group 0 (5 query heads, 1 K/V head)")
    out, lse = _run_gqa(qs, ks, vs, BF, F, want_lse=True, use_ws=True)
    assert not np.any(np.isnan(out))
    rows = {(0, hd): _sample_rows(w.S, 200, 60 + hd) for hd in range(hq[1] - hq[0])}
    _check_sampled(out, qs, ks, vs, BF, w.B, w.S, rows, lse=lse)


def test_very_long_sequence_sampled():
    """S = 1048583 (16385 key tiles with a ragged tail, one head, D = 128;
    past the split range, so every entry point walks each row's keys whole):
    the default and workspace entry points agree bit for bit, and sampled
    rows (the ends and rows around 256-row tiles and the middle key tile)
    match the oracle over all keys."""
    B, S, h, D = 1, 1_048_583, 1, 128
    q, k, v = synth.draw_qkv(B, S, h, D, seed=91)
    log(f"attention very long sequence S={S} (default)")
    out, lse = _run(q, k, v, BF, F, want_lse=True)
    log(f"attention very long sequence S={S} (workspace)")
    out_ws, lse_ws = _run_ws(q, k, v, BF, F, want_lse=True)
    assert out.tobytes() == out_ws.tobytes() and lse.tobytes() == lse_ws.tobytes()
    assert not np.any(np.isnan(out))
    half = (S + 63) // 64 // 2 * 64     # first key of the second half
    extra = np.array([255, 256, half - 1, half, half + 1, S - 257, S - 256])
    rows = {(0, 0): np.unique(np.concatenate([_sample_rows(S, 40, 92), extra]))}
    _check_sampled(out, q, k, v, BF, B, S, rows, lse=lse)


@pytest.mark.parametrize("S,h,D,what", [
    (61700, 136, 128, "key halves / key groups, ragged last tile"),
    (262147, 64, 64, "whole walks (4097 key tiles), ragged last tile"),
])
def test_slab_beyond_2gib(S, h, D, what):
    """A (batch, K/V head) slab of S * h * D * 2 >= 2^31 bytes: the K/V
    loads then rebuild their buffer resource at every tile instead of
    offsetting one resource. Only the last head is computed (the other heads
    hold zeros and must stay untouched in the output); the workspace form,
    the default call and the key-group kernel agree bit for bit, and sampled
    rows match the oracle."""
    import torch
    assert S * h * D * 2 >= 2 ** 31 - 1
    hd = h - 1
    q1, k1, v1 = synth.draw_qkv(1, S, 1, D, seed=97)
    dev = {}
    for name, x in (("q", q1), ("k", k1), ("v", v1)):
        t = torch.zeros((1, S, h, D), dtype=torch.bfloat16, device=DEV)
        t[:, :, hd:hd + 1] = to_dev(x, BF)
        dev[name] = t
    outs = []
    for form in ("workspace", "default", "no pool"):
        log(f"attention slab beyond 2 GiB ({what}): S={S} h={h} D={D} head {hd} {form}")
        o = poisoned((1, S, h, D), F)
        lse = torch.full((1, h, S), float("nan"), device=DEV)
        if form == "workspace":
            nb = usp.usp_attention_workspace_bytes(usp.USP_BF16, 1, S, 1, D)
            ws = torch.full((nb // 4,), float("nan"), device=DEV)
            usp.usp_attention_fwd_ws(dev["q"], dev["k"], dev["v"], o, ws, head_lo=hd, head_hi=h, lse=lse)
            del ws
        elif form == "default":
            usp.usp_attention_fwd(dev["q"], dev["k"], dev["v"], o, head_lo=hd, head_hi=h, lse=lse)
        else:
            with no_pool():  # the key-group kernel where the keys split
                usp.usp_attention_fwd(dev["q"], dev["k"], dev["v"], o, head_lo=hd, head_hi=h, lse=lse)
        torch.cuda.synchronize()
        assert bool(torch.isnan(o[:, :, :hd]).all()) and bool(torch.isnan(lse[:, :hd]).all())
        outs.append((to_host(o[:, :, hd:h]), lse[:, hd:h].cpu().numpy()))
        del o, lse
    (out, lse) = outs[0]
    for out2, lse2 in outs[1:]:
        assert out.tobytes() == out2.tobytes() and lse.tobytes() == lse2.tobytes()
    assert not np.any(np.isnan(out))
    rows = {(0, 0): np.unique(np.concatenate([_sample_rows(S, 24, 98), [0, S - 1]]))}
    _check_sampled(out, q1, k1, v1, BF, 1, S, rows, lse=lse)


def test_default_call_on_two_streams():
    """The workspace pool under concurrent use: two streams, each running the
    default call (keys split in halves, so each call takes a workspace from
    the pool) on its own inputs several times over, interleaved; every output
    equals the same call run alone, bit for bit."""
    import torch
    B, S, h, D = 1, 3000, 6, 128
    ins = [[to_dev(x, BF) for x in synth.draw_qkv(B, S, h, D, seed=71 + i)] for i in range(2)]
    ref = []
    for q, k, v in ins:
        o = torch.empty((B, S, h, D), dtype=torch.float32, device=DEV)
        usp.usp_attention_fwd(q, k, v, o)
        torch.cuda.synchronize()
        ref.append(o.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full((B, S, h, D), float("nan"), device=DEV) for _ in range(4)] for _ in range(2)]
    torch.cuda.synchronize()
    log("default attention on two streams at once")
    for r in range(4):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                q, k, v = ins[i]
                usp.usp_attention_fwd(q, k, v, outs[i][r], stream=st)
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(4):
            assert torch.equal(outs[i][r].view(torch.int32), ref[i].view(torch.int32)), (i, r)
