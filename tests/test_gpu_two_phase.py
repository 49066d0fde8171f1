"""GPU parity of the head-chunked (two-phase) exchange: the per-chunk pack
and unpack against the oracle bit for bit, and the two-phase step (per
chunk: pack -> attention on the chunk's heads -> unpack) against the
single-shot step bit for bit.

Inputs of the relayouts are index-coded and the outputs start poisoned, and
the oracle starts from a copy of the same poisoned bytes, so a phase that
writes outside its heads or rows fails the byte compare."""
import numpy as np
import pytest

import ulysses_sequence_attention_amd as usp
from oracle import ranges as R
from oracle import relayout as X
from oracle import ulysses as U
from ulysses_sequence_attention_amd import synth

from gpu_util import coded, BF16_MAX_ABS, BF16_REL_FROB, DEV, err, log, poisoned, to_dev, to_host, widen

pytestmark = pytest.mark.gpu

BF, F = synth.BF16, synth.F32

CHUNK_CASES = [  # B, S, H, D, P, chunks, dtype (equal head groups of h = H / P)
    (1, 257, 6, 64, 3, 2, F),       # tiny workload's shape, h = 2: 1/1
    (32, 577, 16, 64, 4, 2, BF),    # ViT-L/16, h = 4: 2/2
    (2, 37, 15, 64, 3, 3, BF),      # h = 5: 2/2/1, ragged tokens
    (1, 100, 16, 128, 2, 3, F),     # h = 8: 3/3/2
    (1, 64, 64, 8, 64, 1, BF),      # P = 64, one 16-byte head per group
    (3, 11, 5, 16, 1, 2, BF),       # P = 1, h = 5: 3/2
]


def _plan(h, chunks):
    b = R.head_chunk_ranges(h, chunks)
    return [(b[c], b[c + 1]) for c in range(chunks)]


@pytest.mark.parametrize("B,S,H,D,P,chunks,dtype", CHUNK_CASES)
def test_chunk_phases_world(B, S, H, D, P, chunks, dtype):
    import torch
    h = H // P
    seq = coded((B, S, H, D), dtype)
    d_seq = to_dev(seq, dtype)
    blocks = [poisoned((B, S, h, D), dtype) for _ in range(P)]
    ref = [to_host(b) for b in blocks]
    for lo, hi in _plan(h, chunks):
        log(f"pack chunk [{lo},{hi}) world B={B} S={S} H={H} D={D} P={P} {dtype}")
        usp.usp_pack_seq_to_heads_chunk(d_seq, blocks, lo, hi)
        torch.cuda.synchronize()
        X.pack_heads_chunk(seq, ref, S, lo, hi)
        for j in range(P):
            assert to_host(blocks[j]).tobytes() == ref[j].tobytes(), f"block {j} after [{lo},{hi})"
    # over the plan: the whole-group pack
    for j in range(P):
        assert ref[j].tobytes() == X.pack_seq_to_heads(seq, P)[j].tobytes()
    out = poisoned((B, S, H, D), dtype)
    ref_out = to_host(out)
    for lo, hi in _plan(h, chunks):
        log(f"unpack chunk [{lo},{hi}) world")
        usp.usp_unpack_heads_to_seq_chunk(blocks, out, lo, hi)
        torch.cuda.synchronize()
        X.unpack_heads_chunk(ref, ref_out, S, lo, hi)
        assert to_host(out).tobytes() == ref_out.tobytes(), f"after [{lo},{hi})"
    assert ref_out.tobytes() == seq.tobytes()


@pytest.mark.parametrize("B,S,H,D,P,chunks,dtype", [(1, 257, 6, 64, 3, 2, F),
                                                    (2, 37, 15, 64, 3, 3, BF),
                                                    (2, 65537, 12, 64, 4, 2, BF),
                                                    (1, 9, 9, 8, 9, 1, BF)])
def test_chunk_phases_rank_share(B, S, H, D, P, chunks, dtype):
    import torch
    h = H // P
    seq = coded((B, S, H, D), dtype)
    tb = R.balanced_ranges(S, P)
    world = X.pack_seq_to_heads(seq, P)
    d_world = [to_dev(w, dtype) for w in world]
    for r in range(P):
        shard = np.ascontiguousarray(seq[:, tb[r]:tb[r + 1]])
        d_shard = to_dev(shard, dtype)
        blocks = [poisoned((B, S, h, D), dtype) for _ in range(P)]
        ref = [to_host(b) for b in blocks]
        out = poisoned(shard.shape, dtype)
        ref_out = to_host(out)
        for lo, hi in _plan(h, chunks):
            log(f"pack chunk [{lo},{hi}) rank {r} B={B} S={S} H={H} D={D} P={P} {dtype}")
            usp.usp_pack_seq_to_heads_chunk(d_shard, blocks, lo, hi, rank=r)
            log(f"unpack chunk [{lo},{hi}) rank {r}")
            usp.usp_unpack_heads_to_seq_chunk(d_world, out, lo, hi, rank=r)
            torch.cuda.synchronize()
            X.pack_heads_chunk(shard, ref, S, lo, hi, rank=r)
            X.unpack_heads_chunk(world, ref_out, S, lo, hi, rank=r)
            for j in range(P):
                assert to_host(blocks[j]).tobytes() == ref[j].tobytes(), f"rank {r} block {j}"
            assert to_host(out).tobytes() == ref_out.tobytes(), f"rank {r} shard"
        assert ref_out.tobytes() == shard.tobytes()


def test_chunk_phases_beyond_one_launch():
    """A phase moving 2^31 + 12.8M chunks (S = 22500000, H = 8, D = 128, bf16,
    P = 2, heads [1, 4) of each group of 4: 46 GB tensors), more than one
    launch's 32-bit flat index, so the row walk is split in two launches
    (boundary after row 22369621). Device-side compare against the
    definition: the chunk's heads moved, head 0 of every group untouched."""
    import torch
    B, S, H, D, P, lo, hi = 1, 22_500_000, 8, 128, 2, 1, 4
    h = H // P
    torch.manual_seed(6)
    bits = torch.randint(-32768, 32768, (B, S, H, D), dtype=torch.int16, device=DEV)
    blocks = [torch.full((B, S, h, D), 7, dtype=torch.int16, device=DEV) for _ in range(P)]
    log(f"pack chunk [{lo},{hi}) beyond one launch S={S} H={H} D={D} P={P} (46 GB)")
    usp.usp_pack_seq_to_heads_chunk(bits.view(torch.bfloat16), [b.view(torch.bfloat16) for b in blocks],
                                    lo, hi)
    torch.cuda.synchronize()
    for j in range(P):
        assert torch.equal(blocks[j][:, :, lo:hi], bits[:, :, j * h + lo:j * h + hi]), f"block {j}"
        assert bool((blocks[j][:, :, :lo] == 7).all()), f"block {j} head 0 written"
    back = torch.full((B, S, H, D), 9, dtype=torch.int16, device=DEV)
    log("unpack chunk beyond one launch")
    usp.usp_unpack_heads_to_seq_chunk([b.view(torch.bfloat16) for b in blocks],
                                      back.view(torch.bfloat16), lo, hi)
    torch.cuda.synchronize()
    for j in range(P):
        assert torch.equal(back[:, :, j * h + lo:j * h + hi], bits[:, :, j * h + lo:j * h + hi])
        assert bool((back[:, :, j * h:j * h + lo] == 9).all())
    del bits, blocks, back
    torch.cuda.empty_cache()


def _attend(qb, kb, vb, ob, lo, hi):
    """usp_attention_fwd_ws on heads [lo, hi) of every block."""
    import torch
    B, S, h, D = qb[0].shape
    nb = usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, hi - lo, D)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    for j in range(len(qb)):
        usp.usp_attention_fwd_ws(qb[j], kb[j], vb[j], ob[j], ws, head_lo=lo, head_hi=hi)


def _steps(q, k, v, P, chunks, S, rank=-1, world=None):
    """Single-shot and two-phase steps of one rank (rank >= 0: q, k, v are
    its shards and ``world`` the blocks of every rank, which it overwrites
    with its rows) or of the world. Returns both outputs (bf16)."""
    import torch
    B, L, H, D = q.shape
    h = H // P

    def fresh():
        if world is None:
            return [[torch.empty((B, S, h, D), dtype=torch.bfloat16, device=DEV) for _ in range(P)]
                    for _ in range(3)]
        return [[w.clone() for w in t] for t in world]

    # single shot: whole-group pack, attention on all heads, whole-group unpack
    qb, kb, vb = fresh()
    ob = [torch.empty((B, S, h, D), dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    for x, xb in ((q, qb), (k, kb), (v, vb)):
        usp.usp_pack_seq_to_heads(x, xb, rank=rank)
    _attend(qb, kb, vb, ob, 0, h)
    one = torch.empty((B, L, H, D), dtype=torch.bfloat16, device=DEV)
    usp.usp_unpack_heads_to_seq(ob, one, rank=rank)
    # two phases per chunk: pack the chunk's heads, attend them, unpack them
    qb, kb, vb = fresh()
    ob = [torch.empty((B, S, h, D), dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    two = torch.empty((B, L, H, D), dtype=torch.bfloat16, device=DEV)
    for lo, hi in _plan(h, chunks):
        for x, xb in ((q, qb), (k, kb), (v, vb)):
            usp.usp_pack_seq_to_heads_chunk(x, xb, lo, hi, rank=rank)
        _attend(qb, kb, vb, ob, lo, hi)
        usp.usp_unpack_heads_to_seq_chunk(ob, two, lo, hi, rank=rank)
    torch.cuda.synchronize()
    return one, two


@pytest.mark.parametrize("B,S,H,D,P,chunks", [(2, 300, 15, 64, 3, 3), (1, 1000, 16, 128, 2, 3),
                                              (3, 77, 8, 64, 1, 2)])
def test_two_phase_world_equals_single_shot(B, S, H, D, P, chunks):
    q, k, v = synth.draw_qkv(B, S, H, D, 40 + P)
    log(f"two-phase world B={B} S={S} H={H} D={D} P={P} chunks={chunks}")
    one, two = _steps(*(to_dev(x, BF) for x in (q, k, v)), P, chunks, S)
    assert to_host(two).tobytes() == to_host(one).tobytes()
    ref = U.ulysses_two_phase_world(*(widen(x, BF) for x in (q, k, v)), P, chunks)
    max_abs, rel = err(widen(to_host(two), BF), ref)
    assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_FROB, (max_abs, rel)


def test_two_phase_rank_share_equals_single_shot():
    import torch
    B, S, H, D, P, chunks = 2, 517, 12, 64, 4, 2
    q, k, v = synth.draw_qkv(B, S, H, D, 44)
    tb = R.balanced_ranges(S, P)
    world = [[to_dev(b, BF) for b in X.pack_seq_to_heads(x, P)] for x in (q, k, v)]
    for r in range(P):
        shards = [to_dev(np.ascontiguousarray(x[:, tb[r]:tb[r + 1]]), BF) for x in (q, k, v)]
        log(f"two-phase rank {r} B={B} S={S} H={H} D={D} P={P} chunks={chunks}")
        one, two = _steps(*shards, P, chunks, S, rank=r, world=world)
        assert torch.equal(one.view(torch.int16), two.view(torch.int16)), f"rank {r}"


def test_two_phase_video_dit_world():
    """The video-DiT world (S = 32760, H = 40, D = 128, P = 8: groups of 5
    heads) in chunks 2/2/1 equals the single-shot world bit for bit."""
    import torch
    w = synth.WORKLOADS["video_dit_share"]
    q, k, v = synth.draw_workload(w)
    log("two-phase video-DiT world, chunks 2/2/1")
    one, two = _steps(*(to_dev(x, BF) for x in (q, k, v)), w.P, 3, w.S)
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


@pytest.mark.parametrize("B,S,H,Hkv,D,P,chunks", [(2, 300, 20, 10, 64, 2, 3), (1, 4096, 32, 8, 128, 4, 2)])
def test_two_phase_grouped_heads_equals_single_shot(B, S, H, Hkv, D, P, chunks):
    """Grouped K/V heads: the plan runs over each group's K/V heads and a
    chunk [lo, hi) carries query heads [lo G, hi G); per chunk, pack those
    query heads of q and K/V heads of k and v, usp_attention_fwd_gqa on the
    chunk's query heads, unpack them. Bitwise equal to the single-shot
    grouped step, and the oracle's two-phase result within tolerance."""
    import torch
    G, h, hkv = H // Hkv, H // P, Hkv // P
    q, k, v = synth.draw_qkv(B, S, H, D, 50 + P, hkv=Hkv)
    dq, dk, dv = (to_dev(x, BF) for x in (q, k, v))

    def blocks(heads):
        return [torch.empty((B, S, heads, D), dtype=torch.bfloat16, device=DEV) for _ in range(P)]

    def attend(qb, kb, vb, ob, lo, hi):
        nb = usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, hi - lo, D)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        for j in range(P):
            usp.usp_attention_fwd_gqa(qb[j], kb[j], vb[j], ob[j], head_lo=lo, head_hi=hi, ws=ws)

    log(f"two-phase grouped B={B} S={S} H={H} Hkv={Hkv} D={D} P={P} chunks={chunks}")
    qb, kb, vb, ob = blocks(h), blocks(hkv), blocks(hkv), blocks(h)
    usp.usp_pack_seq_to_heads(dq, qb)
    usp.usp_pack_seq_to_heads(dk, kb)
    usp.usp_pack_seq_to_heads(dv, vb)
    attend(qb, kb, vb, ob, 0, h)
    one = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV)
    usp.usp_unpack_heads_to_seq(ob, one)
    qb, kb, vb, ob = blocks(h), blocks(hkv), blocks(hkv), blocks(h)
    two = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV)
    for lo, hi in _plan(hkv, chunks):
        usp.usp_pack_seq_to_heads_chunk(dq, qb, lo * G, hi * G)
        usp.usp_pack_seq_to_heads_chunk(dk, kb, lo, hi)
        usp.usp_pack_seq_to_heads_chunk(dv, vb, lo, hi)
        attend(qb, kb, vb, ob, lo * G, hi * G)
        usp.usp_unpack_heads_to_seq_chunk(ob, two, lo * G, hi * G)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    if S <= 512:
        ref = U.ulysses_two_phase_world(*(widen(x, BF) for x in (q, k, v)), P, chunks)
        max_abs, rel = err(widen(to_host(two), BF), ref)
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_FROB, (max_abs, rel)
