"""GPU parity of ranges and relayouts against the oracle: bit-exact.

Inputs are index-coded (each element holds its own flat index) and outputs
start poisoned (NaN patterns), so a missed, doubled or misplaced element
fails the byte compare."""
import numpy as np
import pytest

import ulysses_sequence_attention_amd as usp
from oracle import ranges as R
from oracle import relayout as X
from ulysses_sequence_attention_amd import synth

from gpu_util import coded, DEV, log, poisoned, to_dev, to_host

pytestmark = pytest.mark.gpu

BF, F = synth.BF16, synth.F32

WORLD_CASES = [  # B, S, H, D, P, dtype
    (1, 257, 6, 64, 3, F),       # tiny fp32 workload
    (32, 577, 16, 64, 4, BF),    # ViT-L/16 workload
    (2, 37, 7, 64, 3, BF),       # ragged heads 3/2/2, ragged tokens
    (1, 100, 10, 128, 4, F),     # ragged heads 3/3/2/2
    (1, 64, 64, 8, 64, BF),      # P at its maximum, 16-byte heads
    (3, 11, 5, 16, 1, BF),       # P = 1
    (2, 9, 9, 4, 9, F),          # one head and one token per rank
]


def test_device_ranges():
    import torch
    for total, parts in [(257, 3), (577, 4), (32760, 8), (65537, 4), (12, 4), (40, 8), (1, 1),
                         (2**40 + 7, 64), (1000, 999)]:
        log(f"usp_balanced_ranges_device total={total} parts={parts}")
        out = torch.full((parts + 1,), -1, dtype=torch.int64, device=DEV)
        usp.usp_balanced_ranges_device(total, parts, out)
        torch.cuda.synchronize()
        assert out.cpu().tolist() == R.balanced_ranges(total, parts)


def _world_roundtrip(B, S, H, D, P, dtype):
    import torch
    seq = coded((B, S, H, D), dtype)
    ref_blocks = X.pack_seq_to_heads(seq, P)
    hb = R.balanced_ranges(H, P)
    d_seq = to_dev(seq, dtype)
    blocks = [poisoned((B, S, hb[j + 1] - hb[j], D), dtype) for j in range(P)]
    log(f"pack world B={B} S={S} H={H} D={D} P={P} {dtype}")
    usp.usp_pack_seq_to_heads(d_seq, blocks)
    torch.cuda.synchronize()
    for j in range(P):
        assert to_host(blocks[j]).tobytes() == ref_blocks[j].tobytes(), f"block {j}"
    back = poisoned((B, S, H, D), dtype)
    log(f"unpack world B={B} S={S} H={H} D={D} P={P} {dtype}")
    usp.usp_unpack_heads_to_seq(blocks, back)
    torch.cuda.synchronize()
    assert to_host(back).tobytes() == seq.tobytes()


@pytest.mark.parametrize("B,S,H,D,P,dtype", WORLD_CASES)
def test_world_pack_unpack(B, S, H, D, P, dtype):
    _world_roundtrip(B, S, H, D, P, dtype)


def test_world_pack_unpack_indivisible_long():
    _world_roundtrip(2, 65537, 12, 64, 4, BF)


def test_world_pack_unpack_video_dit():
    _world_roundtrip(1, 32760, 40, 128, 8, BF)


@pytest.mark.parametrize("B,S,H,D,P,dtype", [(1, 257, 6, 64, 3, F), (2, 37, 7, 64, 3, BF),
                                             (2, 65537, 12, 64, 4, BF), (1, 9, 9, 8, 9, BF)])
def test_rank_share_pack_unpack(B, S, H, D, P, dtype):
    import torch
    seq = coded((B, S, H, D), dtype)
    world = X.pack_seq_to_heads(seq, P)
    hb = R.balanced_ranges(H, P)
    tb = R.balanced_ranges(S, P)
    for r in range(P):
        shard = X.scatter_sequence(seq, P, r)
        blocks = [poisoned((B, S, hb[j + 1] - hb[j], D), dtype) for j in range(P)]
        log(f"pack rank {r} B={B} S={S} H={H} D={D} P={P} {dtype}")
        usp.usp_pack_seq_to_heads(to_dev(shard, dtype), blocks, rank=r)
        torch.cuda.synchronize()
        for j in range(P):
            got = to_host(blocks[j])
            # rank r's rows equal the world pack, every other row is untouched
            assert got[:, tb[r]:tb[r + 1]].tobytes() == world[j][:, tb[r]:tb[r + 1]].tobytes()
            poison = to_host(poisoned((1,), dtype)).tobytes()
            rest = np.concatenate([got[:, :tb[r]], got[:, tb[r + 1]:]], axis=1)
            assert rest.tobytes() == poison * rest.size
        d_world = [to_dev(w, dtype) for w in world]
        out = poisoned(shard.shape, dtype)
        log(f"unpack rank {r}")
        usp.usp_unpack_heads_to_seq(d_world, out, rank=r)
        torch.cuda.synchronize()
        assert to_host(out).tobytes() == X.unpack_rank_share(world, H, r).tobytes()


def test_p1_is_byte_identical():
    import torch
    x = synth.draw_qkv(2, 33, 3, 64, 11)[0]
    blk = poisoned((2, 33, 3, 64), BF)
    log("pack P=1")
    usp.usp_pack_seq_to_heads(to_dev(x, BF), [blk])
    torch.cuda.synchronize()
    assert to_host(blk).tobytes() == x.tobytes()


def test_world_pack_unpack_beyond_one_launch():
    """A 34.8 GB bf16 tensor (S = 17000003, H = 8, D = 128): 2^31 + 28M chunks,
    more than one launch's 32-bit flat index, so the row walk is split in two
    launches. Device-side full compare against the definition (block j holds
    heads [c_j, c_{j+1})), the round trip, and the oracle on sampled rows
    around the launch boundary (row 2^31 // 128 - 1 = 16777215)."""
    import torch
    B, S, H, D, P = 1, 17_000_003, 8, 128, 3
    hb = R.balanced_ranges(H, P)
    torch.manual_seed(5)
    bits = torch.randint(-32768, 32768, (B, S, H, D), dtype=torch.int16, device=DEV)
    blocks = [torch.empty((B, S, hb[j + 1] - hb[j], D), dtype=torch.bfloat16, device=DEV)
              for j in range(P)]
    log(f"pack world beyond one launch S={S} H={H} D={D} P={P} (34.8 GB)")
    usp.usp_pack_seq_to_heads(bits.view(torch.bfloat16), blocks)
    torch.cuda.synchronize()
    for j in range(P):
        assert torch.equal(blocks[j].view(torch.int16), bits[:, :, hb[j]:hb[j + 1]]), f"block {j}"
    rows = np.array([0, 1, 16777213, 16777214, 16777215, 16777216, 16777217, S - 2, S - 1])
    host = bits[:, rows].cpu().numpy().view(np.uint16)
    ref = X.pack_seq_to_heads(host, P)
    for j in range(P):
        assert blocks[j][:, rows].view(torch.int16).cpu().numpy().view(np.uint16).tobytes() == \
            ref[j].tobytes()
    back = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV)
    log("unpack world beyond one launch")
    usp.usp_unpack_heads_to_seq(blocks, back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), bits)
    del bits, blocks, back
    torch.cuda.empty_cache()


# several tensors (q, k, v) through one launch: bitwise the single-plane calls
PLANE_CASES = [  # B, S, H, D, P, dtype, rank, (head_lo, head_hi) or None
    (1, 32760, 40, 128, 8, BF, -1, None),      # video-DiT world
    (1, 32760, 40, 128, 8, BF, 0, None),       # rank 0's share of it (the benched step)
    (1, 32760, 40, 128, 8, BF, 7, (0, 2)),     # a head-chunk phase of rank 7's share
    (2, 65537, 12, 64, 4, BF, 3, None),        # indivisible tokens, last rank
    (2, 37, 7, 64, 3, BF, 1, None),            # ragged heads 3/2/2
    (1, 257, 6, 64, 3, F, -1, (1, 2)),         # fp32 world, one head of each group
]


@pytest.mark.parametrize("B,S,H,D,P,dtype,rank,heads", PLANE_CASES)
def test_planes_equal_single_plane_calls(B, S, H, D, P, dtype, rank, heads):
    import torch
    n = 3
    tb, hb = R.balanced_ranges(S, P), R.balanced_ranges(H, P)
    L = S if rank < 0 else tb[rank + 1] - tb[rank]
    lo, hi = heads or (0, 0)
    seqs = [to_dev(coded((B, L, H, D), dtype, seed=40 + t), dtype) for t in range(n)]
    blk_a = [[poisoned((B, S, hb[j + 1] - hb[j], D), dtype) for j in range(P)] for _ in range(n)]
    blk_b = [[poisoned((B, S, hb[j + 1] - hb[j], D), dtype) for j in range(P)] for _ in range(n)]
    log(f"planes pack n={n} B={B} S={S} H={H} D={D} P={P} {dtype} rank={rank} heads={heads}")
    usp.usp_pack_seq_to_heads_planes(seqs, blk_a, rank=rank, head_lo=lo, head_hi=hi)
    for t in range(n):
        if heads:
            usp.usp_pack_seq_to_heads_chunk(seqs[t], blk_b[t], lo, hi, rank=rank)
        else:
            usp.usp_pack_seq_to_heads(seqs[t], blk_b[t], rank=rank)
    torch.cuda.synchronize()
    for t in range(n):
        for j in range(P):
            assert to_host(blk_a[t][j]).tobytes() == to_host(blk_b[t][j]).tobytes(), f"plane {t} block {j}"
    out_a = [poisoned((B, L, H, D), dtype) for _ in range(n)]
    out_b = [poisoned((B, L, H, D), dtype) for _ in range(n)]
    log(f"planes unpack n={n} B={B} S={S} H={H} D={D} P={P} {dtype} rank={rank} heads={heads}")
    usp.usp_unpack_heads_to_seq_planes(blk_a, out_a, rank=rank, head_lo=lo, head_hi=hi)
    for t in range(n):
        if heads:
            usp.usp_unpack_heads_to_seq_chunk(blk_a[t], out_b[t], lo, hi, rank=rank)
        else:
            usp.usp_unpack_heads_to_seq(blk_a[t], out_b[t], rank=rank)
    torch.cuda.synchronize()
    for t in range(n):
        got = to_host(out_a[t])
        assert got.tobytes() == to_host(out_b[t]).tobytes(), f"plane {t}"
        if not heads:
            assert got.tobytes() == to_host(seqs[t]).tobytes(), f"plane {t} round trip"


def test_planes_world_against_oracle():
    import torch
    B, S, H, D, P = 2, 37, 7, 64, 3
    seqs = [coded((B, S, H, D), BF, seed=60 + t) for t in range(2)]
    hb = R.balanced_ranges(H, P)
    blocks = [[poisoned((B, S, hb[j + 1] - hb[j], D), BF) for j in range(P)] for _ in range(2)]
    log("planes pack n=2 against the oracle")
    usp.usp_pack_seq_to_heads_planes([to_dev(x, BF) for x in seqs], blocks)
    torch.cuda.synchronize()
    for t in range(2):
        ref = X.pack_seq_to_heads(seqs[t], P)
        for j in range(P):
            assert to_host(blocks[t][j]).tobytes() == ref[j].tobytes()
