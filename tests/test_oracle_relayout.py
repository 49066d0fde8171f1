"""Pins for the oracle's relayouts and scatter / gather (CPU only).

Index-coded tensors (every element holds its own flat index) make each
destination element's expected value a closed form of its position."""
import numpy as np
import pytest

from oracle import relayout as X
from ulysses_sequence_attention_amd import synth

SHAPES = [  # B, S, H, D, P
    (1, 7, 6, 4, 3),
    (2, 5, 7, 2, 3),     # ragged heads 3/2/2
    (1, 9, 4, 3, 4),     # ragged tokens 3/2/2/2
    (3, 5, 5, 1, 5),     # one head and one token per group
    (1, 6, 3, 2, 1),     # P = 1
]


def _heads_groups(H, P):
    # head groups from an independent library routine (same remainder rule)
    return np.array_split(np.arange(H), P)


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_pack_closed_form(B, S, H, D, P):
    seq = synth.index_coded((B, S, H, D), "f32")
    blocks = X.pack_seq_to_heads(seq, P)
    groups = _heads_groups(H, P)
    for j in range(P):
        assert blocks[j].shape == (B, S, len(groups[j]), D)
        for b in range(B):
            for s in range(S):
                for i, head in enumerate(groups[j]):
                    for d in range(D):
                        assert blocks[j][b, s, i, d] == ((b * S + s) * H + head) * D + d


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_pack_matches_library_split(B, S, H, D, P):
    seq = synth.index_coded((B, S, H, D), "bf16")
    blocks = X.pack_seq_to_heads(seq, P)
    for j, ref in enumerate(np.array_split(seq, P, axis=2)):
        assert np.array_equal(blocks[j], ref)


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_roundtrips(B, S, H, D, P):
    seq = synth.index_coded((B, S, H, D), "bf16")
    blocks = X.pack_seq_to_heads(seq, P)
    back = X.unpack_heads_to_seq(blocks, H)
    assert back.tobytes() == seq.tobytes()
    again = X.pack_seq_to_heads(back, P)
    for a, b in zip(blocks, again):
        assert a.tobytes() == b.tobytes()


def test_p1_is_byte_identical():
    seq = synth.index_coded((2, 5, 3, 4), "bf16")
    (blk,) = X.pack_seq_to_heads(seq, 1)
    assert blk.tobytes() == seq.tobytes()
    assert X.unpack_heads_to_seq([blk], 3).tobytes() == seq.tobytes()


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_elementwise_variant_agrees(B, S, H, D, P):
    seq = synth.index_coded((B, S, H, D), "f32")
    a = X.pack_seq_to_heads(seq, P)
    b = X.pack_seq_to_heads_elementwise(seq, P)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_rank_shares_tile_the_world(B, S, H, D, P):
    seq = synth.index_coded((B, S, H, D), "f32")
    world = X.pack_seq_to_heads(seq, P)
    groups = _heads_groups(H, P)
    tok = np.array_split(np.arange(S), P)
    sentinel = -1.0
    blocks = [np.full((B, S, len(g), D), sentinel, np.float32) for g in groups]
    for r in range(P):
        shard = X.scatter_sequence(seq, P, r)
        before = [blk.copy() for blk in blocks]
        X.pack_rank_share(shard, blocks, S, r)
        for j in range(P):
            changed = np.any(blocks[j] != before[j], axis=(0, 2, 3))
            # only rank r's rows may change
            assert set(np.nonzero(changed)[0]) <= set(tok[r].tolist())
    for j in range(P):
        assert np.array_equal(blocks[j], world[j])
    for r in range(P):
        assert np.array_equal(X.unpack_rank_share(world, H, r),
                              X.scatter_sequence(seq, P, r))


@pytest.mark.parametrize("S,P", [(7, 3), (9, 4), (5, 5), (6, 1)])
def test_scatter_gather_identity(S, P):
    x = synth.index_coded((2, S, 3), "f32")
    shards = [X.scatter_sequence(x, P, r) for r in range(P)]
    assert [s.shape[1] for s in shards] == [len(t) for t in np.array_split(np.arange(S), P)]
    assert np.array_equal(X.gather_sequence(shards), x)


# ---- reduce-scatter of rows (h3 reduce_scatter_rows) ----------------------

@pytest.mark.parametrize("S,P", [(10, 3), (9, 4), (17, 1), (64, 8)])
def test_reduce_scatter_integer_partials_exact(S, P):
    rng = np.random.default_rng(S * P)
    parts = [rng.integers(-1000, 1000, size=(2, S, 5)).astype(np.float64) for _ in range(P)]
    total = np.zeros((2, S, 5))
    for x in parts:
        total = total + x
    for r in range(P):
        assert np.array_equal(X.reduce_scatter_rows(parts, r), X.scatter_sequence(total, P, r))


def test_reduce_scatter_single_rank_is_passthrough():
    x = np.random.default_rng(1).standard_normal((1, 7, 3))
    assert np.array_equal(X.reduce_scatter_rows([x], 0), x)


def test_reduce_scatter_matches_loops():
    rng = np.random.default_rng(3)
    S, P, W = 11, 3, 4
    parts = [rng.standard_normal((1, S, W)) for _ in range(P)]
    bounds = [0, 4, 8, 11]  # 11 rows over 3 ranks: 4, 4, 3
    for r in range(P):
        got = X.reduce_scatter_rows(parts, r)
        for i, s in enumerate(range(bounds[r], bounds[r + 1])):
            for w in range(W):
                ref = 0.0
                for j in range(P):
                    ref += float(parts[j][0, s, w])
                assert abs(got[0, i, w] - ref) <= 1e-15


def test_reduce_scatter_ranges_tile_the_sum():
    rng = np.random.default_rng(4)
    parts = [rng.standard_normal((2, 13, 3)) for _ in range(5)]
    out = X.gather_sequence([X.reduce_scatter_rows(parts, r) for r in range(5)])
    assert np.max(np.abs(out - sum(parts))) <= 1e-14


def test_reduce_scatter_rejects_mismatched_partials():
    with pytest.raises(ValueError):
        X.reduce_scatter_rows([np.zeros((1, 8, 2)), np.zeros((1, 7, 2))], 0)


# ---- head-chunk phases of the two-phase exchange ----------------------------
CHUNK_SHAPES = [  # B, S, H, D, P, chunks (equal head groups of h = H / P)
    (1, 7, 6, 4, 3, 2),     # h = 2: chunks 1/1
    (2, 9, 15, 2, 3, 3),    # h = 5: 2/2/1, ragged tokens 3/3/3 -> remainder chunk
    (1, 9, 16, 3, 2, 3),    # h = 8: 3/3/2
    (3, 5, 5, 2, 5, 1),     # one head per group, one chunk
    (1, 6, 3, 2, 1, 2),     # P = 1, h = 3: 2/1
]


def _chunks(h, chunks):
    # the plan, restated: ceil(h / chunks) heads per chunk, the last one short
    size = -(-h // chunks)
    return [(c * size, min((c + 1) * size, h)) for c in range(chunks)]


@pytest.mark.parametrize("B,S,H,D,P,chunks", CHUNK_SHAPES)
def test_chunk_packs_fill_the_blocks_chunk_by_chunk(B, S, H, D, P, chunks):
    seq = synth.index_coded((B, S, H, D), "f32")
    groups = _heads_groups(H, P)
    h = H // P
    blocks = [np.full((B, S, h, D), -1.0, np.float32) for _ in range(P)]
    done = set()
    for lo, hi in _chunks(h, chunks):
        before = [b.copy() for b in blocks]
        X.pack_heads_chunk(seq, blocks, S, lo, hi)
        for j in range(P):
            changed = set(np.nonzero(np.any(blocks[j] != before[j], axis=(0, 1, 3)))[0].tolist())
            assert changed == set(range(lo, hi))          # its heads, all rows
        done |= set(range(lo, hi))
    assert done == set(range(h))
    for j in range(P):                                     # closed form of every element
        for b in range(B):
            for s in range(S):
                for i, head in enumerate(groups[j]):
                    assert np.all(blocks[j][b, s, i] == ((b * S + s) * H + head) * D + np.arange(D))


@pytest.mark.parametrize("B,S,H,D,P,chunks", CHUNK_SHAPES)
def test_chunk_unpacks_rebuild_the_sequence_chunk_by_chunk(B, S, H, D, P, chunks):
    seq = synth.index_coded((B, S, H, D), "bf16")
    blocks = np.array_split(seq, P, axis=2)               # head blocks from a library split
    out = np.zeros_like(seq)
    h = H // P
    for lo, hi in _chunks(h, chunks):
        before = out.copy()
        X.unpack_heads_chunk(blocks, out, S, lo, hi)
        heads = set(np.nonzero(np.any(out != before, axis=(0, 1, 3)))[0].tolist())
        assert heads <= {j * h + i for j in range(P) for i in range(lo, hi)}
    assert out.tobytes() == seq.tobytes()


@pytest.mark.parametrize("B,S,H,D,P,chunks", CHUNK_SHAPES)
def test_chunk_rank_shares_tile_the_world(B, S, H, D, P, chunks):
    seq = synth.index_coded((B, S, H, D), "f32")
    world = np.array_split(seq, P, axis=2)
    tok = np.array_split(np.arange(S), P)
    h = H // P
    blocks = [np.full((B, S, h, D), -1.0, np.float32) for _ in range(P)]
    for lo, hi in _chunks(h, chunks):
        for r in range(P):
            before = [b.copy() for b in blocks]
            X.pack_heads_chunk(seq[:, tok[r]], blocks, S, lo, hi, rank=r)
            for j in range(P):
                rows = set(np.nonzero(np.any(blocks[j] != before[j], axis=(0, 2, 3)))[0].tolist())
                assert rows <= set(tok[r].tolist())
    for j in range(P):
        assert np.array_equal(blocks[j], world[j])
    for r in range(P):
        shard = np.zeros((B, len(tok[r]), H, D), np.float32)
        for lo, hi in _chunks(h, chunks):
            X.unpack_heads_chunk(world, shard, S, lo, hi, rank=r)
        assert np.array_equal(shard, seq[:, tok[r]])


def test_chunk_relayouts_reject_bad_plans():
    seq = synth.index_coded((1, 6, 6, 2), "f32")
    blocks = [np.zeros((1, 6, 2, 2), np.float32) for _ in range(3)]
    with pytest.raises(ValueError, match="equal head groups"):
        X.pack_heads_chunk(synth.index_coded((1, 6, 7, 2), "f32"), blocks, 6, 0, 1)
    for lo, hi in [(0, 0), (1, 3), (-1, 1), (2, 1)]:
        with pytest.raises(ValueError, match="head chunk"):
            X.pack_heads_chunk(seq, blocks, 6, lo, hi)
        with pytest.raises(ValueError, match="head chunk"):
            X.unpack_heads_chunk(blocks, np.zeros_like(seq), 6, lo, hi)
    with pytest.raises(ValueError, match="rows"):
        X.pack_heads_chunk(seq[:, :3], blocks, 6, 0, 1, rank=0)   # rank 0 holds 2 rows
