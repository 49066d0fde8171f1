"""The Python binding's argument checks (CPU only): the C ABI receives bare
pointers, so shapes, dtypes and devices are checked in the binding, and a
mismatch raises ValueError before anything reaches the library."""
import pytest
import torch

import ulysses_sequence_attention_amd as usp

BF, F = torch.bfloat16, torch.float32


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def test_attention_shapes_dtypes_and_device():
    q, k, v, o = t(1, 8, 2, 64), t(1, 8, 2, 64), t(1, 8, 2, 64), t(1, 8, 2, 64, dtype=F)
    with pytest.raises(ValueError, match="k has shape"):
        usp.usp_attention_fwd(q, t(1, 7, 2, 64), v, o)
    with pytest.raises(ValueError, match="v has dtype"):
        usp.usp_attention_fwd(q, k, t(1, 8, 2, 64, dtype=F), o)
    with pytest.raises(ValueError, match="o has dtype"):
        usp.usp_attention_fwd(q, k, v, t(1, 8, 2, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="lse has shape"):
        usp.usp_attention_fwd(q, k, v, o, lse=t(1, 8, 2, dtype=F))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        usp.usp_attention_fwd(q, k, v, o)
    with pytest.raises(ValueError, match="q must be a 4-dimensional"):
        usp.usp_attention_fwd(t(8, 2, 64), k, v, o)


def test_grouped_block_and_chunked_shapes():
    q, o = t(1, 8, 4, 64), t(1, 8, 4, 64, dtype=F)
    with pytest.raises(ValueError, match="v has shape"):
        usp.usp_attention_fwd_gqa(q, t(1, 8, 2, 64), t(1, 8, 1, 64), o)
    with pytest.raises(ValueError, match="v has shape"):
        usp.usp_attention_fwd_block(q, t(1, 5, 2, 64), t(1, 6, 2, 64), o)
    with pytest.raises(ValueError, match="lse has shape"):
        usp.usp_attention_fwd_block(q, t(1, 5, 2, 64), t(1, 5, 2, 64), o, lse=t(1, 4, 5, dtype=F))
    with pytest.raises(ValueError, match="k has shape"):
        usp.usp_attention_fwd_chunked(q, t(1, 8, 2, 64), t(1, 8, 4, 64), o, 2)


def test_block_whole_shapes_and_device():
    q, o = t(1, 8, 4, 64), t(1, 8, 4, 64, dtype=F)
    with pytest.raises(ValueError, match="v has shape"):
        usp.usp_attention_fwd_block_whole(q, t(1, 5, 2, 64), t(1, 6, 2, 64), o)
    with pytest.raises(ValueError, match="v has dtype"):
        usp.usp_attention_fwd_block_whole(q, t(1, 5, 2, 64), t(1, 5, 2, 64, dtype=F), o)
    with pytest.raises(ValueError, match="lse has shape"):
        usp.usp_attention_fwd_block_whole(q, t(1, 5, 2, 64), t(1, 5, 2, 64), o,
                                          lse=t(1, 4, 5, dtype=F))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        usp.usp_attention_fwd_block_whole(q, t(1, 5, 2, 64), t(1, 5, 2, 64), o)


def test_merge_shapes():
    oa, la = t(1, 8, 2, 64, dtype=F), t(1, 2, 8, dtype=F)
    with pytest.raises(ValueError, match="o_b has shape"):
        usp.usp_attention_merge(oa, la, t(1, 8, 2, 32, dtype=F), la, oa)
    with pytest.raises(ValueError, match="lse_b has shape"):
        usp.usp_attention_merge(oa, la, oa, t(1, 8, 2, dtype=F), oa)
    with pytest.raises(ValueError, match="o_a has dtype"):
        usp.usp_attention_merge(t(1, 8, 2, 64), la, oa, la, oa)


def test_relayout_block_shapes_follow_the_balanced_ranges():
    seq = t(2, 10, 7, 64)                       # 7 heads over 3 ranks: 3 / 2 / 2
    good = [t(2, 10, 3, 64), t(2, 10, 2, 64), t(2, 10, 2, 64)]
    bad = [t(2, 10, 2, 64), t(2, 10, 3, 64), t(2, 10, 2, 64)]
    with pytest.raises(ValueError, match=r"blocks\[0\] has shape"):
        usp.usp_pack_seq_to_heads(seq, bad)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        usp.usp_pack_seq_to_heads(seq, good)
    with pytest.raises(ValueError, match=r"blocks\[1\] has dtype"):
        usp.usp_unpack_heads_to_seq([good[0], t(2, 10, 2, 64, dtype=F), good[2]], seq)
    # rank share: rank 1 of 10 tokens over 3 ranks holds 3 rows
    with pytest.raises(ValueError, match="seq has shape"):
        usp.usp_pack_seq_to_heads(t(2, 4, 7, 64), good, rank=1)


def test_chunk_relayout_block_shapes():
    seq = t(2, 10, 6, 64)                       # 6 heads over 3 ranks: groups of 2
    good = [t(2, 10, 2, 64) for _ in range(3)]
    with pytest.raises(ValueError, match=r"blocks\[2\] has shape"):
        usp.usp_pack_seq_to_heads_chunk(seq, good[:2] + [t(2, 10, 3, 64)], 0, 1)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        usp.usp_pack_seq_to_heads_chunk(seq, good, 0, 1)
    with pytest.raises(ValueError, match=r"blocks\[0\] has dtype"):
        usp.usp_unpack_heads_to_seq_chunk([t(2, 10, 2, 64, dtype=F)] + good[1:], seq, 1, 2)
    with pytest.raises(ValueError, match="seq has shape"):           # rank 0 holds 4 rows
        usp.usp_unpack_heads_to_seq_chunk(good, t(2, 3, 6, 64), 0, 2, rank=0)


def test_row_shard_shapes_follow_the_balanced_ranges():
    full = t(1, 10, 16)                         # 10 rows over 3 ranks: 4 / 3 / 3
    with pytest.raises(ValueError, match=r"shards\[0\] has shape"):
        usp.usp_scatter_rows(full, [t(1, 3, 16), t(1, 3, 16), t(1, 4, 16)])
    with pytest.raises(ValueError, match=r"shards\[2\] has shape"):
        usp.usp_scatter_rows(full, [None, None, t(1, 4, 16)], rank=2)
    with pytest.raises(ValueError, match=r"partials\[1\] has shape"):
        usp.usp_reduce_scatter_rows([full, t(1, 9, 16), full], [t(1, 4, 16), t(1, 3, 16), t(1, 3, 16)])
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        usp.usp_gather_rows([t(1, 4, 16), t(1, 3, 16), t(1, 3, 16)], full)
