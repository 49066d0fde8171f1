"""Sequence-sharded <-> head-sharded relayouts (oracle; test infrastructure).

What the pages define:
  * m-star ``sequence_parallel`` module description: before attention an
    all-to-all converts each rank's token shard, shape ``[seq/P, heads,
    dim]``, into all tokens over the rank's own head group, shape ``[seq,
    heads/P, dim]``; after attention a second all-to-all converts the output
    the opposite way.
  * h3-blackwell-runtime ``distributed.py``, ``SequenceParallelContext.
    seq_to_heads``: rank r sends, to each rank j, its own token rows restricted
    to j's head range; rank j concatenates what it receives in source-rank
    order along the token axis, so it ends with every token over its own
    heads. ``heads_to_seq`` is the inverse: rank j sends each rank r the token
    rows r owns, and r concatenates the pieces along the head axis in rank
    order.
  * m-star ``sp_head_slice``: rank j's heads are the contiguous group
    ``[c_j, c_{j+1})`` (``[rank*H/P, (rank+1)*H/P)`` for an even split).
  * m-star ``scatter_sequence`` / ``gather_sequence``: a rank's shard is its
    contiguous token window; gathering concatenates shards in rank order.

Layouts ("world" = all P ranks held side by side on one host):
  * sequence-sharded world: ``seq[B, S, H, D]``; rank r owns rows
    ``[t_r, t_{r+1})`` of every batch row.
  * head-sharded world: a list of P blocks, block j ``[B, S, h_j, D]`` holding
    heads ``[c_j, c_{j+1})`` — what rank j holds after the first all-to-all.

Everything below is explicit index loops copying D-vectors (or single
elements, in the ``*_elementwise`` variants), with no vectorised slicing
tricks, so the mapping can be read off directly.
"""
from __future__ import annotations

import numpy as np

from .ranges import balanced_ranges


def _plan(S: int, H: int, P: int):
    return balanced_ranges(S, P), balanced_ranges(H, P)


def pack_seq_to_heads(seq: np.ndarray, P: int) -> list[np.ndarray]:
    """World pack: ``seq[B,S,H,D]`` -> P blocks ``[B,S,h_j,D]`` with
    ``block_j[b,s,i,:] = seq[b,s,c_j+i,:]``."""
    B, S, H, D = seq.shape
    _, hb = _plan(S, H, P)
    blocks = [np.empty((B, S, hb[j + 1] - hb[j], D), dtype=seq.dtype) for j in range(P)]
    for j in range(P):
        for b in range(B):
            for s in range(S):
                for i in range(hb[j + 1] - hb[j]):
                    blocks[j][b, s, i, :] = seq[b, s, hb[j] + i, :]
    return blocks


def unpack_heads_to_seq(blocks: list[np.ndarray], H: int) -> np.ndarray:
    """World unpack: P blocks ``[B,S,h_j,D]`` -> ``seq[B,S,H,D]`` with
    ``seq[b,s,c_j+i,:] = block_j[b,s,i,:]``."""
    P = len(blocks)
    B, S, _, D = blocks[0].shape
    _, hb = _plan(S, H, P)
    seq = np.empty((B, S, H, D), dtype=blocks[0].dtype)
    for j in range(P):
        assert blocks[j].shape == (B, S, hb[j + 1] - hb[j], D)
        for b in range(B):
            for s in range(S):
                for i in range(hb[j + 1] - hb[j]):
                    seq[b, s, hb[j] + i, :] = blocks[j][b, s, i, :]
    return seq


def pack_rank_share(shard: np.ndarray, blocks: list[np.ndarray], S: int, rank: int) -> None:
    """Rank ``rank``'s share of the pack: its shard ``[B, len_r, H, D]`` is
    written into rows ``[t_r, t_{r+1})`` of every block (in place); no other
    rows of the blocks are touched.

    h3-blackwell-runtime ``seq_to_heads``: rank r's send to rank j is exactly
    its own token rows over j's heads, and j places it at r's token offset.
    """
    P = len(blocks)
    B, L, H, D = shard.shape
    tb, hb = _plan(S, H, P)
    assert L == tb[rank + 1] - tb[rank]
    for j in range(P):
        for b in range(B):
            for s in range(L):
                for i in range(hb[j + 1] - hb[j]):
                    blocks[j][b, tb[rank] + s, i, :] = shard[b, s, hb[j] + i, :]


def unpack_rank_share(blocks: list[np.ndarray], H: int, rank: int) -> np.ndarray:
    """Rank ``rank``'s share of the unpack: rows ``[t_r, t_{r+1})`` of every
    block, put back side by side over all heads -> ``[B, len_r, H, D]``.

    h3-blackwell-runtime ``heads_to_seq``: rank r receives, from each rank j,
    its own token rows over j's heads and concatenates them along heads in
    rank order.
    """
    P = len(blocks)
    B, S, _, D = blocks[0].shape
    tb, hb = _plan(S, H, P)
    L = tb[rank + 1] - tb[rank]
    out = np.empty((B, L, H, D), dtype=blocks[0].dtype)
    for j in range(P):
        for b in range(B):
            for s in range(L):
                for i in range(hb[j + 1] - hb[j]):
                    out[b, s, hb[j] + i, :] = blocks[j][b, tb[rank] + s, i, :]
    return out


def pack_seq_to_heads_elementwise(seq: np.ndarray, P: int) -> list[np.ndarray]:
    """Same mapping as ``pack_seq_to_heads``, one element at a time (used on
    tiny shapes to pin the D-vector loop)."""
    B, S, H, D = seq.shape
    _, hb = _plan(S, H, P)
    blocks = [np.empty((B, S, hb[j + 1] - hb[j], D), dtype=seq.dtype) for j in range(P)]
    for j in range(P):
        for b in range(B):
            for s in range(S):
                for i in range(hb[j + 1] - hb[j]):
                    for d in range(D):
                        blocks[j][b, s, i, d] = seq[b, s, hb[j] + i, d]
    return blocks


def _chunk_plan(S: int, H: int, P: int, lo: int, hi: int):
    """Token ranges and the per-group head count for a head-chunk relayout;
    the chunk ``[lo, hi)`` indexes heads within each (equal) group."""
    if H % P:
        raise ValueError(f"head-chunk relayouts need equal head groups: P ({P}) has to divide H ({H})")
    h = H // P
    if not 0 <= lo < hi <= h:
        raise ValueError(f"head chunk [{lo}, {hi}) is empty or outside a group of {h} heads")
    return balanced_ranges(S, P), balanced_ranges(H, P)


def pack_heads_chunk(src: np.ndarray, blocks: list[np.ndarray], S: int, lo: int, hi: int,
                     rank: int | None = None) -> None:
    """One phase of the head-chunked exchange, pack side (in place).

    maxdiffusion PR #428 (description): the exchange and the attention run
    once per chunk of every rank's heads, so only heads ``[lo, hi)`` of each
    group move in a phase. With equal groups of h = H / P heads, block j
    receives ``block_j[b, t, i, :] = seq[b, t, c_j + i, :]`` for ``lo <= i <
    hi`` and every row t (world, ``src`` = ``seq[B, S, H, D]``) or only rows
    ``[t_r, t_{r+1})`` (rank r's share, ``src`` = its shard ``[B, len_r, H,
    D]``); nothing else in the blocks is written.
    """
    P = len(blocks)
    B, L, H, D = src.shape
    tb, hb = _chunk_plan(S, H, P, lo, hi)
    t0 = 0 if rank is None else tb[rank]
    if L != (S if rank is None else tb[rank + 1] - tb[rank]):
        raise ValueError(f"source has {L} rows, expected {S if rank is None else tb[rank + 1] - tb[rank]}")
    for j in range(P):
        for b in range(B):
            for s in range(L):
                for i in range(lo, hi):
                    blocks[j][b, t0 + s, i, :] = src[b, s, hb[j] + i, :]


def unpack_heads_chunk(blocks: list[np.ndarray], dst: np.ndarray, S: int, lo: int, hi: int,
                       rank: int | None = None) -> None:
    """Unpack side of one head-chunk phase (in place): heads ``[lo, hi)`` of
    every block go back to their place among all heads,
    ``dst[b, s, c_j + i, :] = block_j[b, t0 + s, i, :]`` (world: ``dst`` =
    ``[B, S, H, D]``, t0 = 0; rank r's share: ``dst`` = ``[B, len_r, H, D]``,
    t0 = t_r); other heads of ``dst`` are not written."""
    P = len(blocks)
    B, L, H, D = dst.shape
    tb, hb = _chunk_plan(S, H, P, lo, hi)
    t0 = 0 if rank is None else tb[rank]
    if L != (S if rank is None else tb[rank + 1] - tb[rank]):
        raise ValueError(f"destination has {L} rows, expected {S if rank is None else tb[rank + 1] - tb[rank]}")
    for j in range(P):
        for b in range(B):
            for s in range(L):
                for i in range(lo, hi):
                    dst[b, s, hb[j] + i, :] = blocks[j][b, t0 + s, i, :]


def scatter_sequence(x_full: np.ndarray, P: int, rank: int) -> np.ndarray:
    """m-star ``scatter_sequence``: rank r's contiguous window of tokens
    (axis 1) of a replicated ``[B, S, ...]`` tensor."""
    tb = balanced_ranges(x_full.shape[1], P)
    return x_full[:, tb[rank]:tb[rank + 1]].copy()


def gather_sequence(shards: list[np.ndarray]) -> np.ndarray:
    """m-star ``gather_sequence``: concatenate per-rank token shards (axis 1)
    in rank order."""
    return np.concatenate(shards, axis=1)


def reduce_scatter_rows(partials: list[np.ndarray], rank: int) -> np.ndarray:
    """h3 ``reduce_scatter_rows``: each of the P ranks holds a partial sum of
    the full sequence ``[B, S, ...]`` (tensor-parallel partials); rank r
    receives rows [t_r, t_{r+1}) (balanced ranges of S) of their sum, added
    in rank order, in float64."""
    P = len(partials)
    S = partials[0].shape[1]
    for x in partials:
        if x.shape != partials[0].shape:
            raise ValueError("partials must all cover the same [B, S, ...] rows")
    tb = balanced_ranges(S, P)
    acc = np.zeros(partials[0][:, tb[rank]:tb[rank + 1]].shape, dtype=np.float64)
    for j in range(P):
        acc += np.asarray(partials[j][:, tb[rank]:tb[rank + 1]], dtype=np.float64)
    return acc
