"""Balanced contiguous ranges and the head-chunk plan (oracle; test infrastructure).

Sources:
  * h3-blackwell-runtime ``distributed.py`` (blame view), function
    ``balanced_ranges``: the items, in order, go to ``parts`` consecutive
    runs, none of them empty; every run has ``q = total // parts`` items and
    the lowest ``total % parts`` runs one more; asking for no runs at all,
    or for more runs than items, raises an error.
  * m-star ``sequence_parallel`` API page, ``sp_seq_split``: how many tokens
    each rank gets; the counts add up to the sequence length and differ by
    at most one, the first total mod P ranks holding the extra token.
  * maxdiffusion PR #428 "two-phase (head-chunked) Ulysses all-to-all",
    description: one pass per group of heads, the last one taking the heads
    left over.
"""
from __future__ import annotations

import itertools


def balanced_ranges(total: int, parts: int) -> list[int]:
    """Boundaries ``[b_0 = 0, b_1, ..., b_parts = total]``; range r is
    ``[b_r, b_{r+1})``.

    h3-blackwell-runtime ``distributed.py``, ``balanced_ranges``: the
    lowest ``total % parts`` runs hold ``q + 1`` items, the others ``q``;
    the boundaries are the running sums of those sizes.
    """
    if parts < 1:
        raise ValueError(f"need at least one range (got {parts})")
    if total < parts:
        raise ValueError(f"{total} items are too few for {parts} ranges of one item or more")
    q, longer = total // parts, total % parts
    sizes = [q + 1] * longer + [q] * (parts - longer)
    return [0] + list(itertools.accumulate(sizes))


def range_lengths(bounds: list[int]) -> list[int]:
    """``stop - start`` per range (h3-blackwell-runtime, ``range_lengths``)."""
    return [bounds[r + 1] - bounds[r] for r in range(len(bounds) - 1)]


def seq_split(total: int, world_size: int) -> list[int]:
    """Per-rank token counts (m-star ``sp_seq_split``): the lengths of
    ``balanced_ranges``."""
    return range_lengths(balanced_ranges(total, world_size))


def head_chunk_ranges(heads: int, chunks: int) -> list[int]:
    """Boundaries of ``chunks`` head-chunk passes over ``heads`` local heads.

    maxdiffusion PR #428 runs the exchange and the attention once per group
    of heads, in turn; an uneven count leaves the last group short. Reading
    taken here:
    every chunk but the last holds ``ceil(heads / chunks)`` heads and the last
    holds what is left (8 heads in 3 chunks: 3/3/2). A plan that would leave a
    chunk empty is rejected.
    """
    if chunks < 1:
        raise ValueError("chunks must be positive")
    if heads < 1:
        raise ValueError("heads must be positive")
    if chunks > heads:
        raise ValueError(f"cannot run {heads} heads in {chunks} non-empty chunks")
    size = -(-heads // chunks)
    bounds = [min(c * size, heads) for c in range(chunks)] + [heads]
    for c in range(chunks):
        if bounds[c + 1] <= bounds[c]:
            raise ValueError(f"{chunks} chunks of {size} heads leave chunk {c} empty "
                             f"for {heads} heads")
    return bounds
