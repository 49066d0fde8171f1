"""Balanced contiguous ranges and the head-chunk plan (oracle; test infrastructure).

Sources:
  * h3-blackwell-runtime ``distributed.py`` (blame view), function
    ``balanced_ranges``: split ``total`` ordered items into ``parts``
    contiguous, non-empty ranges whose lengths are ``base`` or ``base + 1``
    with ``base, extra = divmod(total, parts)``; the first ``extra`` ranks
    take the longer length; fewer items than parts, or fewer than one part,
    is an error.
  * m-star ``sequence_parallel`` API page, ``sp_seq_split``: per-rank token
    counts summing to the total, the first total mod P ranks holding one extra
    item.
  * maxdiffusion PR #428 "two-phase (head-chunked) Ulysses all-to-all",
    description: head-group passes, the last one taking the heads left over.
"""
from __future__ import annotations


def balanced_ranges(total: int, parts: int) -> list[int]:
    """Boundaries ``[b_0 = 0, b_1, ..., b_parts = total]``; range r is
    ``[b_r, b_{r+1})``.

    h3-blackwell-runtime ``distributed.py``, ``balanced_ranges``.
    """
    if parts < 1:
        raise ValueError("parts must be positive")
    if total < parts:
        raise ValueError(f"cannot split {total} items into {parts} non-empty ranges")
    base, extra = divmod(total, parts)
    bounds = [0]
    for rank in range(parts):
        length = base + (1 if rank < extra else 0)
        bounds.append(bounds[-1] + length)
    return bounds


def range_lengths(bounds: list[int]) -> list[int]:
    """``stop - start`` per range (h3-blackwell-runtime, ``range_lengths``)."""
    return [bounds[r + 1] - bounds[r] for r in range(len(bounds) - 1)]


def seq_split(total: int, world_size: int) -> list[int]:
    """Per-rank token counts (m-star ``sp_seq_split``): the lengths of
    ``balanced_ranges``."""
    return range_lengths(balanced_ranges(total, world_size))


def head_chunk_ranges(heads: int, chunks: int) -> list[int]:
    """Boundaries of ``chunks`` head-chunk passes over ``heads`` local heads.

    maxdiffusion PR #428 splits the all-to-all plus attention into head-group
    passes, the last pass taking whatever heads are left. Reading taken here:
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
