"""Pins for the oracle's balanced ranges and head-chunk plan (CPU only)."""
import os

import numpy as np
import pytest

from oracle import ranges as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "range_splits.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("[")[0].strip()
            if not line or line.startswith("#"):
                continue
            kind, total, parts, *lengths = line.split()
            rows.append((kind, int(total), int(parts), [int(x) for x in lengths]))
    return rows


@pytest.mark.parametrize("kind,total,parts,lengths", _golden())
def test_golden_splits(kind, total, parts, lengths):
    if kind == "chunks":
        b = R.head_chunk_ranges(total, parts)
    else:
        b = R.balanced_ranges(total, parts)
    assert R.range_lengths(b) == lengths
    assert b[0] == 0 and b[-1] == total


def test_matches_numpy_array_split():
    # numpy.array_split gives the first (total % parts) pieces one extra item:
    # the same convention, from an independent library routine.
    for total in range(1, 65):
        for parts in range(1, total + 1):
            ref = [len(x) for x in np.array_split(np.arange(total), parts)]
            assert R.seq_split(total, parts) == ref


def test_properties_brute_force():
    for total in range(1, 65):
        for parts in range(1, total + 1):
            b = R.balanced_ranges(total, parts)
            L = R.range_lengths(b)
            assert len(b) == parts + 1 and b[0] == 0 and b[-1] == total
            assert sum(L) == total
            assert min(L) >= 1
            assert max(L) - min(L) <= 1
            assert all(L[i] >= L[i + 1] for i in range(parts - 1))
            # the longer ranges are exactly the first total % parts ranks
            assert sum(1 for x in L if x > total // parts) == total % parts
            # contiguous and rank ordered
            assert all(b[i] < b[i + 1] for i in range(parts))


@pytest.mark.parametrize("total,parts", [(5, 0), (5, -1), (3, 4), (0, 1)])
def test_errors(total, parts):
    with pytest.raises(ValueError):
        R.balanced_ranges(total, parts)


def test_chunk_plan_properties():
    for heads in range(1, 33):
        for chunks in range(1, heads + 1):
            try:
                b = R.head_chunk_ranges(heads, chunks)
            except ValueError:
                # only plans whose ceil-sized chunks run out before the last
                size = -(-heads // chunks)
                assert (chunks - 1) * size >= heads
                continue
            L = R.range_lengths(b)
            assert len(L) == chunks and sum(L) == heads and min(L) >= 1
            size = -(-heads // chunks)
            assert all(x == size for x in L[:-1]) and L[-1] <= size


@pytest.mark.parametrize("heads,chunks", [(8, 0), (3, 4), (0, 1), (5, 4)])
def test_chunk_errors(heads, chunks):
    # (5, 4): chunks of ceil(5/4) = 2 would leave the fourth chunk empty
    with pytest.raises(ValueError):
        R.head_chunk_ranges(heads, chunks)
