"""Non-causal multi-head attention, float64 (oracle; test infrastructure).

What the pages define: m-star ``sequence_parallel`` module description and
``ulysses_attention`` — of the model's steps only attention mixes
information across all tokens; under Ulysses each rank runs the unchanged
attention kernel over the full sequence for its own group of heads, and no
head reads another head's data (maxdiffusion PR #428 description: for that
reason head-chunked passes give exactly the single-shot result). The
kernel itself is opaque on the pages; what it computes is taken as standard
scaled dot-product attention, non-causal, per head:

    O[s, :] = sum_t softmax_t(sigma * <Q[s,:], K[t,:]>) * V[t, :]

with sigma = 1/sqrt(D) unless another scale is given (the pages never state
the scale; 1/sqrt(D) is the standard choice).

Grouped K/V heads (m-star ``ulysses_attention``: q has Hq heads, k and v Hkv,
the SP degree dividing both): query head n attends with key/value head
floor(n / G), G = Hq / Hkv, i.e. each run of G consecutive query heads shares
one K/V head. The pages do not spell out the mapping; this is the one under
which contiguous head sharding keeps every rank's query heads with its own
K/V heads, which the divisibility rule requires.

The query rows and the keys may come from different sequence blocks (a
query block of Sq rows against a key/value block of Sk rows): the formula is
the same with t running over the Sk keys of the block.

The oracle evaluates it directly and in two passes (not online): scores,
row maximum, exponentials, row sum, then the weighted sum divided by the row
sum, all in float64, over blocks of query rows. ``lse`` is the natural-log
normaliser ``log sum_t exp(sigma * <Q[s], K[t]>)``.
"""
from __future__ import annotations

import math
import os

import numpy as np


def _scale(D: int, scale) -> float:
    return 1.0 / math.sqrt(D) if scale is None or scale <= 0 else float(scale)


def kv_head(h: int, hkv: int, head: int) -> int:
    """K/V head of query ``head`` when ``h`` query heads share ``hkv``."""
    if hkv < 1 or h % hkv:
        raise ValueError(f"{h} query heads cannot share {hkv} key/value heads evenly")
    return head // (h // hkv)


def _rows_one_head(Qh: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, sigma: float):
    """Two-pass softmax attention of query rows ``Qh [n, D]`` against
    ``Kh, Vh [S, D]`` (all float64). Returns ``(O [n, D], lse [n])``."""
    s = sigma * (Qh @ Kh.T)                  # [n, S] scores
    m = s.max(axis=1, keepdims=True)         # row maximum (first pass)
    p = np.exp(s - m)                        # unnormalised probabilities
    l = p.sum(axis=1, keepdims=True)         # row sum
    o = (p @ Vh) / l                         # second pass: weighted sum of V
    lse = (m + np.log(l))[:, 0]
    return o, lse


def attention(q, k, v, scale=None, row_block: int = 256, return_lse: bool = False):
    """Attention over every head of ``q [B, S, h, D]`` with ``k, v
    [B, Sk, hkv, D]`` (``hkv`` divides ``h``; ``Sk`` defaults to the query
    length but may differ; any float dtype, computed in float64). Returns
    ``O [B, S, h, D]`` float64 and, if asked, ``lse [B, h, S]``."""
    B, S, h, D = q.shape
    Sk, hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, Sk, hkv, D) and v.shape == (B, Sk, hkv, D) and Sk >= 1
    sigma = _scale(D, scale)
    out = np.empty((B, S, h, D), dtype=np.float64)
    lse = np.empty((B, h, S), dtype=np.float64)
    for b in range(B):
        for hd in range(h):
            kh = kv_head(h, hkv, hd)
            Qh = np.ascontiguousarray(q[b, :, hd, :], dtype=np.float64)
            Kh = np.ascontiguousarray(k[b, :, kh, :], dtype=np.float64)
            Vh = np.ascontiguousarray(v[b, :, kh, :], dtype=np.float64)
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                o, ls = _rows_one_head(Qh[r0:r1], Kh, Vh, sigma)
                out[b, r0:r1, hd, :] = o
                lse[b, hd, r0:r1] = ls
    return (out, lse) if return_lse else out


def attention_rows(q, k, v, b: int, head: int, rows, scale=None):
    """Attention for selected query ``rows`` of one ``(b, head)``; returns
    ``(O [len(rows), D], lse [len(rows)])`` in float64."""
    D = q.shape[3]
    kh = kv_head(q.shape[2], k.shape[2], head)
    rows = np.asarray(rows, dtype=np.int64)
    Qh = np.asarray(q[b, rows, head, :], dtype=np.float64)
    Kh = np.ascontiguousarray(k[b, :, kh, :], dtype=np.float64)
    Vh = np.ascontiguousarray(v[b, :, kh, :], dtype=np.float64)
    return _rows_one_head(Qh, Kh, Vh, _scale(D, scale))


def attention_bruteforce(q, k, v, scale=None):
    """Pure-Python triple loops with ``math.exp`` (tiny inputs only). Same
    definition, no NumPy arithmetic: independent check of ``attention``."""
    B, S, h, D = q.shape
    Sk = k.shape[1]
    G = h // k.shape[2]
    sigma = _scale(D, scale)
    out = np.zeros((B, S, h, D), dtype=np.float64)
    for b in range(B):
        for hd in range(h):
            kh = hd // G
            for s in range(S):
                scores = []
                for t in range(Sk):
                    dot = 0.0
                    for d in range(D):
                        dot += float(q[b, s, hd, d]) * float(k[b, t, kh, d])
                    scores.append(sigma * dot)
                mx = max(scores)
                weights = [math.exp(x - mx) for x in scores]
                total = sum(weights)
                for d in range(D):
                    acc = 0.0
                    for t in range(Sk):
                        acc += weights[t] * float(v[b, t, kh, d])
                    out[b, s, hd, d] = acc / total
    return out


# --------------------------------------------------------------------------
# Process-pool driver: the same computation spread over host cores, one BLAS
# thread per worker. Work items are (b, head, row block); workers inherit the
# inputs through fork and convert each (b, head) plane to float64 once.
# --------------------------------------------------------------------------
_POOL_INPUTS = None
_POOL_CACHE = {}


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _pool_task(task):
    b, hd, rows, sigma = task
    q, k, v = _POOL_INPUTS
    kh = kv_head(q.shape[2], k.shape[2], hd)
    key = (b, kh)
    if key not in _POOL_CACHE:
        _POOL_CACHE.clear()
        _POOL_CACHE[key] = (np.ascontiguousarray(k[b, :, kh, :], dtype=np.float64),
                            np.ascontiguousarray(v[b, :, kh, :], dtype=np.float64))
    Kh, Vh = _POOL_CACHE[key]
    Qh = np.asarray(q[b, rows, hd, :], dtype=np.float64)
    o, lse = _rows_one_head(Qh, Kh, Vh, sigma)
    return b, hd, rows, o, lse


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def attention_parallel(q, k, v, scale=None, rows_per_head=None, workers=None,
                       row_block: int = 256):
    """``attention`` over all heads, or over ``rows_per_head[(b, head)]``
    (an index array) for a sampled subset, run on ``workers`` processes
    (default: every host core this process may run on).

    Returns a dict ``{(b, head): (rows, O [n, D], lse [n])}``.
    """
    import multiprocessing as mp

    global _POOL_INPUTS
    B, S, h, D = q.shape
    sigma = _scale(D, scale)
    tasks = []
    for b in range(B):
        for hd in range(h):
            rows = (np.arange(S, dtype=np.int64) if rows_per_head is None
                    else np.asarray(rows_per_head[(b, hd)], dtype=np.int64))
            for r0 in range(0, len(rows), row_block):
                tasks.append((b, hd, rows[r0:r0 + row_block], sigma))
    workers = workers or host_cores()
    _POOL_INPUTS = (q, k, v)
    try:
        ctx = mp.get_context("fork")
        with ctx.Pool(processes=workers, initializer=_pool_init) as pool:
            results = pool.map(_pool_task, tasks, chunksize=1)
    finally:
        _POOL_INPUTS = None
    out = {}
    for b, hd, rows, o, lse in results:
        prev = out.get((b, hd))
        if prev is None:
            out[(b, hd)] = (rows, o, lse)
        else:
            out[(b, hd)] = (np.concatenate([prev[0], rows]), np.concatenate([prev[1], o]),
                            np.concatenate([prev[2], lse]))
    return out
