"""Ulysses+Ring: attention over key blocks merged by log-sum-exp (oracle;
test infrastructure).

maxdiffusion PR #428 (description, and the review thread on it) applies the
head-chunked Ulysses passes to a "Ulysses+Ring" layout as well, whose ring
half the pages do not describe. Reading taken here (the plainest one that
the rest supports): the P ranks form a U x R grid. The sequence is cut into
R ring blocks by the balanced ranges; ring group r (U ranks) runs Ulysses on
its block, so after the first all-to-all rank (r, j) holds q, k, v
[B, S_r, h_j, D] for head group j (balanced ranges over the heads with U
parts). The ring then brings rank (r, j) the K/V blocks of the other ring
groups for the same head group, and the rank attends its query block to each
one in turn. Attention over the whole sequence is attention over the union
of the ring blocks' keys, so it is recovered exactly from the per-block
results by the log-sum-exp merge below.

Merge (a statement of softmax over a union of key sets): for a query row
with per-block outputs O_a, O_b and natural-log normalisers lse_a, lse_b
(lse = log sum_t exp(sigma * <q, k_t>) over the block's keys),

    lse = log(exp(lse_a) + exp(lse_b))
    O   = exp(lse_a - lse) * O_a + exp(lse_b - lse) * O_b

since block a holds the fraction exp(lse_a - lse) of the row's total weight
and O_a is that block's weight-normalised sum of values.
"""
from __future__ import annotations

import numpy as np

from . import relayout
from .attention import attention
from .ranges import balanced_ranges, head_chunk_ranges


def merge(o_a, lse_a, o_b, lse_b):
    """Log-sum-exp merge of two block results (float64).

    ``o_* [B, S, h, D]``, ``lse_* [B, h, S]``; returns ``(O, lse)`` of the
    union of the two blocks' keys. ``lse = -inf`` (a block with no keys)
    gives that block weight 0; a row with no keys in either block has no
    softmax at all and is given O = 0, lse = -inf."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    none = np.isneginf(m)                     # no keys in either block
    ms = np.where(none, 0.0, m)
    wa = np.exp(lse_a - ms)                   # exp(-inf) = 0 for an empty block
    wb = np.exp(lse_b - ms)
    lse = np.where(none, -np.inf, ms + np.log(np.where(none, 1.0, wa + wb)))
    ls = np.where(none, 0.0, lse)
    fa = np.where(none, 0.0, np.exp(lse_a - ls))
    fb = np.where(none, 0.0, np.exp(lse_b - ls))
    # weights per (b, head, row), laid out for o's [B, S, h, D]
    fa = fa.transpose(0, 2, 1)[..., None]
    fb = fb.transpose(0, 2, 1)[..., None]
    return fa * o_a + fb * o_b, lse


def ring_order(r: int, R: int):
    """Order in which ring member r meets the K/V blocks: its own block, then
    the block of r - 1, r - 2, ... (mod R) as the ring passes them on."""
    return [(r - i) % R for i in range(R)]


def ring_attention(q, kv_blocks, scale=None, order=None):
    """Attention of the query block ``q [B, Sq, h, D]`` over the keys of
    every block in ``kv_blocks = [(k_i [B, S_i, hkv, D], v_i), ...]``, one
    block at a time, folded with :func:`merge` in ``order`` (default: list
    order). Returns ``(O [B, Sq, h, D], lse [B, h, Sq])`` in float64."""
    order = list(range(len(kv_blocks))) if order is None else list(order)
    o = lse = None
    for i in order:
        k_i, v_i = kv_blocks[i]
        o_i, lse_i = attention(q, k_i, v_i, scale=scale, return_lse=True)
        if o is None:
            o, lse = o_i, lse_i
        else:
            o, lse = merge(o, lse, o_i, lse_i)
    return o, lse


def ulysses_ring_world(q, k, v, U: int, R: int, scale=None):
    """The U x R Ulysses+Ring composition on world layouts: ring blocks of
    the sequence by balanced ranges; inside ring block r, pack (U parts) ->
    for each head group j, ring attention of block r's queries over all R
    blocks' keys of group j (order :func:`ring_order`) -> unpack. Returns
    ``O [B, S, H, D]`` float64. With grouped K/V heads U has to divide
    H and Hkv."""
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    if Hkv != H and (H % U or Hkv % U or H % Hkv):
        raise ValueError(f"grouped heads: U ({U}) has to divide H ({H}) and Hkv ({Hkv})")
    T = balanced_ranges(S, R)
    # ring group r's Ulysses blocks: qb[r][j] = [B, S_r, h_j, D]
    qb = [relayout.pack_seq_to_heads(q[:, T[r]:T[r + 1]], U) for r in range(R)]
    kb = [relayout.pack_seq_to_heads(k[:, T[r]:T[r + 1]], U) for r in range(R)]
    vb = [relayout.pack_seq_to_heads(v[:, T[r]:T[r + 1]], U) for r in range(R)]
    out = np.empty((B, S, H, D), dtype=np.float64)
    for r in range(R):
        ob = []
        for j in range(U):
            blocks = [(kb[i][j], vb[i][j]) for i in range(R)]
            o, _ = ring_attention(qb[r][j], blocks, scale=scale, order=ring_order(r, R))
            ob.append(o)
        out[:, T[r]:T[r + 1]] = relayout.unpack_heads_to_seq(ob, H)
    return out


def ulysses_ring_two_phase_world(q, k, v, U: int, R: int, chunks: int, scale=None):
    """:func:`ulysses_ring_world` with the Ulysses exchange in head-chunk
    phases (maxdiffusion PR #428 applies its chunking to Ulysses+Ring too):
    for each chunk ``[lo, hi)`` of the plan over a Ulysses group's K/V heads
    (hkv = Hkv / U; query heads ``[lo G, hi G)``, G = H / Hkv), in turn: pack
    those heads of every ring block, run every rank's ring pass on them,
    unpack them. Needs U to divide H and Hkv. Returns ``O [B, S, H, D]``."""
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    if H % Hkv or H % U or Hkv % U:
        raise ValueError(f"head chunks need equal head groups: U ({U}) has to divide H ({H}) "
                         f"and Hkv ({Hkv}), and Hkv has to divide H")
    G, h, hkv = H // Hkv, H // U, Hkv // U
    T = balanced_ranges(S, R)
    L = [T[r + 1] - T[r] for r in range(R)]
    x64 = [np.asarray(x, dtype=np.float64) for x in (q, k, v)]
    qb = [[np.zeros((B, L[r], h, D)) for _ in range(U)] for r in range(R)]
    kb = [[np.zeros((B, L[r], hkv, D)) for _ in range(U)] for r in range(R)]
    vb = [[np.zeros((B, L[r], hkv, D)) for _ in range(U)] for r in range(R)]
    ob = [[np.zeros((B, L[r], h, D)) for _ in range(U)] for r in range(R)]
    out = np.zeros((B, S, H, D), dtype=np.float64)
    kc = head_chunk_ranges(hkv, chunks)
    for c in range(chunks):
        lo, hi = kc[c], kc[c + 1]
        for r in range(R):
            rows = slice(T[r], T[r + 1])
            relayout.pack_heads_chunk(x64[0][:, rows], qb[r], L[r], lo * G, hi * G)
            relayout.pack_heads_chunk(x64[1][:, rows], kb[r], L[r], lo, hi)
            relayout.pack_heads_chunk(x64[2][:, rows], vb[r], L[r], lo, hi)
        for r in range(R):
            for j in range(U):
                blocks = [(kb[i][j][:, :, lo:hi], vb[i][j][:, :, lo:hi]) for i in range(R)]
                o, _ = ring_attention(qb[r][j][:, :, lo * G:hi * G], blocks, scale=scale,
                                      order=ring_order(r, R))
                ob[r][j][:, :, lo * G:hi * G] = o
        for r in range(R):
            relayout.unpack_heads_chunk(ob[r], out[:, T[r]:T[r + 1]], L[r], lo * G, hi * G)
    return out
