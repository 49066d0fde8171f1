"""The Ulysses composition and head-chunked passes (oracle; test infrastructure).

m-star ``sequence_parallel`` module description / ``ulysses_attention``: the
first all-to-all makes each rank hold the full sequence over its head group,
attention runs locally, the second all-to-all returns to the sequence shard;
the result is the attention of the unsharded tensor. maxdiffusion PR #428
description: the head-chunked two-phase variant runs the exchange plus
attention over head sub-groups in turn; since no head's attention reads
another head's data, it gives exactly the single-shot result. Both forms are
here: ``attention_chunked`` (the passes over one block) and
``ulysses_two_phase_world`` (the exchange itself in per-chunk phases).
"""
from __future__ import annotations

import numpy as np

from . import relayout
from .attention import attention, kv_head
from .ranges import head_chunk_ranges


def ulysses_world(q, k, v, P: int, scale=None, attn=attention):
    """pack q, k, v -> ``attn`` on each head-group block -> unpack.

    ``attn`` maps ``(q_blk, k_blk, v_blk) -> o_blk`` for one block
    ``[B, S, h_j, D]``; it defaults to the oracle attention (a layout-only
    mock such as ``lambda q, k, v: v`` isolates the relayouts). With grouped
    K/V heads (k, v ``[B, S, Hkv, D]``, Hkv < H) P has to divide H and Hkv,
    so that block j's query heads share block j's K/V heads
    (m-star ``ulysses_attention``)."""
    H, Hkv = q.shape[2], k.shape[2]
    if Hkv != H and (H % P or Hkv % P or H % Hkv):
        raise ValueError(f"grouped heads: P ({P}) has to divide H ({H}) and Hkv ({Hkv})")
    qb = relayout.pack_seq_to_heads(q, P)
    kb = relayout.pack_seq_to_heads(k, P)
    vb = relayout.pack_seq_to_heads(v, P)
    if attn is attention:
        ob = [attention(qb[j], kb[j], vb[j], scale=scale) for j in range(P)]
    else:
        ob = [attn(qb[j], kb[j], vb[j]) for j in range(P)]
    return relayout.unpack_heads_to_seq(ob, H)


def ulysses_two_phase_world(q, k, v, P: int, chunks: int, scale=None, attn=attention):
    """The head-chunked two-phase exchange on world layouts (maxdiffusion PR
    #428 description): for each chunk ``[k_c, k_{c+1})`` of the plan over a
    group's K/V heads, in turn, pack those heads of k and v and their query
    heads of q into the head blocks, run ``attn`` on those heads of every
    block, and unpack them from the output blocks. Returns ``O [B, S, H, D]``.

    Needs equal head groups (P divides H and Hkv). With grouped K/V heads (G =
    H / Hkv query heads per K/V head) the plan runs over the hkv = Hkv / P K/V
    heads of a group and chunk ``[lo, hi)`` carries query heads ``[lo G, hi
    G)``, so no chunk splits the query heads of one K/V head; with G = 1 it is
    the plan over the group's H / P heads."""
    B, S, H, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or Hkv < 1 or H % Hkv:
        raise ValueError("the two-phase composition takes q [B,S,H,D] and k, v [B,S,Hkv,D] "
                         "with Hkv dividing H")
    if H % P or Hkv % P:
        raise ValueError(f"head chunks need equal head groups: P ({P}) has to divide H ({H}) "
                         f"and Hkv ({Hkv})")
    G, h, hkv = H // Hkv, H // P, Hkv // P
    kc = head_chunk_ranges(hkv, chunks)
    qb, ob = ([np.zeros((B, S, h, D), dtype=np.float64) for _ in range(P)] for _ in range(2))
    kb, vb = ([np.zeros((B, S, hkv, D), dtype=np.float64) for _ in range(P)] for _ in range(2))
    out = np.zeros((B, S, H, D), dtype=np.float64)
    for c in range(chunks):
        lo, hi = kc[c], kc[c + 1]
        relayout.pack_heads_chunk(np.asarray(q, dtype=np.float64), qb, S, lo * G, hi * G)
        for x, xb in ((k, kb), (v, vb)):
            relayout.pack_heads_chunk(np.asarray(x, dtype=np.float64), xb, S, lo, hi)
        for j in range(P):
            part = (qb[j][:, :, lo * G:hi * G], kb[j][:, :, lo:hi], vb[j][:, :, lo:hi])
            ob[j][:, :, lo * G:hi * G] = (attention(*part, scale=scale) if attn is attention
                                          else attn(*part))
        relayout.unpack_heads_chunk(ob, out, S, lo * G, hi * G)
    return out


def attention_chunked(q, k, v, chunks: int, scale=None):
    """Attention of ``q [B, S, h, D]`` run as ``chunks`` head-chunk passes,
    each pass over query heads ``[k_c, k_{c+1})`` of the plan, assembled side
    by side. With grouped K/V heads a pass need not start on a group
    boundary: each query head takes its own K/V head."""
    h, hkv = q.shape[2], k.shape[2]
    hb = head_chunk_ranges(h, chunks)
    out = np.empty(q.shape, dtype=np.float64)
    for c in range(chunks):
        for n in range(hb[c], hb[c + 1]):
            j = kv_head(h, hkv, n)
            out[:, :, n:n + 1, :] = attention(q[:, :, n:n + 1, :], k[:, :, j:j + 1, :],
                                              v[:, :, j:j + 1, :], scale=scale)
    return out
