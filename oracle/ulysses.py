"""The Ulysses composition and head-chunked passes (oracle; test infrastructure).

m-star ``sequence_parallel`` module description / ``ulysses_attention``: the
first all-to-all makes each rank hold the full sequence over its head group,
attention runs locally, the second all-to-all returns to the sequence shard;
the result is the attention of the unsharded tensor. maxdiffusion PR #428
description: the head-chunked two-phase variant runs the exchange plus
attention over head sub-groups in turn; since no head's attention reads
another head's data, it gives exactly the single-shot result.
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
