"""MI355X-native hot path of Ulysses sequence-parallel attention.

One rank's share of the work behind a small C ABI (``include/usp.h``,
``libusp.so``, hand-written HIP kernels for gfx950):

  * ``usp_balanced_ranges`` / ``usp_head_chunk_ranges`` — ragged contiguous
    token and head ranges, head-chunk plans;
  * ``usp_pack_seq_to_heads`` / ``usp_unpack_heads_to_seq`` — the
    sequence-sharded <-> head-sharded relayouts around the all-to-alls, and
    their ``_chunk`` forms, one head chunk per phase of the two-phase exchange,
    and ``_planes`` forms moving several tensors (q, k, v) in one launch;
  * ``usp_scatter_rows`` / ``usp_gather_rows`` / ``usp_reduce_scatter_rows``
    — ragged token rows at the model boundary;
  * ``usp_attention_fwd`` / ``usp_attention_fwd_chunked`` (``_ws``) — flash-style
    non-causal attention over the full sequence for a head group (a
    workspace, where needed, from the library's stream-ordered pool);
    ``usp_attention_fwd_ws`` the same with a caller workspace (same kernels,
    same bits), sized by ``usp_attention_workspace_bytes``;
    ``usp_attention_fwd_noalloc`` the same with the library's static scratch
    (for callers that cannot allocate); ``usp_attention_fwd_gqa`` with
    grouped key/value heads;
  * ``usp_attention_fwd_block`` / ``usp_attention_merge`` — a query block
    against one key/value block with its log-sum-exp, and the merge of such
    results: one ring step of Ulysses+Ring attention;
    ``usp_attention_fwd_block_whole`` the block call with whole key walks,
    for ring blocks run on separate streams at once.

The Python functions of the same names only marshal arguments (PyTorch
tensors for device memory, PyTorch streams); ``synth`` draws seeded inputs.
"""
from ._binding import (  # noqa: F401
    USP_BF16, USP_F32, USP_MAX_PARTS, UspError, header_symbols, lib, usp_attention_fwd,
    usp_attention_fwd_block, usp_attention_fwd_block_whole, usp_attention_fwd_chunked, usp_attention_fwd_chunked_ws,
    usp_attention_fwd_gqa, usp_attention_fwd_noalloc,
    usp_attention_fwd_ws, usp_attention_merge,
    usp_attention_workspace_bytes,
    usp_balanced_ranges, usp_balanced_ranges_device,
    usp_gather_rows, usp_head_chunk_ranges, usp_last_error, usp_pack_seq_to_heads,
    usp_pack_seq_to_heads_chunk, usp_pack_seq_to_heads_planes, usp_reduce_scatter_rows,
    usp_scatter_rows, usp_unpack_heads_to_seq, usp_unpack_heads_to_seq_chunk,
    usp_unpack_heads_to_seq_planes, usp_version)
