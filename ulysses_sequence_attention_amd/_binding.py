"""ctypes binding of libusp.so: argument marshalling only.

Every function has the name of the C entry point it calls (include/usp.h) and
takes PyTorch tensors for device buffers (PyTorch provides device memory and
streams; all work runs in the library's HIP kernels). Shapes become integer
arguments, dtypes the usp_dtype enum, tensors their data pointers, and the
stream defaults to PyTorch's current stream on the tensor's device. A
negative status raises ``UspError`` with the library's message.

The C ABI sees only pointers, so the binding checks what a pointer cannot
carry before any call: every tensor's shape against the others (and, for
block and shard lists, against the library's own balanced ranges), matching
dtypes, and that all tensors live on the same GPU; a mismatch raises
``ValueError`` instead of letting a kernel read or write past a buffer.

The library must have been built (``python -m ulysses_sequence_attention_amd.build``);
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libusp.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "usp.h")

USP_F32, USP_BF16 = 0, 1
STATUS = {0: "USP_OK", -1: "USP_EINVAL", -2: "USP_ESHAPE", -3: "USP_EDTYPE", -4: "USP_EALIGN",
          -5: "USP_ENOSYS", -6: "USP_EHIP"}
USP_MAX_PARTS = 64

_i32, _i64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class UspError(RuntimeError):
    def __init__(self, status: int, fn: str, message: str):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {message}")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libusp.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m ulysses_sequence_attention_amd.build`")
        # PyTorch ships its own HIP runtime (libamdhip64.so.7). Load it first so
        # libusp's dependency on that soname resolves to the same copy: one HIP
        # runtime per process. Loading libusp first would bring in the system
        # runtime and leave PyTorch running on a runtime it was not built for.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.usp_last_error.restype = ctypes.c_char_p
        L.usp_last_error.argtypes = []
        L.usp_version.restype = ctypes.c_char_p
        L.usp_version.argtypes = []
        L.usp_balanced_ranges.argtypes = [_i64, _i32, ctypes.POINTER(_i64)]
        L.usp_balanced_ranges_device.argtypes = [_i64, _i32, _vp, _vp]
        L.usp_head_chunk_ranges.argtypes = [_i32, _i32, ctypes.POINTER(_i32)]
        rel = [_vp, _vp, ctypes.c_int, _i64, _i64, _i32, _i32, _i32, _i32, _vp]
        L.usp_pack_seq_to_heads.argtypes = rel
        L.usp_unpack_heads_to_seq.argtypes = rel
        rel_chunk = rel[:-1] + [_i32, _i32, _vp]
        L.usp_pack_seq_to_heads_chunk.argtypes = rel_chunk
        rel_planes = [_i32, _vp, _vp, ctypes.c_int, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                      _vp]
        L.usp_pack_seq_to_heads_planes.argtypes = rel_planes
        L.usp_unpack_heads_to_seq_planes.argtypes = rel_planes
        L.usp_unpack_heads_to_seq_chunk.argtypes = rel_chunk
        L.usp_attention_fwd.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _i64,
                                        _i64, _i32, _i32, _i32, _i32, _f32, _vp, _vp]
        L.usp_attention_fwd_noalloc.argtypes = L.usp_attention_fwd.argtypes
        L.usp_attention_fwd_chunked.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                                _i64, _i64, _i32, _i32, _f32, _vp, _i32, _vp]
        L.usp_attention_fwd_chunked_ws.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                                   _i64, _i64, _i32, _i32, _f32, _vp, _i32, _vp,
                                                   ctypes.c_size_t, _vp]
        L.usp_attention_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64, _i32, _i32,
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.usp_attention_fwd_ws.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _i64,
                                           _i64, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                           ctypes.c_size_t, _vp]
        L.usp_attention_fwd_gqa.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _i64,
                                            _i64, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                            ctypes.c_size_t, _vp]
        L.usp_attention_fwd_block.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                              _i64, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                              _f32, _vp, _vp, ctypes.c_size_t, _vp]
        L.usp_attention_fwd_block_whole.argtypes = L.usp_attention_fwd_block.argtypes[:16] + [_vp]
        L.usp_attention_merge.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _i64, _i64,
                                          _i32, _i32, _i32, _i32, _vp]
        rows = [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _vp]
        L.usp_scatter_rows.argtypes = rows
        L.usp_reduce_scatter_rows.argtypes = rows
        L.usp_gather_rows.argtypes = [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i32, _vp]
        for name in ("usp_balanced_ranges", "usp_balanced_ranges_device", "usp_head_chunk_ranges",
                     "usp_pack_seq_to_heads", "usp_unpack_heads_to_seq", "usp_attention_fwd",
                     "usp_attention_fwd_chunked", "usp_attention_fwd_chunked_ws",
                     "usp_attention_workspace_bytes",
                     "usp_attention_fwd_ws", "usp_attention_fwd_gqa", "usp_attention_fwd_block",
                     "usp_attention_fwd_block_whole", "usp_attention_merge", "usp_scatter_rows",
                     "usp_gather_rows", "usp_reduce_scatter_rows"):
            getattr(L, name).restype = ctypes.c_int
        _LIB = L
    return _LIB


def header_symbols() -> list[str]:
    """Function names declared in include/usp.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(usp_\w+)\s*\(", text, re.M)))


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise UspError(status, fn, lib().usp_last_error().decode())


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return USP_F32
    if t.dtype == torch.bfloat16:
        return USP_BF16
    return 99  # rejected by the library with USP_EDTYPE


def _stream(t, stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _torch():
    import torch
    return torch


def _need(t, name, shape, dtypes=None):
    """Raise ValueError unless ``t`` has ``shape`` (and one of ``dtypes``)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")


def _on_gpu(named):
    """Raise ValueError unless every (name, tensor) in ``named`` that is not
    None is a GPU tensor on the first one's device (checked after shapes)."""
    ref = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if ref is None:
            ref = t
        elif t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {ref.device}")


def _dims(t, name, n):
    if t is None or t.dim() != n:
        raise ValueError(f"{name} must be a {n}-dimensional tensor")
    return tuple(t.shape)


def _attn_io(q, k, v, o, lse, ws=None, kv_rows=None, kv_heads=None):
    """Checks of q, o [B,S,h,D], k, v [B,kv_rows,kv_heads,D], lse [B,h,S]
    and the workspace's device."""
    torch = _torch()
    B, S, h, D = _dims(q, "q", 4)
    kr = S if kv_rows is None else kv_rows
    kh = h if kv_heads is None else kv_heads
    _need(k, "k", (B, kr, kh, D), (q.dtype,))
    _need(v, "v", (B, kr, kh, D), (q.dtype,))
    _need(o, "o", (B, S, h, D), (torch.float32, torch.bfloat16))
    if lse is not None:
        _need(lse, "lse", (B, h, S), (torch.float32,))
    _on_gpu([("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("ws", ws)])


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libusp must be contiguous")
    return t.data_ptr()


def usp_version() -> str:
    return lib().usp_version().decode()


def usp_last_error() -> str:
    return lib().usp_last_error().decode()


def usp_balanced_ranges(total: int, parts: int) -> list[int]:
    """Host boundaries [0, ..., total] of ``parts`` balanced ranges."""
    n = max(int(parts), 0) + 1
    buf = (_i64 * n)()
    _check(lib().usp_balanced_ranges(total, parts, buf), "usp_balanced_ranges")
    return list(buf)


def usp_balanced_ranges_device(total: int, parts: int, out, stream=None) -> None:
    """Boundaries into the device int64 tensor ``out`` (parts + 1 elements)."""
    if parts >= 1:
        _need(out, "out", (int(parts) + 1,), (_torch().int64,))
        _on_gpu([("out", out)])
    _check(lib().usp_balanced_ranges_device(total, parts, _ptr(out), _stream(out, stream)),
           "usp_balanced_ranges_device")


def usp_head_chunk_ranges(heads: int, chunks: int) -> list[int]:
    n = max(int(chunks), 0) + 1
    buf = (_i32 * n)()
    _check(lib().usp_head_chunk_ranges(heads, chunks, buf), "usp_head_chunk_ranges")
    return list(buf)


def _relayout_dims(seq, blocks, rank):
    B, L, H, D = _dims(seq, "seq", 4)
    P = len(blocks)
    if P < 1:
        return B, L, H, D
    S = _dims(blocks[0], "blocks[0]", 4)[1] if rank >= 0 else L
    # shapes are checked where the library would accept the sizes; otherwise
    # the call itself reports the error
    if 1 <= P <= min(H, USP_MAX_PARTS) and S >= P and rank < P:
        hb = usp_balanced_ranges(H, P)
        for j in range(P):
            _need(blocks[j], f"blocks[{j}]", (B, S, hb[j + 1] - hb[j], D), (seq.dtype,))
        rows = S
        if rank >= 0:
            tb = usp_balanced_ranges(S, P)
            rows = tb[rank + 1] - tb[rank]
        _need(seq, "seq", (B, rows, H, D))
        _on_gpu([("seq", seq)] + [(f"blocks[{j}]", blocks[j]) for j in range(P)])
    return B, S, H, D


def usp_pack_seq_to_heads(seq, blocks, rank: int = -1, stream=None) -> None:
    """seq [B,S,H,D] (world, rank < 0) or rank's shard [B,len_r,H,D] ->
    blocks[j] [B,S,h_j,D]; P = len(blocks)."""
    P = len(blocks)
    arr = (_vp * max(P, 1))(*[_ptr(b) for b in blocks])
    B, S, H, D = _relayout_dims(seq, blocks, rank)
    _check(lib().usp_pack_seq_to_heads(_ptr(seq), arr, _dtype(seq), B, S, H, D, P, rank,
                                       _stream(seq, stream)), "usp_pack_seq_to_heads")


def usp_unpack_heads_to_seq(blocks, seq, rank: int = -1, stream=None) -> None:
    """blocks[j] [B,S,h_j,D] -> seq [B,S,H,D] (world) or rank's shard."""
    P = len(blocks)
    arr = (_vp * max(P, 1))(*[_ptr(b) for b in blocks])
    B, S, H, D = _relayout_dims(seq, blocks, rank)
    _check(lib().usp_unpack_heads_to_seq(arr, _ptr(seq), _dtype(seq), B, S, H, D, P, rank,
                                         _stream(seq, stream)), "usp_unpack_heads_to_seq")


def usp_pack_seq_to_heads_chunk(seq, blocks, head_lo: int, head_hi: int, rank: int = -1,
                                stream=None) -> None:
    """One head-chunk phase of the pack: heads [head_lo, head_hi) of every
    (equal) group of seq [B,S,H,D] (world) or of rank's shard -> the same
    heads of blocks[j] [B,S,H/P,D]; nothing else is written."""
    P = len(blocks)
    arr = (_vp * max(P, 1))(*[_ptr(b) for b in blocks])
    B, S, H, D = _relayout_dims(seq, blocks, rank)
    _check(lib().usp_pack_seq_to_heads_chunk(_ptr(seq), arr, _dtype(seq), B, S, H, D, P, rank,
                                             head_lo, head_hi, _stream(seq, stream)),
           "usp_pack_seq_to_heads_chunk")


def usp_unpack_heads_to_seq_chunk(blocks, seq, head_lo: int, head_hi: int, rank: int = -1,
                                  stream=None) -> None:
    """One head-chunk phase of the unpack: heads [head_lo, head_hi) of every
    blocks[j] -> their place in seq (world) or in rank's shard."""
    P = len(blocks)
    arr = (_vp * max(P, 1))(*[_ptr(b) for b in blocks])
    B, S, H, D = _relayout_dims(seq, blocks, rank)
    _check(lib().usp_unpack_heads_to_seq_chunk(arr, _ptr(seq), _dtype(seq), B, S, H, D, P, rank,
                                               head_lo, head_hi, _stream(seq, stream)),
           "usp_unpack_heads_to_seq_chunk")


def _planes(seqs, blocks, rank):
    """Marshal n planes: the same checks as the single-plane calls for each
    plane, plus one shape and dtype for all (the kernel takes one geometry)."""
    n = len(seqs)
    if n != len(blocks) or n < 1:
        raise ValueError(f"{n} sequence tensors but {len(blocks)} block lists")
    P = len(blocks[0])
    dims = None
    for t in range(n):
        if len(blocks[t]) != P:
            raise ValueError("every plane needs the same number of blocks")
        d = _relayout_dims(seqs[t], blocks[t], rank)
        if dims is not None and (d != dims or seqs[t].dtype != seqs[0].dtype):
            raise ValueError(f"plane {t} has another shape or dtype than plane 0")
        dims = d
    sarr = (_vp * n)(*[_ptr(x) for x in seqs])
    barr = (_vp * max(n * P, 1))(*[_ptr(b) for bl in blocks for b in bl])
    return n, P, sarr, barr, dims


def usp_pack_seq_to_heads_planes(seqs, blocks, rank: int = -1, head_lo: int = 0, head_hi: int = 0,
                                 stream=None) -> None:
    """usp_pack_seq_to_heads (head_hi = 0) or its head-chunk phase for n
    tensors of one shape in one launch: seqs[t] -> blocks[t][j]."""
    n, P, sarr, barr, (B, S, H, D) = _planes(seqs, blocks, rank)
    _check(lib().usp_pack_seq_to_heads_planes(n, sarr, barr, _dtype(seqs[0]), B, S, H, D, P, rank,
                                              head_lo, head_hi, _stream(seqs[0], stream)),
           "usp_pack_seq_to_heads_planes")


def usp_unpack_heads_to_seq_planes(blocks, seqs, rank: int = -1, head_lo: int = 0,
                                   head_hi: int = 0, stream=None) -> None:
    """The inverse of usp_pack_seq_to_heads_planes: blocks[t][j] -> seqs[t]."""
    n, P, sarr, barr, (B, S, H, D) = _planes(seqs, blocks, rank)
    _check(lib().usp_unpack_heads_to_seq_planes(n, barr, sarr, _dtype(seqs[0]), B, S, H, D, P, rank,
                                                head_lo, head_hi, _stream(seqs[0], stream)),
           "usp_unpack_heads_to_seq_planes")


def _row_dims(full_like):
    if full_like is None or full_like.dim() < 2:
        raise ValueError("row tensors must have at least 2 dimensions [B, S, ...]")
    B, S = full_like.shape[0], full_like.shape[1]
    W = 1
    for n in full_like.shape[2:]:
        W *= n
    return B, S, W


def _check_shards(full_like, shards, which, name):
    """shards[r] must be [B, len_r, ...] for the ranks in ``which``."""
    B, S = full_like.shape[0], full_like.shape[1]
    P = len(shards)
    if not (1 <= P <= USP_MAX_PARTS and S >= P):
        return
    tb = usp_balanced_ranges(S, P)
    which = [r for r in which if 0 <= r < P]
    for r in which:
        _need(shards[r], f"{name}[{r}]", (B, tb[r + 1] - tb[r]) + tuple(full_like.shape[2:]),
              (full_like.dtype,))
    _on_gpu([("full", full_like)] + [(f"{name}[{r}]", shards[r]) for r in which])


def _ptr_array(tensors, P):
    return (_vp * max(P, 1))(*[_ptr(t) if t is not None else None for t in tensors])


def usp_scatter_rows(full, shards, rank: int = -1, stream=None) -> None:
    """full [B,S,...] -> shards[r] [B,len_r,...] for every rank (rank < 0) or
    for ``rank`` only (the other entries may be None)."""
    P = len(shards)
    B, S, W = _row_dims(full)
    _check_shards(full, shards, range(P) if rank < 0 else [rank], "shards")
    _check(lib().usp_scatter_rows(_ptr(full), _ptr_array(shards, P), _dtype(full), B, S, W, P,
                                  rank, _stream(full, stream)), "usp_scatter_rows")


def usp_gather_rows(shards, full, stream=None) -> None:
    """shards[r] [B,len_r,...] -> full [B,S,...] in rank order."""
    P = len(shards)
    B, S, W = _row_dims(full)
    _check_shards(full, shards, range(P), "shards")
    _check(lib().usp_gather_rows(_ptr_array(shards, P), _ptr(full), _dtype(full), B, S, W, P,
                                 _stream(full, stream)), "usp_gather_rows")


def usp_reduce_scatter_rows(partials, out, rank: int = -1, stream=None) -> None:
    """out[r] = rank r's rows of sum(partials) (P partials [B,S,...]), for
    every rank (rank < 0) or ``rank`` only."""
    P = len(partials)
    B, S, W = _row_dims(partials[0])
    for j in range(P):
        _need(partials[j], f"partials[{j}]", tuple(partials[0].shape), (partials[0].dtype,))
    _check_shards(partials[0], out, range(P) if rank < 0 else [rank], "out")
    _on_gpu([(f"partials[{j}]", partials[j]) for j in range(P)])
    _check(lib().usp_reduce_scatter_rows(_ptr_array(partials, P), _ptr_array(out, P),
                                         _dtype(partials[0]), B, S, W, P, rank,
                                         _stream(partials[0], stream)), "usp_reduce_scatter_rows")


def usp_attention_fwd(q, k, v, o, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                      lse=None, stream=None) -> None:
    """Attention over heads [head_lo, head_hi) of q, k, v, o [B,S,h,D]; a
    workspace, where the shape needs one, comes from the library's
    stream-ordered pool (USP_ATTENTION_POOL=0 in the environment: none)."""
    _attn_io(q, k, v, o, lse)
    B, S, h, D = q.shape
    hi = h if head_hi is None else head_hi
    _check(lib().usp_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q), _dtype(o), B, S,
                                   h, D, head_lo, hi, scale, _ptr(lse), _stream(q, stream)),
           "usp_attention_fwd")


def usp_attention_fwd_noalloc(q, k, v, o, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                              lse=None, stream=None) -> None:
    """usp_attention_fwd_ws with the library's static scratch as workspace
    (no allocation; calls that overlap on one GPU race)."""
    _attn_io(q, k, v, o, lse)
    B, S, h, D = q.shape
    hi = h if head_hi is None else head_hi
    _check(lib().usp_attention_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q), _dtype(o),
                                           B, S, h, D, head_lo, hi, scale, _ptr(lse),
                                           _stream(q, stream)), "usp_attention_fwd_noalloc")


def usp_attention_workspace_bytes(in_dtype: int, B: int, S: int, heads: int, D: int) -> int:
    """Workspace bytes usp_attention_fwd_ws needs (``in_dtype``: USP_F32 or USP_BF16)."""
    out = ctypes.c_size_t(0)
    _check(lib().usp_attention_workspace_bytes(in_dtype, B, S, heads, D, ctypes.byref(out)),
           "usp_attention_workspace_bytes")
    return out.value


def usp_attention_fwd_ws(q, k, v, o, ws, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                         lse=None, stream=None) -> None:
    """usp_attention_fwd with the caller's workspace tensor ``ws`` (any dtype;
    its byte size is passed; None for fp32 inputs)."""
    _attn_io(q, k, v, o, lse, ws)
    B, S, h, D = q.shape
    hi = h if head_hi is None else head_hi
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().usp_attention_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q), _dtype(o), B,
                                      S, h, D, head_lo, hi, scale, _ptr(lse), _ptr(ws), nbytes,
                                      _stream(q, stream)), "usp_attention_fwd_ws")


def usp_attention_fwd_gqa(q, k, v, o, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                          lse=None, ws=None, stream=None) -> None:
    """Attention over query heads [head_lo, head_hi) of q, o [B,S,h,D] with
    k, v [B,S,h_kv,D] (query head n uses K/V head n // (h // h_kv));
    ``ws`` an optional workspace tensor as for usp_attention_fwd_ws."""
    _attn_io(q, k, v, o, lse, ws, kv_heads=_dims(k, "k", 4)[2])
    B, S, h, D = q.shape
    hi = h if head_hi is None else head_hi
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().usp_attention_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q), _dtype(o), B,
                                       S, h, k.shape[2], D, head_lo, hi, scale, _ptr(lse), _ptr(ws),
                                       nbytes, _stream(q, stream)), "usp_attention_fwd_gqa")


def usp_attention_fwd_block(q, k, v, o, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                            lse=None, ws=None, stream=None) -> None:
    """Attention of the query block q, o [B,Sq,h,D] against the key/value
    block k, v [B,Sk,h_kv,D] for query heads [head_lo, head_hi); ``lse``
    fp32 [B,h,Sq] or None; ``ws`` an optional workspace tensor sized for
    Sq query rows."""
    kd = _dims(k, "k", 4)
    _attn_io(q, k, v, o, lse, ws, kv_rows=kd[1], kv_heads=kd[2])
    B, Sq, h, D = q.shape
    hi = h if head_hi is None else head_hi
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().usp_attention_fwd_block(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q), _dtype(o),
                                         B, Sq, k.shape[1], h, k.shape[2], D, head_lo, hi, scale,
                                         _ptr(lse), _ptr(ws), nbytes, _stream(q, stream)),
           "usp_attention_fwd_block")


def usp_attention_fwd_block_whole(q, k, v, o, head_lo: int = 0, head_hi=None, scale: float = 0.0,
                                  lse=None, stream=None) -> None:
    """usp_attention_fwd_block with every query row's keys walked in one pass
    (no workspace): for the key blocks of a ring pass run on separate
    streams at the same time."""
    kd = _dims(k, "k", 4)
    _attn_io(q, k, v, o, lse, None, kv_rows=kd[1], kv_heads=kd[2])
    B, Sq, h, D = q.shape
    hi = h if head_hi is None else head_hi
    _check(lib().usp_attention_fwd_block_whole(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q),
                                               _dtype(o), B, Sq, k.shape[1], h, k.shape[2], D,
                                               head_lo, hi, scale, _ptr(lse), _stream(q, stream)),
           "usp_attention_fwd_block_whole")


def usp_attention_merge(o_a, lse_a, o_b, lse_b, o, lse=None, head_lo: int = 0, head_hi=None,
                        stream=None) -> None:
    """Log-sum-exp merge of (o_a, lse_a) and (o_b, lse_b) — fp32 [B,S,h,D]
    and [B,h,S] — into o (fp32 or bf16; may be o_a itself when fp32) and
    lse (may be lse_a itself, or None)."""
    torch = _torch()
    B, S, h, D = _dims(o_a, "o_a", 4)
    _need(o_a, "o_a", (B, S, h, D), (torch.float32,))
    _need(o_b, "o_b", (B, S, h, D), (torch.float32,))
    _need(lse_a, "lse_a", (B, h, S), (torch.float32,))
    _need(lse_b, "lse_b", (B, h, S), (torch.float32,))
    _need(o, "o", (B, S, h, D), (torch.float32, torch.bfloat16))
    if lse is not None:
        _need(lse, "lse", (B, h, S), (torch.float32,))
    _on_gpu([("o_a", o_a), ("lse_a", lse_a), ("o_b", o_b), ("lse_b", lse_b), ("o", o),
             ("lse", lse)])
    hi = h if head_hi is None else head_hi
    _check(lib().usp_attention_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o),
                                     _ptr(lse), _dtype(o), B, S, h, D, head_lo, hi,
                                     _stream(o_a, stream)), "usp_attention_merge")


def usp_attention_fwd_chunked(q, k, v, o, chunks: int, scale: float = 0.0, lse=None,
                              stream=None) -> None:
    """Attention as ``chunks`` head-chunk passes (bitwise equal to single shot)."""
    _attn_io(q, k, v, o, lse)
    B, S, h, D = q.shape
    _check(lib().usp_attention_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q),
                                           _dtype(o), B, S, h, D, scale, _ptr(lse), chunks,
                                           _stream(q, stream)), "usp_attention_fwd_chunked")


def usp_attention_fwd_chunked_ws(q, k, v, o, chunks: int, ws, scale: float = 0.0, lse=None,
                                 stream=None) -> None:
    """usp_attention_fwd_chunked with the caller's workspace tensor ``ws``
    (sized for ceil(h / chunks) heads; None for fp32 inputs)."""
    _attn_io(q, k, v, o, lse, ws)
    B, S, h, D = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().usp_attention_fwd_chunked_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _dtype(q),
                                              _dtype(o), B, S, h, D, scale, _ptr(lse), chunks,
                                              _ptr(ws), nbytes, _stream(q, stream)),
           "usp_attention_fwd_chunked_ws")
