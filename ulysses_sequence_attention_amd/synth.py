"""Seeded synthetic inputs for the Ulysses sequence-parallel hot path.

This module only draws random tensors and converts their storage format. It
holds none of the method's arithmetic (no ranges, no relayout, no softmax), so
both the CPU oracle's tests and the HIP path's tests and benchmark may use it.

Recipe (same for every workload):
  * NumPy ``default_rng(seed)`` (PCG64), ``standard_normal`` drawn in float32,
    in the order Q, K, V, Q of the full ``[B, S, H, D]`` shape and K, V of
    ``[B, S, Hkv, D]`` (Hkv = H unless the workload groups K/V heads);
  * an optional per-tensor float32 multiplier (Q scaled by 1/sqrt(D) for the
    video-DiT share, all three scaled by 0.5 for the long chunked share);
  * for the "peaky" workload, after V is drawn: per batch row b = 0, 1, ...
    ``round(frac * S)`` distinct token indices from ``rng.choice`` without
    replacement, and K at those tokens (all heads) multiplied by 8;
  * bf16 workloads are rounded from float32 to bfloat16 with
    round-to-nearest-even on the host; both sides read the same bits.

The workload shapes stand in for the pages' model workloads (a ViT-L/16
encoder, a Wan-like video DiT with 21x40x39 latent tokens, a long sequence
with head-chunked passes); no dataset or weights are involved.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    """One seeded synthetic workload of the Ulysses hot path.

    B, S, H, D: batch, full sequence length, heads of the seq-sharded tensor,
    head dim. P: sequence-parallel degree (token ranges and head groups).
    chunks: number of head-chunk passes (1 = single shot). Hkv: heads of K
    and V (0: same as H); with Hkv < H, H / Hkv query heads share each.
    ring: ring blocks of the sequence for Ulysses+Ring (1: plain Ulysses);
    with ring = R the P ranks of each ring group split one ring block.
    """

    name: str
    B: int
    S: int
    H: int
    D: int
    P: int
    dtype: str
    seed: int
    q_mult: float = 1.0
    kv_mult: float = 1.0
    peaky_frac: float = 0.0
    chunks: int = 1
    Hkv: int = 0
    ring: int = 1

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def esize(self) -> int:
        return 4 if self.dtype == F32 else 2


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", B=1, S=257, H=6, D=64, P=3, dtype=F32, seed=1),
    "vit_l16": Workload("vit_l16", B=32, S=577, H=16, D=64, P=4, dtype=BF16, seed=2),
    "video_dit_share": Workload("video_dit_share", B=1, S=32760, H=40, D=128, P=8,
                                dtype=BF16, seed=3, q_mult=1.0 / math.sqrt(128.0)),
    "long_chunked": Workload("long_chunked", B=1, S=131072, H=8, D=128, P=1,
                             dtype=BF16, seed=4, q_mult=0.5, kv_mult=0.5, chunks=3),
    "indivisible_long": Workload("indivisible_long", B=2, S=65537, H=12, D=64, P=4,
                                 dtype=BF16, seed=5, peaky_frac=0.01),
    # grouped K/V heads: the video-DiT share with 8 K/V heads (5 query heads
    # per K/V head), and a smaller one that the oracle covers in full
    "gqa_video_share": Workload("gqa_video_share", B=1, S=32760, H=40, D=128, P=8,
                                dtype=BF16, seed=6, q_mult=1.0 / math.sqrt(128.0), Hkv=8),
    "gqa_small": Workload("gqa_small", B=2, S=1500, H=16, D=64, P=4, dtype=BF16, seed=7,
                          Hkv=4),
    # Ulysses+Ring: the video-DiT sequence on a 4 (Ulysses) x 2 (ring) grid
    # of 8 ranks, each rank holding 10 heads of a 16380-token ring block and
    # attending them to both ring blocks; and a small ragged one (ring
    # blocks 501/500/500, grouped K/V heads) that the oracle covers in full
    "video_dit_ring": Workload("video_dit_ring", B=1, S=32760, H=40, D=128, P=4, dtype=BF16,
                               seed=8, q_mult=1.0 / math.sqrt(128.0), ring=2),
    "ring_small": Workload("ring_small", B=2, S=1501, H=12, D=64, P=2, dtype=BF16, seed=9,
                           Hkv=4, ring=3),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits.

    Inputs are finite by construction (no NaN handling needed).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_qkv(B: int, S: int, H: int, D: int, seed: int, *, dtype: str = BF16,
             q_mult: float = 1.0, kv_mult: float = 1.0, peaky_frac: float = 0.0,
             hkv: int = 0):
    """Draw Q ``[B, S, H, D]`` and K, V ``[B, S, hkv or H, D]`` per the recipe
    above.

    Returns three arrays: float32 for ``dtype == "f32"``, uint16 bfloat16 bits
    for ``dtype == "bf16"``.
    """
    rng = np.random.default_rng(seed)
    kv_shape = (B, S, hkv or H, D)
    out = []
    for shape, mult in (((B, S, H, D), q_mult), (kv_shape, kv_mult), (kv_shape, kv_mult)):
        t = rng.standard_normal(shape, dtype=np.float32)
        if mult != 1.0:
            t *= np.float32(mult)
        out.append(t)
    if peaky_frac > 0.0:
        n = int(round(peaky_frac * S))
        for b in range(B):
            idx = rng.choice(S, size=n, replace=False)
            out[1][b, idx] *= np.float32(8.0)
    if dtype == BF16:
        out = [f32_to_bf16_bits(t) for t in out]
    return tuple(out)


def draw_rows(B: int, S: int, W: int, seed: int, dtype: str = BF16) -> np.ndarray:
    """One ``[B, S, W]`` tensor of token rows: ``default_rng(seed)``
    ``standard_normal`` in float32, rounded to bf16 (RNE) for bf16."""
    t = np.random.default_rng(seed).standard_normal((B, S, W), dtype=np.float32)
    return f32_to_bf16_bits(t) if dtype == BF16 else t


def draw_workload(w: Workload):
    """Q, K, V of a named workload at its full size."""
    return draw_qkv(w.B, w.S, w.H, w.D, w.seed, dtype=w.dtype, q_mult=w.q_mult,
                    kv_mult=w.kv_mult, peaky_frac=w.peaky_frac, hkv=w.Hkv)


def index_coded(shape, dtype: str) -> np.ndarray:
    """Tensor whose every element encodes its own flat index.

    f32: the index as float32 (exact below 2**24). bf16: ``index mod 65024``
    mapped one-to-one onto the uint16 patterns whose high byte is neither 0x7F
    nor 0xFF (so no Inf/NaN pattern occurs); a misplaced, missed or duplicated
    element is visible under a bitwise compare on tensors of up to 65024
    elements and, through the position pattern, almost surely on larger ones.
    """
    n = int(np.prod(shape))
    idx = np.arange(n, dtype=np.int64)
    if dtype == F32:
        if n >= (1 << 24):
            raise ValueError("index-coded f32 tensors must have < 2**24 elements")
        return idx.astype(np.float32).reshape(shape)
    return _finite_bf16_pattern(idx % 65024).reshape(shape)


def _finite_bf16_pattern(code: np.ndarray) -> np.ndarray:
    """Codes 0 .. 65023 one-to-one onto the uint16 patterns whose high byte
    is neither 0x7F nor 0xFF (no Inf/NaN pattern)."""
    code = np.asarray(code).astype(np.uint32)
    hi = code >> 8                              # 0 .. 253
    lo = code & 0xFF
    hi = np.where(hi >= 0x7F, hi + 1, hi)       # 0..0x7E, 0x80..0xFE
    return ((hi << 8) | lo).astype(np.uint16)


def random_coded(shape, dtype: str, seed: int) -> np.ndarray:
    """Tensor of independent random element codes (``default_rng(seed)``):
    bf16: uniform over the 65024 finite patterns of ``index_coded``; f32:
    integers below 2**24 as float32 (exact). Unlike ``index_coded`` nothing
    repeats with a period, so a block of elements moved to a wrong place
    differs from what belongs there with overwhelming probability, at any
    size (the bitwise relayout tests on full-size tensors use it)."""
    rng = np.random.default_rng(seed)
    if dtype == F32:
        return rng.integers(0, 1 << 24, size=shape).astype(np.float32)
    return _finite_bf16_pattern(rng.integers(0, 65024, size=shape))
