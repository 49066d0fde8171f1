"""Helpers shared by the GPU parity tests (host <-> device marshalling, error
metrics). Not a test module."""
import sys

import numpy as np

from ulysses_sequence_attention_amd import synth

DEV = "cuda:0"


class no_pool:
    """Within the block, attention calls given no workspace run the key-group
    kernel instead of taking a workspace from the library's pool (the
    library reads USP_ATTENTION_POOL at every call)."""

    def __enter__(self):
        import os
        self._old = os.environ.get("USP_ATTENTION_POOL")
        os.environ["USP_ATTENTION_POOL"] = "0"
        return self

    def __exit__(self, *exc):
        import os
        if self._old is None:
            os.environ.pop("USP_ATTENTION_POOL", None)
        else:
            os.environ["USP_ATTENTION_POOL"] = self._old
        return False


def log(msg):
    """Name the case before each GPU step so a failing run says what it ran."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype):
    import torch
    if dtype == synth.BF16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(DEV)


def to_host(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def poisoned(shape, dtype):
    """Device tensor filled with a NaN pattern (bf16 0xFFFF / fp32 NaN)."""
    import torch
    if dtype == synth.BF16:
        return torch.full(shape, -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def widen(arr, dtype):
    """Stored values (bf16 bits or fp32) as float64."""
    if dtype == synth.BF16:
        return synth.bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def err(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = out - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


# Tolerances stated for the attention path: bf16 inputs (fp32 output
# epilogue) and the all-fp32 path.
BF16_MAX_ABS, BF16_REL_FROB = 1e-2, 5e-3
F32_MAX_ABS, F32_REL_FROB = 1e-5, 1e-5
# Natural-log normaliser of the bf16 path: the row sum is taken over the
# weights after their rounding to bf16 (8 significant bits, unit roundoff
# 2^-8), so the sum is within a relative 2^-8 of the exact one and its log
# within 2^-8 (plus fp32 accumulation error, well under 1e-5 at these
# lengths). Rows with few keys do not average the rounding out.
BF16_LSE_ABS = 2.0 ** -8 + 1e-5


def coded(shape, dtype, seed=0):
    """Input for the bitwise movement tests: ``index_coded`` (each element
    its own index) while no code repeats, random codes beyond that (the
    index code repeats every 65024 bf16 elements, so a shift by a multiple
    of that period would go unseen)."""
    n = int(np.prod(shape))
    if (dtype == synth.BF16 and n <= 65024) or (dtype == synth.F32 and n < (1 << 24)):
        return synth.index_coded(shape, dtype)
    return synth.random_coded(shape, dtype, seed)


def bf16_ulp(x):
    """One bf16 ulp at |x| (for grading the bf16-output epilogue)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)
