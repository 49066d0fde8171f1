"""usp_attention_fwd_noalloc (the key-half workspace in the library's static
scratch) against usp_attention_fwd_ws with a caller workspace: the same
kernels, so every output bit must agree. Two calls in a row on one GPU, the
second smaller, both through the C ABI (the binding only marshals)."""
import numpy as np
import pytest

import ulysses_sequence_attention_amd as usp
from ulysses_sequence_attention_amd import synth

from gpu_util import DEV, log, poisoned, to_dev, to_host

pytestmark = pytest.mark.gpu

# (B, S, h, head range, D, output dtype, seed): the first call leaves its
# state in the scratch, the second (fewer rows, other D) must not see it
CASES = [
    (1, 4099, 5, (0, 5), 128, synth.BF16, 71),
    (2, 700, 4, (1, 3), 64, synth.F32, 72),
]


def _run(B, S, h, lohi, D, odt, seed):
    import torch
    lo, hi = lohi
    q, k, v = synth.draw_qkv(B, S, h, D, seed=seed)
    qd, kd, vd = (to_dev(x, synth.BF16) for x in (q, k, v))
    o_ref, o_na = poisoned((B, S, h, D), odt), poisoned((B, S, h, D), odt)
    l_ref = torch.full((B, h, S), float("nan"), device=DEV)
    l_na = torch.full((B, h, S), float("nan"), device=DEV)
    ws = torch.empty(usp.usp_attention_workspace_bytes(usp.USP_BF16, B, S, hi - lo, D),
                     dtype=torch.uint8, device=DEV)
    log(f"noalloc B={B} S={S} h={h} heads [{lo},{hi}) D={D} out={'bf16' if odt == synth.BF16 else 'f32'}")
    usp.usp_attention_fwd_ws(qd, kd, vd, o_ref, ws, head_lo=lo, head_hi=hi, lse=l_ref)
    usp.usp_attention_fwd_noalloc(qd, kd, vd, o_na, head_lo=lo, head_hi=hi, lse=l_na)
    torch.cuda.synchronize()
    a, b = to_host(o_ref), to_host(o_na)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "outputs differ"
    la, lb = to_host(l_ref), to_host(l_na)
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), "lse differs"
    # heads outside the range stay poisoned
    assert np.all(np.isnan(synth.bf16_bits_to_f32(b) if odt == synth.BF16 else b)[:, :, :lo])
    assert np.all(np.isnan(synth.bf16_bits_to_f32(b) if odt == synth.BF16 else b)[:, :, hi:])


def test_noalloc_matches_workspace_twice():
    for case in CASES:
        _run(*case)


def test_noalloc_rejects_beyond_scratch():
    import torch
    # 2 x 16384 rows x 8 heads at D = 128 need 268 MB > 192 MiB of scratch
    q = torch.empty((2, 16384, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(usp.UspError, match="scratch"):
        usp.usp_attention_fwd_noalloc(q, q, q, q)
