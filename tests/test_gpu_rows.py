"""GPU parity of the ragged token-row movements (scatter, gather,
reduce-scatter) against the float64 oracle.

Scatter and gather move bits: they are compared bit for bit on index-coded
tensors. The reduce-scatter adds P partials in rank order in fp32 and rounds
once: it is exact on integer-valued partials, and on random ones within the
error of that sum, |err| <= g(P-1) * sum_j |x_j| with g(n) = n u / (1 - n u),
u = 2^-24, plus for bf16 outputs the final rounding, 2^-8 of the magnitude."""
import numpy as np
import pytest

import ulysses_sequence_attention_amd as usp
from oracle import ranges as R
from oracle import relayout as X
from ulysses_sequence_attention_amd import synth

from gpu_util import coded, DEV, log, poisoned, to_dev, to_host, widen

pytestmark = pytest.mark.gpu
BF, F = synth.BF16, synth.F32


def _shards_like(B, S, W, P, dtype):
    tb = R.balanced_ranges(S, P)
    return [poisoned((B, tb[r + 1] - tb[r], W), dtype) for r in range(P)]


def _bits(a):
    return np.ascontiguousarray(a).tobytes()


@pytest.mark.parametrize("dtype", [BF, F])
@pytest.mark.parametrize("B,S,W,P", [(1, 8, 8, 1), (2, 257, 8, 3), (1, 1001, 64, 8), (3, 65, 16, 4)])
def test_scatter_gather_bit_exact(dtype, B, S, W, P):
    import torch
    if dtype == F and W % 4:
        pytest.skip("fp32 rows need W % 4 == 0")
    x = coded((B, S, W), dtype)
    log(f"rows scatter/gather {dtype} B={B} S={S} W={W} P={P}")
    shards = _shards_like(B, S, W, P, dtype)
    usp.usp_scatter_rows(to_dev(x, dtype), shards)
    torch.cuda.synchronize()
    for r in range(P):
        assert _bits(to_host(shards[r])) == _bits(X.scatter_sequence(x, P, r))
    full = poisoned((B, S, W), dtype)
    usp.usp_gather_rows(shards, full)
    torch.cuda.synchronize()
    assert _bits(to_host(full)) == _bits(X.gather_sequence([X.scatter_sequence(x, P, r)
                                                            for r in range(P)]))
    assert _bits(to_host(full)) == _bits(x)


def test_scatter_one_rank_touches_only_its_shard():
    import torch
    B, S, W, P = 2, 100, 8, 3
    x = coded((B, S, W), BF)
    log("rows scatter rank 1 of 3")
    shards = _shards_like(B, S, W, P, BF)
    usp.usp_scatter_rows(to_dev(x, BF), [None, shards[1], None], rank=1)
    torch.cuda.synchronize()
    assert _bits(to_host(shards[1])) == _bits(X.scatter_sequence(x, P, 1))
    for r in (0, 2):
        assert np.all(to_host(shards[r]) == 0xFFFF)


def _rs_bound(parts, dtype):
    P = len(parts)
    u = 2.0 ** -24
    g = (P - 1) * u / (1 - (P - 1) * u)
    mag = np.sum([np.abs(p) for p in parts], axis=0)
    exact = np.sum(parts, axis=0)
    bound = g * mag
    if dtype == BF:
        bound = bound + 2.0 ** -8 * (np.abs(exact) + bound)
    return bound


@pytest.mark.parametrize("dtype", [BF, F])
@pytest.mark.parametrize("B,S,W,P", [(1, 9, 8, 1), (2, 301, 8, 3), (1, 1000, 64, 8), (2, 70, 16, 5)])
def test_reduce_scatter(dtype, B, S, W, P):
    import torch
    if dtype == F and W % 4:
        pytest.skip("fp32 rows need W % 4 == 0")
    rng = np.random.default_rng(S + P)
    tb = R.balanced_ranges(S, P)
    log(f"rows reduce-scatter {dtype} B={B} S={S} W={W} P={P}")
    # integer-valued partials: every partial sum is exact in the dtype -> bit-exact
    ints = [rng.integers(-16, 17, size=(B, S, W)).astype(np.float32) for _ in range(P)]
    parts = [synth.f32_to_bf16_bits(p) if dtype == BF else p for p in ints]
    outs = _shards_like(B, S, W, P, dtype)
    usp.usp_reduce_scatter_rows([to_dev(p, dtype) for p in parts], outs)
    torch.cuda.synchronize()
    for r in range(P):
        ref = X.reduce_scatter_rows([widen(p, dtype) for p in parts], r)
        assert np.array_equal(widen(to_host(outs[r]), dtype), ref)
    # random partials: within the bound of the fp32 rank-order sum
    rnd = [rng.standard_normal((B, S, W)).astype(np.float32) for _ in range(P)]
    parts = [synth.f32_to_bf16_bits(p) if dtype == BF else p for p in rnd]
    wide = [widen(p, dtype) for p in parts]
    outs = _shards_like(B, S, W, P, dtype)
    usp.usp_reduce_scatter_rows([to_dev(p, dtype) for p in parts], outs)
    torch.cuda.synchronize()
    bound = _rs_bound(wide, dtype)
    for r in range(P):
        ref = X.reduce_scatter_rows(wide, r)
        got = widen(to_host(outs[r]), dtype)
        assert np.all(np.abs(got - ref) <= bound[:, tb[r]:tb[r + 1]]), r
    # one rank only
    one = [None] * P
    one[P - 1] = poisoned(outs[P - 1].shape, dtype)
    usp.usp_reduce_scatter_rows([to_dev(p, dtype) for p in parts], one, rank=P - 1)
    torch.cuda.synchronize()
    assert _bits(to_host(one[P - 1])) == _bits(to_host(outs[P - 1]))


def test_video_dit_boundary_full_size():
    """The model boundary of the video-DiT share: [1, 32760, 5120] bf16 rows
    (40 heads x 128) over 8 ranks: scatter and gather bit-exact, and the
    reduce-scatter of 8 partials on sampled rows."""
    import torch
    B, S, W, P = 1, 32760, 5120, 8
    tb = R.balanced_ranges(S, P)
    log("rows full size: scatter/gather [1, 32760, 5120] bf16, P=8")
    x = coded((B, S, W), BF)
    shards = _shards_like(B, S, W, P, BF)
    usp.usp_scatter_rows(to_dev(x, BF), shards)
    torch.cuda.synchronize()
    for r in range(P):
        assert _bits(to_host(shards[r])) == _bits(X.scatter_sequence(x, P, r))
    full = poisoned((B, S, W), BF)
    usp.usp_gather_rows(shards, full)
    torch.cuda.synchronize()
    assert _bits(to_host(full)) == _bits(x)
    del shards, full
    log("rows full size: reduce-scatter of 8 partials [1, 32760, 5120] bf16")
    parts = [synth.draw_rows(B, S, W, seed=70 + j) for j in range(P)]
    outs = _shards_like(B, S, W, P, BF)
    usp.usp_reduce_scatter_rows([to_dev(p, BF) for p in parts], outs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for r in range(P):
        rows = np.unique(np.concatenate([[0, tb[r + 1] - tb[r] - 1],
                                         rng.choice(tb[r + 1] - tb[r], 50, replace=False)]))
        wide = [widen(p[:, tb[r] + rows], BF) for p in parts]
        ref = np.sum(wide, axis=0)
        got = widen(to_host(outs[r])[:, rows], BF)
        assert np.all(np.abs(got - ref) <= _rs_bound(wide, BF))


def test_scatter_gather_beyond_one_launch():
    """[1, 17000003, 1024] bf16 (34.8 GB): more 16-byte chunks than one
    launch's 32-bit flat index, so the walk is split in two launches.
    Device-side full compare (shard r is rows [t_r, t_{r+1})), the gather
    round trip, and the oracle's scatter on sampled rows around the split."""
    import torch
    B, S, W, P = 1, 17_000_003, 1024, 3
    tb = R.balanced_ranges(S, P)
    torch.manual_seed(6)
    full = torch.randint(-32768, 32768, (B, S, W), dtype=torch.int16, device=DEV)
    shards = [torch.empty((B, tb[r + 1] - tb[r], W), dtype=torch.bfloat16, device=DEV)
              for r in range(P)]
    log(f"scatter beyond one launch S={S} W={W} P={P} (34.8 GB)")
    usp.usp_scatter_rows(full.view(torch.bfloat16), shards)
    torch.cuda.synchronize()
    for r in range(P):
        assert torch.equal(shards[r].view(torch.int16), full[:, tb[r]:tb[r + 1]]), f"shard {r}"
    # rows around the launch split (row 16777214) and the shard boundaries
    rows = np.array([0, 16777212, 16777213, 16777214, 16777215, tb[1] - 1, tb[1], tb[2], S - 1])
    for s in rows:
        r = int(np.searchsorted(tb, s, side="right") - 1)
        ref = X.scatter_sequence(full[:, s:s + 1].cpu().numpy(), 1, 0)
        got = shards[r][:, s - tb[r]:s - tb[r] + 1].view(torch.int16).cpu().numpy()
        assert got.tobytes() == ref.tobytes(), s
    back = torch.empty((B, S, W), dtype=torch.bfloat16, device=DEV)
    log("gather beyond one launch")
    usp.usp_gather_rows(shards, back)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), full)
    del full, shards, back
    torch.cuda.empty_cache()
