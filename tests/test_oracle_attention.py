"""Pins for the oracle's attention and the Ulysses composition (CPU only).

Each check is independent of the oracle's own formula: brute-force loops,
PyTorch's CPU scaled_dot_product_attention in float64, closed forms for
special inputs, and invariants of softmax attention."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import ulysses as U


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("B,S,h,D,seed", [(1, 1, 1, 1, 0), (1, 5, 2, 3, 1), (2, 9, 1, 4, 2),
                                          (1, 8, 3, 2, 3)])
def test_matches_bruteforce(B, S, h, D, seed):
    q, k, v = (_rand((B, S, h, D), seed + i) for i in range(3))
    ref = A.attention_bruteforce(q, k, v)
    out = A.attention(q, k, v, row_block=3)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("B,S,h,D,scale", [(2, 100, 3, 16, None), (1, 257, 2, 64, None),
                                           (1, 70, 1, 8, 0.3), (3, 33, 2, 5, 2.0)])
def test_matches_torch_sdpa(B, S, h, D, scale):
    rng = np.random.default_rng(S + D)
    q, k, v = (rng.standard_normal((B, S, h, D)) for _ in range(3))
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    out = A.attention(q, k, v, scale=scale)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_single_key_returns_v():
    q, k, v = (_rand((2, 1, 3, 5), i) for i in range(3))
    assert np.array_equal(A.attention(q, k, v), v)


def test_equal_keys_give_mean_of_v():
    S, D = 11, 4
    q = _rand((1, S, 1, D), 1)
    k = np.repeat(_rand((1, 1, 1, D), 2), S, axis=1)
    v = _rand((1, S, 1, D), 3)
    out = A.attention(q, k, v)
    assert np.max(np.abs(out - v.mean(axis=1, keepdims=True))) <= 1e-13


def test_constant_v_is_reproduced():
    q, k = _rand((1, 13, 2, 6), 1, 3.0), _rand((1, 13, 2, 6), 2, 3.0)
    v = np.full((1, 13, 2, 6), -2.75)
    assert np.max(np.abs(A.attention(q, k, v) + 2.75)) <= 1e-14


@pytest.mark.parametrize("scale", [None, 0.7])
def test_two_keys_logistic(scale):
    # two keys: weight of key 0 = logistic(sigma * (q.k0 - q.k1))
    D = 6
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 1, D))
    k = rng.standard_normal((1, 2, 1, D))
    v = rng.standard_normal((1, 2, 1, D))
    sigma = 1 / math.sqrt(D) if scale is None else scale
    out = A.attention(q, k, v, scale=scale)
    for s in range(2):
        a = sigma * (q[0, s, 0] @ k[0, 0, 0] - q[0, s, 0] @ k[0, 1, 0])
        w0 = 1.0 / (1.0 + math.exp(-a))
        expect = w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0]
        assert np.max(np.abs(out[0, s, 0] - expect)) <= 1e-14


def test_key_permutation_invariance():
    q, k, v = (_rand((2, 17, 2, 5), i) for i in range(3))
    perm = np.random.default_rng(9).permutation(17)
    a = A.attention(q, k, v)
    b = A.attention(q, k[:, perm], v[:, perm])
    assert np.max(np.abs(a - b)) <= 1e-13


def test_rows_are_probabilities():
    # V = identity basis makes O the softmax matrix itself
    S = 12
    q = _rand((1, S, 1, S), 1, 2.0)
    k = _rand((1, S, 1, S), 2, 2.0)
    v = np.eye(S).reshape(1, S, 1, S)
    p = A.attention(q, k, v)[0, :, 0, :]
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12


def test_huge_logits_are_one_hot():
    # scores in the thousands: exp without the max shift would overflow
    S, D = 6, 2
    k = np.zeros((1, S, 1, D)); k[0, :, 0, 0] = np.arange(S) * 1000.0
    q = np.zeros((1, S, 1, D)); q[0, :, 0, 0] = 1.0
    v = _rand((1, S, 1, D), 4)
    out = A.attention(q, k, v, scale=1.0)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out[0, :, 0] - v[0, S - 1, 0])) <= 1e-14


def test_lse_closed_form():
    # all scores equal x -> lse = x + log(S)
    S, D = 9, 3
    q = np.ones((1, S, 1, D)); k = np.ones((1, S, 1, D)) * 0.5
    v = _rand((1, S, 1, D), 1)
    _, lse = A.attention(q, k, v, scale=2.0, return_lse=True)
    assert np.max(np.abs(lse[0, 0, :] - (2.0 * 1.5 + math.log(S)))) <= 1e-13


def test_linear_in_v():
    q, k, v1, v2 = (_rand((1, 20, 2, 4), i) for i in range(4))
    a = A.attention(q, k, 2.0 * v1 - 3.0 * v2)
    b = 2.0 * A.attention(q, k, v1) - 3.0 * A.attention(q, k, v2)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_rows_and_parallel_agree_with_full():
    q, k, v = (_rand((2, 300, 2, 8), i) for i in range(3))
    full, lse = A.attention(q, k, v, return_lse=True)
    rows = np.array([0, 5, 299, 150])
    o, l = A.attention_rows(q, k, v, 1, 1, rows)
    assert np.max(np.abs(o - full[1, rows, 1])) <= 1e-13
    assert np.max(np.abs(l - lse[1, 1, rows])) <= 1e-13
    par = A.attention_parallel(q, k, v, workers=2, row_block=64)
    for (b, hd), (r, o2, l2) in par.items():
        assert np.max(np.abs(o2 - full[b, r, hd])) <= 1e-13
        assert np.max(np.abs(l2 - lse[b, hd, r])) <= 1e-13


@pytest.mark.parametrize("B,S,H,D,P", [(1, 10, 6, 4, 3), (2, 9, 7, 3, 3), (1, 13, 4, 2, 4),
                                       (1, 8, 2, 4, 1)])
def test_ulysses_equals_single_device(B, S, H, D, P):
    q, k, v = (_rand((B, S, H, D), i) for i in range(3))
    direct = A.attention(q, k, v)
    uly = U.ulysses_world(q, k, v, P)
    assert np.array_equal(uly, direct)


def test_identity_mock_roundtrip():
    q, k, v = (_rand((2, 9, 7, 3), i) for i in range(3))
    out = U.ulysses_world(q, k, v, 3, attn=lambda a, b, c: c)
    assert np.array_equal(out, v)


@pytest.mark.parametrize("h", [1, 3, 8])
def test_chunked_equals_single_shot(h):
    q, k, v = (_rand((1, 21, h, 4), i) for i in range(3))
    ref = A.attention(q, k, v)
    for chunks in range(1, h + 1):
        try:
            out = U.attention_chunked(q, k, v, chunks)
        except ValueError:
            continue
        assert np.array_equal(out, ref)


@pytest.mark.parametrize("B,S,H,D,P,chunks", [(1, 10, 6, 4, 3, 2), (2, 9, 15, 3, 3, 3),
                                              (1, 13, 16, 2, 2, 3), (1, 8, 3, 4, 1, 2)])
def test_two_phase_exchange_equals_single_shot(B, S, H, D, P, chunks):
    # the head-chunked exchange (per-chunk pack -> attention -> unpack) gives
    # the single-shot Ulysses result bit for bit and the single-device result
    q, k, v = (_rand((B, S, H, D), i + 20) for i in range(3))
    out = U.ulysses_two_phase_world(q, k, v, P, chunks)
    assert np.array_equal(out, U.ulysses_world(q, k, v, P))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_two_phase_identity_mock_and_errors():
    q, k, v = (_rand((2, 9, 12, 3), i) for i in range(3))
    for chunks in (1, 2, 4):                   # groups of 4 heads: 4, 2/2, 1/1/1/1
        out = U.ulysses_two_phase_world(q, k, v, 3, chunks, attn=lambda a, b, c: c)
        assert np.array_equal(out, v)
    out = U.ulysses_two_phase_world(q, k, v, 3, 2, attn=lambda a, b, c: a + 2 * c)
    assert np.array_equal(out, q + 2 * v)      # elementwise mock: every head back in place
    with pytest.raises(ValueError, match="equal head groups"):
        U.ulysses_two_phase_world(*(_rand((1, 5, 7, 2), i) for i in range(3)), 3, 1)
    with pytest.raises(ValueError, match="Hkv dividing H"):
        U.ulysses_two_phase_world(q, k[:, :, :5], v[:, :, :5], 3, 1)
    with pytest.raises(ValueError, match="equal head groups"):          # Hkv = 4 over P = 3
        U.ulysses_two_phase_world(q, k[:, :, :4], v[:, :, :4], 3, 1)


@pytest.mark.parametrize("B,S,H,Hkv,D,P,chunks", [(1, 11, 12, 6, 4, 3, 2), (2, 9, 20, 10, 3, 2, 3),
                                                  (1, 7, 8, 2, 2, 2, 1), (1, 10, 6, 3, 4, 1, 2)])
def test_two_phase_grouped_heads(B, S, H, Hkv, D, P, chunks):
    # chunks over each group's K/V heads, each with its G query heads: the
    # grouped single-shot result exactly, and SDPA with enable_gqa
    q = _rand((B, S, H, D), 30)
    k, v = (_rand((B, S, Hkv, D), 31 + i) for i in range(2))
    out = U.ulysses_two_phase_world(q, k, v, P, chunks)
    assert np.array_equal(out, U.ulysses_world(q, k, v, P))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v)),
        enable_gqa=True).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


# ---- grouped K/V heads (Hkv < Hq): query head n uses K/V head n // (Hq / Hkv)

@pytest.mark.parametrize("B,S,h,hkv,D,seed", [(1, 5, 4, 2, 3, 7), (2, 7, 6, 1, 2, 8),
                                              (1, 6, 6, 3, 4, 9)])
def test_grouped_matches_bruteforce(B, S, h, hkv, D, seed):
    q = _rand((B, S, h, D), seed)
    k, v = (_rand((B, S, hkv, D), seed + i) for i in (1, 2))
    assert np.max(np.abs(A.attention(q, k, v, row_block=4) - A.attention_bruteforce(q, k, v))) <= 1e-12


@pytest.mark.parametrize("B,S,h,hkv,D", [(2, 90, 8, 2, 16), (1, 257, 6, 3, 64), (1, 40, 5, 1, 8)])
def test_grouped_matches_torch_sdpa(B, S, h, hkv, D):
    # torch's enable_gqa repeats each K/V head for consecutive query heads
    rng = np.random.default_rng(S + h)
    q = rng.standard_normal((B, S, h, D))
    k, v = (rng.standard_normal((B, S, hkv, D)) for _ in range(2))
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(A.attention(q, k, v) - ref)) <= 1e-12


def test_grouped_is_attention_over_repeated_heads():
    q = _rand((1, 33, 6, 5), 1)
    k, v = (_rand((1, 33, 2, 5), i) for i in (2, 3))
    rep = A.attention(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2))
    assert np.array_equal(A.attention(q, k, v), rep)
    # the other plausible convention (head n with K/V head n mod Hkv) differs
    tiled = A.attention(q, np.tile(k, (1, 1, 3, 1)), np.tile(v, (1, 1, 3, 1)))
    assert np.max(np.abs(tiled - rep)) > 1e-3


def test_grouped_rows_and_parallel_agree_with_full():
    q = _rand((2, 50, 4, 8), 4)
    k, v = (_rand((2, 50, 2, 8), i) for i in (5, 6))
    full, lse = A.attention(q, k, v, return_lse=True)
    o, ls = A.attention_rows(q, k, v, 1, 3, [0, 7, 49])
    assert np.max(np.abs(o - full[1, [0, 7, 49], 3])) <= 1e-13
    par = A.attention_parallel(q, k, v, workers=2)
    for (b, hd), (rows, o, ls) in par.items():
        assert np.max(np.abs(o - full[b, rows, hd])) <= 1e-13
        assert np.max(np.abs(ls - lse[b, hd, rows])) <= 1e-13


@pytest.mark.parametrize("B,S,H,Hkv,D,P", [(1, 10, 8, 4, 4, 4), (2, 9, 6, 2, 3, 2), (1, 12, 4, 4, 2, 2)])
def test_grouped_ulysses_equals_single_device(B, S, H, Hkv, D, P):
    q = _rand((B, S, H, D), 1)
    k, v = (_rand((B, S, Hkv, D), i) for i in (2, 3))
    assert np.array_equal(U.ulysses_world(q, k, v, P), A.attention(q, k, v))


def test_grouped_ulysses_needs_divisible_heads():
    q = _rand((1, 8, 6, 2), 1)
    k, v = (_rand((1, 8, 2, 2), i) for i in (2, 3))
    with pytest.raises(ValueError):
        U.ulysses_world(q, k, v, 4)  # 6 and 2 heads over 4 ranks
    with pytest.raises(ValueError):
        A.kv_head(6, 4, 0)


def test_grouped_chunks_across_group_boundaries():
    # 8 query heads over 2 K/V heads in 3 passes (3/3/2): the middle pass
    # holds query heads 3-5, i.e. both K/V heads
    q = _rand((1, 21, 8, 4), 1)
    k, v = (_rand((1, 21, 2, 4), i) for i in (2, 3))
    assert np.array_equal(U.attention_chunked(q, k, v, 3), A.attention(q, k, v))
