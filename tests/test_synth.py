"""The seeded input generators (no method arithmetic): finite bf16 patterns,
reproducible draws."""
import numpy as np

from ulysses_sequence_attention_amd import synth


def _finite_bf16(bits):
    hi = bits >> 8
    return not np.any((hi == 0x7F) | (hi == 0xFF))


def test_index_coded_is_one_to_one_below_its_period():
    x = synth.index_coded((65024,), synth.BF16)
    assert len(np.unique(x)) == 65024 and _finite_bf16(x)
    y = synth.index_coded((3, 70000), synth.BF16)
    assert np.array_equal(y.reshape(-1)[65024:65024 + 100], x[:100])  # the period


def test_random_coded_is_finite_reproducible_and_aperiodic():
    a = synth.random_coded((4, 50000), synth.BF16, seed=5)
    assert a.dtype == np.uint16 and _finite_bf16(a)
    assert np.array_equal(a, synth.random_coded((4, 50000), synth.BF16, seed=5))
    assert not np.array_equal(a, synth.random_coded((4, 50000), synth.BF16, seed=6))
    flat = a.reshape(-1)
    # no period: a shift by the index code's period (or a row) changes most elements
    assert np.mean(flat[65024:] == flat[:-65024]) < 0.01
    f = synth.random_coded((1000,), synth.F32, seed=1)
    assert f.dtype == np.float32 and np.all(f == np.round(f)) and np.all((f >= 0) & (f < 2 ** 24))
