"""The seeded input generator against its published definition (SplitMix64,
Steele, Lea & Flood 2014) and against the distributions it claims."""
import numpy as np
import pytest
from scipy import stats

from host_memory_streamed_amd import synth

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _word(seed, stream, i):
    key = _mix(_mix(seed) ^ ((stream * 0xD1B54A32D192ED03) & M64))
    return _mix((key + (i + 1) * GAMMA) & M64)


def test_splitmix_reference_vector():
    # SplitMix64 seeded with 0 first outputs 0xE220A8397B1DCDAF; key(0, 0) is 0.
    assert int(synth.words(0, 0, 0, 1)[0]) == 0xE220A8397B1DCDAF


@pytest.mark.parametrize("seed,stream", [(0, 0), (1, 7), (12345, 1 << 40)])
def test_words_match_definition(seed, stream):
    w = synth.words(seed, stream, 1000, 16)
    assert [int(x) for x in w] == [_word(seed, stream, 1000 + i) for i in range(16)]


def test_normal_box_muller_definition():
    seed, stream = 3, 11
    x = synth.normal(seed, stream, (8,), 1.0)
    for j in range(4):
        w = _word(seed, stream, j)
        u1 = ((w >> 32) + 0.5) / 2**32
        u2 = ((w & 0xFFFFFFFF) + 0.5) / 2**32
        r = np.sqrt(-2 * np.log(u1))
        assert x[2 * j] == np.float32(r * np.cos(2 * np.pi * u2))
        assert x[2 * j + 1] == np.float32(r * np.sin(2 * np.pi * u2))


def test_normal_distribution_and_slices():
    x = synth.normal(0, 5, (400_000,), 0.02)
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 1e-4
    assert stats.kstest(x / 0.02, "norm").pvalue > 1e-3
    part = synth.normal(0, 5, (1001,), 0.02, offset=12345)
    assert np.array_equal(part, x[12345:12345 + 1001])


def test_tokens_uniform_and_shifted():
    tok, tgt = synth.token_batch(0, 4, 5000, 256)
    assert tok.dtype == np.int32 and tok.shape == (4, 5000)
    assert np.array_equal(tok[:, 1:], tgt[:, :-1])
    assert tok.min() >= 0 and tok.max() < 256
    counts = np.bincount(tok.ravel(), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-3
