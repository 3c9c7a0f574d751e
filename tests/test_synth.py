"""The seeded input generator: determinism, stream separation, value recipes."""
import numpy as np

import synth


def test_same_seed_same_bits():
    a = synth.codes(3, 64, 1024)
    b = synth.codes(3, 64, 1024)
    assert np.array_equal(a, b)
    assert np.array_equal(synth.scales(3, 64, 1024), synth.scales(3, 64, 1024))
    assert np.array_equal(synth.activations(3, 4, 1024), synth.activations(3, 4, 1024))


def test_streams_differ():
    assert not np.array_equal(synth.codes(3, 8, 256), synth.codes(4, 8, 256))
    assert not np.array_equal(synth.codes(3, 8, 256, seed=1), synth.codes(3, 8, 256))


def test_prefix_property_and_threading():
    """Element i depends only on (seed, stream, i): a longer draw extends a shorter one."""
    small = synth.activations(9, 1, 512)
    big = synth.activations(9, 2, 512 * 300)  # large enough to use several threads
    assert np.array_equal(small[0], big[0, :512])
    c1 = synth.codes(9, 1, 1024)
    c2 = synth.codes(9, 4096, 1024)
    assert np.array_equal(c1[0], c2[0])


def test_value_recipes():
    c = synth.codes(5, 2048, 1024)
    nib = np.concatenate([(c & 0xF).ravel(), (c >> 4).ravel()])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * nib.size / 16 and counts.max() < 1.1 * nib.size / 16
    s = synth.bf16_to_f32(synth.scales(5, 2048, 1024)).astype(np.float64)
    assert s.min() >= 1e-3 * (1 - 2**-8) and abs(s.mean() - (0.02 * np.sqrt(2 / np.pi) + 1e-3)) < 2e-4
    x = synth.bf16_to_f32(synth.activations(5, 8, 65536)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01


def test_bf16_round_to_nearest_even():
    f = synth.bf16_from_double
    assert f(1.0) == 0x3F80 and f(-2.0) == 0xC000 and f(0.0) == 0 and f(-0.0) == 0x8000
    assert f(1.0 + 2.0**-8) == 0x3F80           # tie -> even (down)
    assert f(1.0 + 3 * 2.0**-8) == 0x3F82       # tie -> even (up)
    assert f(1.0 + 2.0**-8 + 2.0**-30) == 0x3F81  # above the tie -> up
    assert f(128.0) == 0x4300 and f(-136.0) == 0xC308


def test_distinct_ids():
    ids = synth.distinct_ids(7, 32768, 248320)
    assert ids.dtype == np.int32 and ids.size == 32768
    assert np.unique(ids).size == 32768 and ids.min() >= 0 and ids.max() < 248320
    assert np.array_equal(ids, synth.distinct_ids(7, 32768, 248320))
    assert not np.all(np.diff(ids) > 0)  # kept in draw order, not sorted
    full = synth.distinct_ids(8, 50, 50)
    assert sorted(full.tolist()) == list(range(50))


def test_weight_rows_equal_rows_of_the_full_weight():
    """The range form of the generator gives the same bits as the whole
    tensor, at any row (stream positions not a multiple of 8 included)."""
    N, K = 300, 1152
    p, s = synth.weight(77, N, K)
    rows = np.array([0, 1, 7, 8, 150, 298, 299])
    pr, sr = synth.weight_rows(77, rows, K)
    assert np.array_equal(pr, p[rows]) and np.array_equal(sr, s[rows])
