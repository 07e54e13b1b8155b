"""The seeded input generator: deterministic, sliceable, unit variance."""
import numpy as np

import synth
from synth import configs


def test_words_are_sliceable_and_deterministic():
    a = synth.words(7, 3, 0, 1000)
    b = synth.words(7, 3, 400, 100)
    np.testing.assert_array_equal(a[400:500], b)
    np.testing.assert_array_equal(synth.words(7, 3, 0, 10), a[:10])
    assert not np.array_equal(synth.words(8, 3, 0, 10), a[:10])
    assert not np.array_equal(synth.words(7, 4, 0, 10), a[:10])


def test_first_word_matches_scalar_definition():
    # scalar SplitMix64 finaliser applied to base + (i + 1) * gamma
    base = synth.stream_base(11, 5)
    for i in (0, 1, 12345):
        z = (base + (i + 1) * synth.GAMMA) & synth.MASK64
        assert int(synth.words(11, 5, i, 1)[0]) == synth._mix_int(z)


def test_normal_moments_and_bounds():
    v = synth.normal(1, 2, 0, 1 << 20)
    assert abs(v.mean()) < 5e-3
    assert abs(v.var() - 1.0) < 5e-3
    assert np.abs(v).max() <= 3.4642
    vb = synth.normal(1, 2, 0, 1 << 12, bf16=True)
    bits = vb.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                       # bf16-representable
    np.testing.assert_allclose(vb, v[: 1 << 12], rtol=2 ** -8)


def test_bf16_rounding_ties_to_even():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)
    r = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    np.testing.assert_array_equal(r, np.array([1.0, 1 + 2 ** -6, -1.0], dtype=np.float32))


def test_presets_shapes():
    p = configs.cfg2()
    assert p.n_chunks == 16384 and p.n_docs == 2048 and p.layers == 18
    p = configs.cfg4()
    assert p.n_chunks == 1_562_496
    assert p.n_chunks * p.layers * p.H * p.d * 2 == 57_599_852_544
    p3 = configs.cfg3()
    assert p3.lengths.sum() == 10_000_000
    assert p3.lengths.min() >= 1 and p3.lengths.max() <= 8192
    assert 150_000 < p3.n_chunks < 175_000
    assert p3.max_doc_chunks == 128
    assert configs.cfg1().n_chunks == 512


def test_needles_are_distinct_and_seeded():
    a = synth.needle_docs(5, 1000, 8)
    assert len(set(a.tolist())) == 8
    np.testing.assert_array_equal(a, synth.needle_docs(5, 1000, 8))
