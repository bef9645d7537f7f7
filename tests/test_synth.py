"""The seeded input generator (no operation arithmetic; CPU only)."""
import numpy as np

import synth


def test_philox_matches_numpy():
    # numpy.random.Philox is Philox4x64-10 and increments its counter before
    # producing a block, so its k-th block is ours at counter k.
    key = np.array([42, 0x301], dtype=np.uint64)
    bg = np.random.Philox(key=key, counter=np.array([0, 7, 0, 0], dtype=np.uint64))
    raw = bg.random_raw(12)
    for blk in range(3):
        ours = synth.philox4x64_10([blk + 1, 7, 0, 0], key)
        np.testing.assert_array_equal(ours, raw[4 * blk:4 * blk + 4])


def test_thread_count_and_slicing_invariance():
    a = synth.generate(300_001, synth.OUTLIER_REPLACE, 5, 1e-3, 0.001, 10.0, threads=1)
    b = synth.generate(300_001, synth.OUTLIER_REPLACE, 5, 1e-3, 0.001, 10.0, threads=7)
    np.testing.assert_array_equal(a, b)
    c = synth.generate(1001, synth.OUTLIER_REPLACE, 5, 1e-3, 0.001, 10.0, offset=123_457)
    np.testing.assert_array_equal(c, a[123_457:124_458])


def test_distributions_have_the_stated_shape():
    n = 1 << 20
    z = synth.generate(n, synth.NORMAL, 11, 0.02)
    assert abs(z.std() / 0.02 - 1) < 0.01 and abs(z.mean()) < 1e-4
    h = synth.generate(n, synth.HALF_NORMAL, 12, 1e-6)
    assert (h >= 0).all() and abs(h.mean() / (1e-6 * np.sqrt(2 / np.pi)) - 1) < 0.01
    o = synth.generate(n, synth.OUTLIER_SCALED, 13, 1e-3, 0.01, 1e4)
    frac = (np.abs(o) > 0.1).mean()  # scaled entries are ~N(0,10)
    assert 0.008 < frac < 0.011
    r = synth.generate(n, synth.OUTLIER_REPLACE, 14, 1e-3, 0.001, 10.0)
    assert 0.0008 < (np.abs(r) > 0.05).mean() < 0.0011
    t = synth.generate(n, synth.STUDENT_T3, 15, 1e-2)
    # t(3): heavy tails; P(|T| > 5) ~ 1.5%.
    assert 0.012 < (np.abs(t) > 0.05).mean() < 0.018
