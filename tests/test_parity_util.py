"""The comparator used by the parity tests can fail (CPU only)."""
import numpy as np
import pytest

from parity_util import assert_bitwise, differing_words


def test_one_changed_word_is_reported():
    a = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    b = a.copy()
    b.view(np.uint32)[417] ^= 1  # last mantissa bit of one word
    assert differing_words(a, b).tolist() == [417]
    with pytest.raises(AssertionError, match="1 of 1000 words differ"):
        assert_bitwise(a, b)


def test_signed_zero_and_nan_words_are_compared_as_words():
    assert differing_words(np.array([0.0], np.float32), np.array([-0.0], np.float32)).tolist() == [0]
    assert_bitwise(np.array([1.5, -2.0], np.float32), np.array([1.5, -2.0], np.float32))
