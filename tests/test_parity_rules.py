"""The comparison rules themselves (no GPU): they accept the reference and
reject errors just beyond the stated bounds."""
import numpy as np
import pytest

from parity import check_bitexact, check_tolerance, sample_indices


def test_bitexact_folds_zero_sign_only():
    a = np.array([0.0, 1.0, -2.5], np.float16)
    check_bitexact(np.array([-0.0, 1.0, -2.5], np.float16), a)
    with pytest.raises(AssertionError):
        check_bitexact(np.array([0.0, np.nextafter(np.float16(1), np.float16(2)), -2.5],
                                np.float16), a)


def test_tolerance_bounds():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(10000).astype(np.float16)
    check_tolerance(ref, ref)
    bad = ref.copy()
    i = int(np.argmax(np.abs(ref)))
    bad[i] = np.float16(float(ref[i]) * 1.01)            # 1% on the largest element
    with pytest.raises(AssertionError):
        check_tolerance(bad, ref)
    drift = (ref.astype(np.float64) * (1 + 1.5e-3)).astype(np.float16)  # uniform 0.15%
    with pytest.raises(AssertionError, match="Frobenius"):
        check_tolerance(drift, ref)


def test_tolerance_requires_matching_infinities():
    ref = np.array([np.inf, 1.0], np.float16)
    check_tolerance(np.array([np.inf, 1.0], np.float16), ref)
    with pytest.raises(AssertionError):
        check_tolerance(np.array([65504.0, 1.0], np.float16), ref)


def test_sample_indices_cover_tails():
    r, c = sample_indices(100, 70, 50)
    assert r.max() == 99 and c.max() == 69 and r.min() == 0 and c.min() == 0
    assert np.any((r == 99) & (c == 69))
