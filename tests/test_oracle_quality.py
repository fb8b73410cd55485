"""Pins for the synthetic quality report's measures (oracle/quality.py): the
relative squared error, the softmax, the KL divergence and the greedy
agreement, against hand-worked values and scipy's own routines (no GPU)."""
import numpy as np
import pytest
import scipy.special

from oracle import quality as Q


def test_relative_sq_error_hand_values():
    w = np.array([3.0, 4.0], np.float32)
    assert Q.relative_sq_error(w, w) == 0.0
    assert Q.relative_sq_error(w, np.array([3.0, 0.0])) == pytest.approx(16.0 / 25.0, abs=0)
    assert Q.relative_sq_error(w, np.array([0.0, 0.0])) == 1.0
    assert Q.relative_sq_error(w, np.array([6.0, 8.0])) == 1.0          # (w - 2w)^2 / w^2
    # sign of the difference does not matter; the denominator is the reference's
    assert Q.relative_sq_error(np.array([2.0]), np.array([1.0])) == 0.25
    assert Q.relative_sq_error(np.array([1.0]), np.array([2.0])) == 1.0


def test_softmax64():
    p = Q.softmax64(np.array([0.0, np.log(3.0)]))
    assert np.allclose(p, [0.25, 0.75], rtol=1e-15)
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000) * 4
    assert abs(Q.softmax64(x).sum() - 1.0) < 1e-13
    assert np.allclose(Q.softmax64(x + 123.0), Q.softmax64(x), rtol=1e-12)
    assert np.allclose(Q.softmax64(x.astype(np.float32)), scipy.special.softmax(x.astype(np.float32).astype(np.float64)),
                       rtol=1e-12)


def test_kl_divergence():
    # hand-made pair: p = (1/4, 3/4), q = (1/2, 1/2)
    a = np.array([0.0, np.log(3.0)])
    b = np.array([5.0, 5.0])
    want = 0.25 * np.log(0.5) + 0.75 * np.log(1.5)
    assert Q.kl_divergence(a, b) == pytest.approx(want, rel=1e-13)
    assert Q.kl_divergence(a, b) == pytest.approx(scipy.special.rel_entr([0.25, 0.75], [0.5, 0.5]).sum(), rel=1e-13)
    # random pairs against scipy; zero for identical inputs; not symmetric
    rng = np.random.default_rng(1)
    for _ in range(20):
        x, y = rng.standard_normal(500) * 3, rng.standard_normal(500) * 3
        ref = scipy.special.rel_entr(scipy.special.softmax(x), scipy.special.softmax(y)).sum()
        assert Q.kl_divergence(x, y) == pytest.approx(ref, rel=1e-10)
        assert Q.kl_divergence(x, y) > 0
        assert Q.kl_divergence(x, x) == 0.0
    assert Q.kl_divergence(a, b) != pytest.approx(Q.kl_divergence(b, a), rel=1e-3)
    # a reference probability that underflows to 0 contributes 0
    assert np.isfinite(Q.kl_divergence(np.array([0.0, -1e4]), np.array([0.0, 0.0])))


def test_greedy_agreement():
    a = list(range(64))
    assert Q.greedy_agreement(a, a) == 1.0
    b = a[:32] + [-1] * 32
    assert Q.greedy_agreement(a, b) == 0.5
    assert Q.greedy_agreement([7] * 64, [8] * 64) == 0.0
    # only the first n positions count
    assert Q.greedy_agreement(a + [1, 2], a + [3, 4], n=64) == 1.0
    assert Q.greedy_agreement([1, 2, 3, 4], [1, 9, 3, 9], n=4) == 0.5
    with pytest.raises(ValueError):
        Q.greedy_agreement(a[:10], a[:10], n=64)
