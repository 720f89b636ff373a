"""Pins of the oracle's mHC Sinkhorn normalisation (CPU): closed forms,
properties every Sinkhorn scaling has, and invariances of its limit."""
import numpy as np
import pytest

import oracle


def check_sinkhorn_closed_forms():
    # constant logits: the uniform matrix, at every iteration count
    for n in (2, 4, 8):
        for it in (0, 1, 10):
            assert np.allclose(oracle.mhc_sinkhorn(np.full((3, n, n), 0.7), it), 1.0 / n, rtol=0, atol=1e-15)
    # 2 x 2: the doubly-stochastic limit of A = [[a, b], [c, d]] is [[p, 1-p], [1-p, p]]
    # with p / (1 - p) = sqrt(ad / bc) (the cross ratio is invariant under row and column scaling)
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 2, 2))
    m = oracle.mhc_sinkhorn(l, 200)
    a = np.exp(l)
    r = np.sqrt(a[:, 0, 0] * a[:, 1, 1] / (a[:, 0, 1] * a[:, 1, 0]))
    p = r / (1 + r)
    assert np.allclose(m[:, 0, 0], p, rtol=1e-12) and np.allclose(m[:, 0, 1], 1 - p, rtol=1e-12)


def test_sinkhorn_closed_forms():
    check_sinkhorn_closed_forms()


def check_sinkhorn_properties():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((100, 4, 4)) * 2.0
    for it in (1, 3, 10):
        m = oracle.mhc_sinkhorn(l, it)
        assert np.all(m > 0)
        assert np.allclose(m.sum(-1), 1.0, rtol=0, atol=1e-14)            # each round ends with the rows
    # the columns converge to 1 (a doubly-stochastic matrix)
    err = [np.abs(oracle.mhc_sinkhorn(l, it).sum(-2) - 1).max() for it in (1, 5, 50, 1000)]
    assert err[0] > err[1] > err[2] > err[3] and err[3] < 1e-12
    # the limit is invariant under adding a constant to a row or a column of the logits
    lim = oracle.mhc_sinkhorn(l, 1000)
    shifted = l + rng.standard_normal((100, 1, 4)) + rng.standard_normal((100, 4, 1))
    assert np.allclose(oracle.mhc_sinkhorn(shifted, 1000), lim, rtol=1e-10, atol=1e-12)
    # large logits: no overflow (the row maximum is subtracted before exp), and
    # the result depends only on differences within a row
    big = l + 720.0
    assert np.allclose(oracle.mhc_sinkhorn(big, 10), oracle.mhc_sinkhorn(l, 10), rtol=1e-12, atol=0)


def test_sinkhorn_properties():
    check_sinkhorn_properties()


def test_sinkhorn_zero_rounds_is_row_softmax():
    l = np.random.default_rng(5).standard_normal((7, 4, 4))
    e = np.exp(l)
    assert np.allclose(oracle.mhc_sinkhorn(l, 0), e / e.sum(-1, keepdims=True), rtol=1e-14)
