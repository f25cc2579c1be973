"""Pins for the oracle's low-rank predictor (CPU only).

DejaVu Guide, "Mathematical Formulation of Lookahead Predictors": scores are a
linear map of the predictor input; stored here as two bias-free factors.
"""
import numpy as np
import pytest

import oracle


def loops_predict(p1, p2, x):
    r, d = len(p1), len(p1[0])
    n = len(p2)
    z = [sum(p1[i][c] * x[c] for c in range(d)) for i in range(r)]
    return [sum(p2[j][i] * z[i] for i in range(r)) for j in range(n)]


def make(rng, d=7, r=3, F=11, H=4, B=2):
    return (rng.standard_normal((r, d)), rng.standard_normal((F, r)),
            rng.standard_normal((r, d)), rng.standard_normal((H, r)),
            rng.standard_normal((B, d)))


def test_brute_force_loops():
    rng = np.random.default_rng(0)
    p1m, p2m, p1h, p2h, x = make(rng)
    sm, sh = oracle.predict(p1m, p2m, p1h, p2h, x)
    for b in range(x.shape[0]):
        np.testing.assert_allclose(sm[b], loops_predict(p1m.tolist(), p2m.tolist(), x[b].tolist()),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sh[b], loops_predict(p1h.tolist(), p2h.tolist(), x[b].tolist()),
                                   rtol=1e-12, atol=1e-12)


def test_associativity_single_projection():
    """x . (P1^T P2^T) is the same single linear projection."""
    rng = np.random.default_rng(1)
    p1m, p2m, p1h, p2h, x = make(rng, d=64, r=16, F=200, H=12, B=3)
    sm, sh = oracle.predict(p1m, p2m, p1h, p2h, x)
    np.testing.assert_allclose(sm, x @ (p1m.T @ p2m.T), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(sh, x @ (p1h.T @ p2h.T), rtol=1e-10, atol=1e-10)


def test_identity_first_factor():
    rng = np.random.default_rng(2)
    d = 9
    p2 = rng.standard_normal((13, d))
    x = rng.standard_normal((1, d))
    sm, _ = oracle.predict(np.eye(d), p2, np.eye(d), p2[:3], x)
    np.testing.assert_array_equal(sm[0], p2 @ x[0])


def test_linearity():
    rng = np.random.default_rng(3)
    p1m, p2m, p1h, p2h, x = make(rng, B=1)
    y = rng.standard_normal(x.shape)
    a = oracle.predict(p1m, p2m, p1h, p2h, x + y)[0]
    b = oracle.predict(p1m, p2m, p1h, p2h, x)[0] + oracle.predict(p1m, p2m, p1h, p2h, y)[0]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_planted_transpose_is_caught():
    rng = np.random.default_rng(4)
    p1m, p2m, p1h, p2h, x = make(rng, d=5, r=5, F=5, H=5, B=1)
    wrong = oracle.predict(p1m, p2m.T, p1h, p2h, x)[0][0]
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(wrong, loops_predict(p1m.tolist(), p2m.tolist(), x[0].tolist()),
                                   rtol=1e-9)
