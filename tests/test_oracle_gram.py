"""Pins of the oracle's Gram Newton-Schulz (Algorithms 2 and 3 of the Gram
Newton-Schulz page) against the standard map it reformulates.

full_matrix_ns is an independent form of the standard map (right-hand Gram
form for tall matrices), itself pinned by the SVD closed form in
test_oracle.py; in exact arithmetic the Gram iteration equals it for any
restart point, so in fp64 they agree to rounding.
"""
import numpy as np
import pytest

from oracle import EPS_DEFAULT, QUINTIC_COEFFS, full_matrix_ns
from oracle.gram_ns import gram_ns

Q5 = [QUINTIC_COEFFS] * 5
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3), (3.0, -3.2, 1.2)]


def rng(seed):
    return np.random.default_rng([91, seed])


@pytest.mark.parametrize("shape", [(40, 110), (110, 40), (64, 64), (7, 300)])
@pytest.mark.parametrize("restart", [0, 1, 2, 4])
def test_equals_standard_map(shape, restart):
    X = rng(shape[0] + restart).standard_normal(shape)
    want = full_matrix_ns(X, MIXED)
    got = gram_ns(X, MIXED, restart=restart)
    assert got.shape == X.shape
    assert np.linalg.norm(got - want) <= 1e-10 * np.linalg.norm(want)


def test_steps_and_coefficients_order():
    """Fewer steps, and the coefficient rows taken in order: a permuted list
    gives a different result, the right one matches the standard map."""
    X = rng(5).standard_normal((30, 90))
    for K in (0, 1, 3):
        assert np.allclose(gram_ns(X, MIXED[:K], K=K), full_matrix_ns(X, MIXED[:K], K=K), atol=1e-12)
    assert not np.allclose(gram_ns(X, MIXED[::-1]), full_matrix_ns(X, MIXED))


def test_rank_one_closed_form():
    """Y = s u v^T: the output is p(s / (s + eps)) u v^T for unit u, v, with
    p the composed step polynomial."""
    u = rng(6).standard_normal(25); u /= np.linalg.norm(u)
    v = rng(7).standard_normal(70); v /= np.linalg.norm(v)
    s = 3.0
    x = s / (s + EPS_DEFAULT)
    for a, b, c in Q5:
        x = a * x + b * x ** 3 + c * x ** 5
    got = gram_ns(s * np.outer(u, v), Q5)
    assert np.allclose(got, x * np.outer(u, v), atol=1e-12)


@pytest.mark.parametrize("restart", [0, 1, 2, 3])
def test_restart_point(restart):
    """The base Q is applied to is the input advanced by exactly `restart`
    standard steps (the page restarts before step 3, i.e. after two), and Q
    carries the remaining steps."""
    X = rng(8).standard_normal((20, 50))
    out, Q, base = gram_ns(X, MIXED, restart=restart, return_parts=True)
    assert np.allclose(base, full_matrix_ns(X, MIXED[:restart], K=restart), atol=1e-12)
    assert np.allclose(Q @ base, out, atol=1e-12)
    assert np.allclose(Q, Q.T, atol=1e-10)        # a polynomial in a symmetric matrix
