"""Pins of the oracle's tiled-versus-full-map diagnostics.

Each pin is fixed by the mathematics rather than by the oracle's own formulas:
brute-force sums, identities of the two measures, the full map recovered when
one tile covers the matrix, the SVD view of the iteration (Gram Newton-Schulz
page, section 3) for the output spectrum, and a closed form of the tiled-to-
full distance for block-diagonal inputs whose blocks are whole tiles.
"""
import math

import numpy as np
import pytest

from oracle import EPS_DEFAULT, QUINTIC_COEFFS, full_matrix_ns, ns_map, tiled_ns
from oracle import diagnostics as D

Q5 = [QUINTIC_COEFFS] * 5
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3)]


def rng(seed):
    return np.random.default_rng([77, seed])


def test_pair_stats_brute_force():
    a = rng(1).standard_normal((3, 4))
    b = rng(2).standard_normal((3, 4))
    dot = aa = bb = 0.0
    for i in range(3):
        for j in range(4):
            dot += a[i][j] * b[i][j]
            aa += a[i][j] * a[i][j]
            bb += b[i][j] * b[i][j]
    got = D.pair_stats(a, b)
    assert got[0] == pytest.approx(dot, rel=1e-14)
    assert got[1] == pytest.approx(aa, rel=1e-14)
    assert got[2] == pytest.approx(bb, rel=1e-14)
    with pytest.raises(ValueError):
        D.pair_stats(a, b[:, :3])


def test_measures_identities():
    x = rng(3).standard_normal((20, 30))
    assert D.rel_distance(x, x) == 0.0
    assert D.cosine(x, x) == pytest.approx(1.0, abs=1e-15)
    assert D.cosine(-x, x) == pytest.approx(-1.0, abs=1e-15)
    assert D.rel_distance(-x, x) == pytest.approx(2.0, rel=1e-15)
    assert D.rel_distance(2 * x, x) == pytest.approx(1.0, rel=1e-15)
    # disjoint supports: orthogonal, distance sqrt(|g|^2 + |r|^2) / |r|
    g = np.zeros((4, 4)); g[0, :] = [1, 2, 3, 4]
    r = np.zeros((4, 4)); r[3, :] = [2, 0, 0, 0]
    assert D.cosine(g, r) == 0.0
    assert D.rel_distance(g, r) == pytest.approx(math.sqrt(30 + 4) / 2, rel=1e-15)
    # the sum forms agree with the direct ones
    y = x + 0.1 * rng(4).standard_normal(x.shape)
    st = D.pair_stats(y, x)
    assert D.distance_from_stats(st) == pytest.approx(D.rel_distance(y, x), rel=1e-10)
    assert D.cosine_from_stats(st) == pytest.approx(D.cosine(y, x), rel=1e-14)


@pytest.mark.parametrize("shape", [(40, 64), (64, 40), (50, 50)])
def test_one_tile_is_the_full_map(shape):
    M = rng(5).standard_normal(shape)
    rows = D.tiled_vs_full(M, [max(shape), 2 * max(shape)], Q5)
    for r in rows:
        assert r["distance"] <= 1e-13
        assert r["cosine"] >= 1 - 1e-13


def test_scalar_map_is_the_matrix_map_on_a_diagonal():
    """ns_map of diag(s) is diag(p(s / (||s|| + eps))): the scalar map against
    the matrix iteration (pinned elsewhere by the SVD closed form)."""
    s = np.array([3.0, 1.0, 0.5, 0.01, 2.0])
    out = ns_map(np.diag(s), MIXED)
    want = D.scalar_map(s / (np.linalg.norm(s) + EPS_DEFAULT), MIXED)
    assert np.allclose(np.diag(out), want, rtol=0, atol=1e-13)
    assert np.count_nonzero(out - np.diag(np.diag(out))) == 0


@pytest.mark.parametrize("shape,coeffs", [((48, 80), Q5), ((90, 36), MIXED)])
def test_spectrum_closed_form(shape, coeffs):
    """Output singular values of the full map are |p(s_i / (||s||_2 + eps))|,
    for an input built from known singular values and random orthogonal
    factors."""
    h, w = shape
    k = min(h, w)
    g = rng(6)
    U, _ = np.linalg.qr(g.standard_normal((h, k)))
    V, _ = np.linalg.qr(g.standard_normal((w, k)))
    s = np.sort(np.exp(g.uniform(np.log(1e-3), 0.0, k)))[::-1]
    M = (U * s) @ V.T
    out = full_matrix_ns(M, coeffs)
    want = np.sort(np.abs(D.scalar_map(s / (np.linalg.norm(s) + EPS_DEFAULT), coeffs)))[::-1]
    got = D.spectrum(out)
    assert got.shape == (k,)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(48, 80), (90, 36), (1, 7), (33, 33)])
def test_spectral_moments_trace_identities(shape):
    """The moments from the spectrum against traces of the Gram matrix of the
    shorter side, G: sum s^2 = tr G, sum s^4 = ||G||_F^2, sum s^6 = tr G^3;
    and the orthogonality residual of a matrix with known singular values."""
    g = rng(8)
    X = g.standard_normal(shape)
    G = X @ X.T if shape[0] <= shape[1] else X.T @ X
    r, m2, m4, m6 = D.spectral_moments(X)
    assert r == min(shape)
    assert m2 == pytest.approx(np.trace(G), rel=1e-12)
    assert m4 == pytest.approx(np.sum(G * G), rel=1e-12)
    assert m6 == pytest.approx(np.trace(G @ G @ G), rel=1e-12)
    h, w = shape
    k = min(h, w)
    U, _ = np.linalg.qr(g.standard_normal((h, k)))
    V, _ = np.linalg.qr(g.standard_normal((w, k)))
    s = g.uniform(0.5, 1.5, k)
    want = math.sqrt(np.mean((s ** 2 - 1.0) ** 2))
    assert D.orthogonality_residual(D.spectral_moments((U * s) @ V.T)) == pytest.approx(want, rel=1e-9, abs=1e-12)
    assert D.orthogonality_residual(D.spectral_moments(U @ V.T)) < 1e-7


def test_block_diagonal_distance_closed_form():
    """M = diag(B1, B2) with B1, B2 whole T x T tiles of equal Frobenius norm r.
    The off-diagonal tiles are zero and stay zero; each diagonal tile is
    normalised by r, the full matrix by sqrt(2) r.  Both outputs keep the
    blocks' singular vectors, so with x = singular values of the blocks
      ||tiled - full||^2 = sum (p(x / (r + eps)) - p(x / (sqrt2 r + eps)))^2,
      ||full||^2        = sum p(x / (sqrt2 r + eps))^2."""
    T = 32
    g = rng(7)
    B1 = g.standard_normal((T, T))
    B2 = g.standard_normal((T, T)) * 0.3
    r = np.linalg.norm(B1)
    B2 *= r / np.linalg.norm(B2)
    M = np.zeros((2 * T, 2 * T))
    M[:T, :T] = B1
    M[T:, T:] = B2
    x = np.concatenate([np.linalg.svd(B1, compute_uv=False), np.linalg.svd(B2, compute_uv=False)])
    pt = D.scalar_map(x / (r + EPS_DEFAULT), Q5)
    pf = D.scalar_map(x / (math.sqrt(2 * r * r) + EPS_DEFAULT), Q5)
    want_d = math.sqrt(np.sum((pt - pf) ** 2) / np.sum(pf ** 2))
    want_c = float(np.sum(pt * pf) / math.sqrt(np.sum(pt ** 2) * np.sum(pf ** 2)))
    row = D.tiled_vs_full(M, [T], Q5, with_spectrum=True)[0]
    assert row["distance"] == pytest.approx(want_d, rel=1e-10)
    assert row["cosine"] == pytest.approx(want_c, rel=1e-12)
    assert want_d > 1e-2   # the two maps really differ here
    assert np.allclose(row["spectrum"], np.sort(np.abs(pt))[::-1], atol=1e-12)
    assert np.allclose(row["full_spectrum"], np.sort(np.abs(pf))[::-1], atol=1e-12)
    # the tiled output is the blockwise map
    t = tiled_ns(M, T, Q5)
    assert np.count_nonzero(t[:T, T:]) == 0 and np.count_nonzero(t[T:, :T]) == 0


def test_distance_shrinks_to_zero_as_T_reaches_the_matrix():
    """Not a closed form, a sanity property: a T that covers the matrix gives
    distance 0, and smaller tiles give a strictly positive distance."""
    M = rng(8).standard_normal((96, 160))
    rows = D.tiled_vs_full(M, [16, 32, 96, 160], Q5)
    assert all(r["distance"] > 1e-3 for r in rows[:3])
    assert rows[-1]["distance"] <= 1e-13
