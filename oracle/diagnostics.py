"""fp64 reference for the tiled-versus-full-map diagnostics (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use this
module; it shares no code with the HIP library.

What is measured.  The HiMuon abstract presents the tiled map as a local
stand-in for the full-matrix Newton-Schulz map (each tile sees only its own
block, where the full map couples all rows and columns).  The pages give no
number for how far apart the two maps are, so these plain measures are used:

* relative Frobenius distance  ||tiled - full||_F / ||full||_F;
* cosine similarity            <tiled, full>_F / (||tiled||_F ||full||_F);
* the singular values of an output.  The "Gram Newton-Schulz" summary page,
  section 3 (the SVD view of the iteration), says each step moves every
  singular value through the same odd polynomial and keeps the singular
  vectors, so an orthogonalised update has its singular values near 1.

The three sums a device reduction returns for a pair of equal-shaped matrices
(sum a*b, sum a*a, sum b*b) are given by pair_stats; the distance and cosine
follow from them, and from the matrices directly, in the functions below.

Parity status: pinned by tests/test_oracle_diagnostics.py (brute-force sums,
the identities of the two measures, the full map recovered at T >= max(H, W),
the SVD closed form of the output spectrum, the spectral moments against
trace identities of the Gram matrix, and a closed form of the tiled-to-full
distance for block-diagonal inputs).
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

from .tiled_ns import EPS_DEFAULT, _coeff_list, full_matrix_ns, tiled_ns


def pair_stats(a, b):
    """(sum a*b, sum a*a, sum b*b) over all elements, in float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError("pair_stats takes two arrays of one shape")
    return float(np.sum(a * b)), float(np.sum(a * a)), float(np.sum(b * b))


def rel_distance(got, ref) -> float:
    """||got - ref||_F / ||ref||_F (ref is the full-matrix map)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def cosine(got, ref) -> float:
    """<got, ref>_F / (||got||_F ||ref||_F)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sum(got * ref) / (np.linalg.norm(got) * np.linalg.norm(ref)))


def distance_from_stats(stats) -> float:
    """rel_distance written with the three pair sums (got first, ref second):
    ||g - r||^2 = sum g^2 + sum r^2 - 2 sum g r."""
    dot, gg, rr = stats
    return math.sqrt(max(gg + rr - 2.0 * dot, 0.0)) / math.sqrt(rr)


def cosine_from_stats(stats) -> float:
    dot, gg, rr = stats
    return dot / math.sqrt(gg * rr)


def spectrum(X):
    """Singular values of X, largest first (LAPACK through numpy)."""
    return np.linalg.svd(np.asarray(X, dtype=np.float64), compute_uv=False)


def spectral_moments(X):
    """(r, sum s^2, sum s^4, sum s^6) over the r = min(H, W) singular values s
    of X, from its spectrum.  With the moments, mean(s^2) = m2 / r and
    ||X^T X - I||_F^2 = sum (s^2 - 1)^2 = m4 - 2 m2 + r (the Gram matrix of
    the shorter side) measure how far an output is from orthogonal."""
    X = np.asarray(X, dtype=np.float64)
    s2 = spectrum(X) ** 2
    return min(X.shape), float(np.sum(s2)), float(np.sum(s2 ** 2)), float(np.sum(s2 ** 3))


def orthogonality_residual(moments) -> float:
    """RMS of s^2 - 1 over the singular values: sqrt((m4 - 2 m2 + r) / r)."""
    r, m2, m4, _ = moments
    return math.sqrt(max(m4 - 2.0 * m2 + r, 0.0) / r) if r > 0 else 0.0


def scalar_map(x, coeffs, K: int | None = None):
    """The odd polynomial one run of steps applies to each (normalised)
    singular value: x <- a x + b x^3 + c x^5 per step (the SVD view of the
    iteration, Gram Newton-Schulz page, section 3)."""
    x = np.array(x, dtype=np.float64, copy=True)
    for a, b, c in _coeff_list(coeffs, K):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def tiled_vs_full(M, Ts: Sequence[int], coeffs, eps: float = EPS_DEFAULT, K: int | None = None,
                  with_spectrum: bool = False):
    """For each T: the distance and cosine between tiledNS_T(M) and the
    full-matrix map of M, and (optionally) both outputs' singular values.

    Returns a list of dicts {T, distance, cosine[, spectrum]} and, when
    with_spectrum, the full map's singular values as the last element's
    "full_spectrum".
    """
    full = full_matrix_ns(M, coeffs, eps=eps, K=K)
    rows = []
    for T in Ts:
        t = tiled_ns(M, T, coeffs, eps=eps, K=K)
        row = {"T": int(T), "distance": rel_distance(t, full), "cosine": cosine(t, full)}
        if with_spectrum:
            row["spectrum"] = spectrum(t)
        rows.append(row)
    if with_spectrum and rows:
        rows[-1]["full_spectrum"] = spectrum(full)
    return rows
