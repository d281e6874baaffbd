"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (dropped term, wrong
sign or coefficient order, transposed operand, wrong epsilon placement, tiles
that leak into each other, wrong edge handling) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (EPS_DEFAULT, QUINTIC_COEFFS, full_matrix_ns, ns_map, ns_map_stack,
                    tile_grid, tiled_ns, tiled_ns_schedule, tiled_ns_tile, muon_step,
                    algorithmic_flops, nominal_flops, tile_rel_errors)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Q5 = [QUINTIC_COEFFS] * 5
# distinct per-step triples so that the step order matters
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3)]


def scalar_poly(x, coeffs):
    """p_K o ... o p_1 applied to scalars (the SVD view: each step maps a
    singular value s to a s + b s^3 + c s^5)."""
    x = np.asarray(x, dtype=np.float64)
    for a, b, c in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def exact_poly(x, coeffs):
    x = Fraction(x)
    for a, b, c in coeffs:
        a, b, c = Fraction(str(a)), Fraction(str(b)), Fraction(str(c))
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def rng(seed):
    return np.random.default_rng([2024, seed])


@pytest.mark.parametrize("shape,T,coeffs", [((96, 160), 32, Q5), ((70, 45), 32, Q5),
                                              ((64, 64), 64, MIXED), ((33, 100), 40, MIXED),
                                              ((128, 20), 64, Q5)])
def test_svd_closed_form(shape, T, coeffs):
    """NS output per tile equals U p(Sigma) V^T of the normalised tile."""
    X = rng(1).standard_normal(shape)
    out = tiled_ns(X, T, coeffs)
    for r0, r1, c0, c1 in tile_grid(*shape, T):
        Y = X[r0:r1, c0:c1]
        Y0 = Y / (np.sqrt((Y * Y).sum()) + EPS_DEFAULT)
        U, S, Vt = np.linalg.svd(Y0, full_matrices=False)
        want = (U * scalar_poly(S, coeffs)) @ Vt
        got = out[r0:r1, c0:c1]
        assert np.linalg.norm(got - want) <= 1e-11 * max(1.0, np.linalg.norm(want))


@pytest.mark.parametrize("shape", [(40, 40), (30, 75), (75, 30), (1, 9), (9, 1)])
def test_full_matrix_reduction(shape):
    """With T >= max(H, W) the tiled map is the full-matrix map (written
    independently, with the other Gram orientation for tall matrices)."""
    X = rng(2).standard_normal(shape)
    for T in (max(shape), max(shape) + 17):
        got = tiled_ns(X, T, MIXED)
        want = full_matrix_ns(X, MIXED)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_tile_independence_bit_exact():
    X = rng(3).standard_normal((100, 130))
    T = 32
    base = tiled_ns(X, T, Q5)
    Y = X.copy()
    Y[32:64, 64:96] += rng(4).standard_normal((32, 32))
    pert = tiled_ns(Y, T, Q5)
    mask = np.zeros_like(X, dtype=bool)
    mask[32:64, 64:96] = True
    assert np.array_equal(base[~mask], pert[~mask])
    assert not np.allclose(base[mask], pert[mask])


def test_nan_containment():
    X = rng(5).standard_normal((64, 96))
    T = 32
    base = tiled_ns(X, T, Q5)
    Y = X.copy()
    Y[40, 70] = np.nan
    out = tiled_ns(Y, T, Q5)
    mask = np.zeros_like(X, dtype=bool)
    mask[32:64, 64:96] = True
    assert np.array_equal(base[~mask], out[~mask])
    assert np.isnan(out[mask]).all()


@pytest.mark.parametrize("shape,T", [((70, 100), 32), ((64, 128), 64), ((45, 45), 20)])
def test_transpose_symmetry(shape, T):
    X = rng(6).standard_normal(shape)
    np.testing.assert_allclose(tiled_ns(X.T, T, MIXED), tiled_ns(X, T, MIXED).T, rtol=0, atol=1e-12)


def test_zero_padding_invariance():
    """An edge tile zero-padded to T x T gives the same block and exact zeros
    (the padded Gram matrix is block diagonal)."""
    X = rng(7).standard_normal((50, 77))
    T = 32
    for r0, r1, c0, c1 in tile_grid(50, 77, T):
        blk = X[r0:r1, c0:c1]
        pad = np.zeros((T, T))
        pad[:r1 - r0, :c1 - c0] = blk
        got = ns_map(pad, Q5)
        np.testing.assert_allclose(got[:r1 - r0, :c1 - c0], ns_map(blk, Q5), rtol=0, atol=1e-13)
        assert np.all(got[r1 - r0:, :] == 0) and np.all(got[:, c1 - c0:] == 0)


def test_scale_invariance_and_eps_placement():
    X = rng(8).standard_normal((64, 64))
    base = ns_map(X, Q5, eps=0.0)
    for alpha in (1e-3, 0.37, 250.0):
        np.testing.assert_allclose(ns_map(alpha * X, Q5, eps=0.0), base, rtol=0, atol=1e-12)
    # eps is added to the norm: a tile of norm 1e-7 is halved before the steps
    Z = X / np.linalg.norm(X) * 1e-7
    half = ns_map(Z, [(1.0, 0.0, 0.0)])
    np.testing.assert_allclose(half, Z / 2e-7, rtol=1e-12, atol=0)


def test_rank_one_closed_form():
    """u v^T normalises to a single singular value 1: output p(1) u v^T / (|u||v|).
    p(1) is computed in exact rational arithmetic."""
    r = rng(9)
    u, v = r.standard_normal(48), r.standard_normal(80)
    p1 = float(exact_poly(1, Q5))
    assert abs(p1 - 0.6964364094697528) < 1e-15
    got = ns_map(np.outer(u, v), Q5, eps=0.0)
    want = p1 * np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    # K = 1 with the quintic: 3.4445 - 4.7750 + 2.0315
    got1 = ns_map(np.outer(u, v), [QUINTIC_COEFFS], eps=0.0)
    np.testing.assert_allclose(got1, 0.701 * np.outer(u, v) / (np.linalg.norm(u) * np.linalg.norm(v)),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [16, 64, 128])
def test_scaled_orthogonal(n):
    """c Q normalises to Q / sqrt(n), so the output is p(1/sqrt(n)) Q."""
    Q, _ = np.linalg.qr(rng(10).standard_normal((n, n)))
    got = ns_map(3.7 * Q, Q5, eps=0.0)
    np.testing.assert_allclose(got, scalar_poly(1 / math.sqrt(n), Q5) * Q, rtol=0, atol=1e-12)
    if n == 64:
        assert abs(scalar_poly(1 / 8, Q5) - 0.688139855776055) < 1e-13


def test_diagonal_tile():
    d = rng(11).standard_normal(30)
    got = ns_map(np.diag(d), MIXED, eps=0.0)
    want = np.diag(np.sign(d) * scalar_poly(np.abs(d) / np.linalg.norm(d), MIXED))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_k0_is_normalisation():
    X = rng(12).standard_normal((20, 33))
    np.testing.assert_allclose(ns_map(X, np.zeros((0, 3))), X / (np.linalg.norm(X) + EPS_DEFAULT),
                               rtol=0, atol=1e-15)


def _fraction_ns(Y, coeffs):
    """Exact rational Newton-Schulz for tiny blocks with an integer norm and eps = 0."""
    h, w = len(Y), len(Y[0])
    ss = sum(x * x for row in Y for x in row)
    nrm = math.isqrt(ss)
    assert nrm * nrm == ss
    X = [[Fraction(x, nrm) for x in row] for row in Y]
    if h > w:
        X = [list(r) for r in zip(*X)]
    mm = lambda P, Q: [[sum(P[i][k] * Q[k][j] for k in range(len(Q))) for j in range(len(Q[0]))] for i in range(len(P))]
    for a, b, c in coeffs:
        a, b, c = Fraction(str(a)), Fraction(str(b)), Fraction(str(c))
        Xt = [list(r) for r in zip(*X)]
        A = mm(X, Xt)
        A2 = mm(A, A)
        B = [[b * A[i][j] + c * A2[i][j] for j in range(len(A))] for i in range(len(A))]
        BX = mm(B, X)
        X = [[a * X[i][j] + BX[i][j] for j in range(len(X[0]))] for i in range(len(X))]
    if h > w:
        X = [list(r) for r in zip(*X)]
    return X


@pytest.mark.parametrize("Y", [[[2, 3], [6, 0]], [[1, 2, 2], [0, 0, 4]], [[3], [4]], [[2, 2, 0], [0, 2, 2], [4, 0, 2]]])
def test_exact_rational_brute_force(Y):
    """fp64 oracle against exact rational arithmetic (eps = 0)."""
    exact = _fraction_ns(Y, Q5[:3])
    got = ns_map(np.array(Y, dtype=np.float64), Q5[:3], eps=0.0)
    want = np.array([[float(x) for x in row] for row in exact])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_stack_matches_single():
    r = rng(13)
    S = r.standard_normal((7, 24, 40))
    got = ns_map_stack(S, MIXED)
    for i in range(7):
        np.testing.assert_allclose(got[i], ns_map(S[i], MIXED), rtol=0, atol=1e-14)
    St = r.standard_normal((5, 40, 24))
    got = ns_map_stack(St, Q5)
    for i in range(5):
        np.testing.assert_allclose(got[i], ns_map(St[i], Q5), rtol=0, atol=1e-14)


@pytest.mark.parametrize("shape,coeffs", [((9, 24, 40), MIXED), ((6, 40, 24), Q5), ((5, 32, 32), Q5)])
def test_stack_torch_matches_single_and_svd(shape, coeffs):
    """The torch batched form against ns_map block by block, and against the
    SVD closed form U p(S) V^T of each normalised block."""
    S = rng(21).standard_normal(shape)
    S[1] *= 1e-3                       # scale does not matter
    S[2] = 0.0                         # zero block stays zero
    got = oracle.ns_map_stack_torch(S, coeffs).numpy()
    for i in range(shape[0]):
        np.testing.assert_allclose(got[i], ns_map(S[i], coeffs), rtol=0, atol=1e-13)
        Y0 = S[i] / (np.linalg.norm(S[i]) + EPS_DEFAULT)
        U, sv, Vt = np.linalg.svd(Y0, full_matrices=False)
        np.testing.assert_allclose(got[i], (U * scalar_poly(sv, coeffs)) @ Vt, rtol=0, atol=1e-11)
    assert not np.any(got[2])


def test_tile_accessor_and_grid():
    X = rng(14).standard_normal((70, 45))
    T = 32
    boxes = tile_grid(70, 45, T)
    assert len(boxes) == math.ceil(70 / T) * math.ceil(45 / T)
    cover = np.zeros((70, 45), dtype=int)
    for r0, r1, c0, c1 in boxes:
        cover[r0:r1, c0:c1] += 1
    assert np.all(cover == 1)
    full = tiled_ns(X, T, Q5)
    np.testing.assert_array_equal(tiled_ns_tile(X, T, 2, 1, Q5), full[64:70, 32:45])


def test_schedule_single_size_equals_tiled():
    X = rng(15).standard_normal((96, 64))
    np.testing.assert_allclose(tiled_ns_schedule(X, [32] * 4, MIXED), tiled_ns(X, 32, MIXED), rtol=0, atol=1e-14)


def test_schedule_block_diagonal_locality():
    """If every coarse tile is block diagonal over the finer tiles, a coarse
    step equals the same step on the finer tiles (the Gram matrix is block
    diagonal), so the schedule 64 -> 32 equals 64 -> 64."""
    X = np.zeros((128, 128))
    r = rng(16)
    for i in range(0, 128, 32):
        X[i:i + 32, i:i + 32] = r.standard_normal((32, 32))
    for i in range(0, 128, 64):
        X[i:i + 32, i + 32:i + 64] = 0
    a = tiled_ns_schedule(X, [64, 32, 32], MIXED[:3])
    b = tiled_ns_schedule(X, [64, 64, 64], MIXED[:3])
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        tiled_ns_schedule(X, [32, 64], MIXED[:2])


def _svd_step_schedule(X, Ts, coeffs, eps=EPS_DEFAULT):
    """The schedule built another way: normalise every Ts[0]-tile, then for
    step t replace every Ts[t]-tile by U p_t(S) V^T from its own SVD (the SVD
    view of one Newton-Schulz step on the Gram Newton-Schulz page, section 3)."""
    X = np.array(X, dtype=np.float64, copy=True)
    H, W = X.shape
    T0 = Ts[0]
    for r0 in range(0, H, T0):
        for c0 in range(0, W, T0):
            blk = X[r0:r0 + T0, c0:c0 + T0]
            X[r0:r0 + T0, c0:c0 + T0] = blk / (np.linalg.norm(blk) + eps)
    for (a, b, c), T in zip(coeffs, Ts):
        for r0 in range(0, H, T):
            for c0 in range(0, W, T):
                U, S, Vt = np.linalg.svd(X[r0:r0 + T, c0:c0 + T], full_matrices=False)
                X[r0:r0 + T, c0:c0 + T] = (U * (a * S + b * S ** 3 + c * S ** 5)) @ Vt
    return X


@pytest.mark.parametrize("shape,Ts", [((150, 200), [64, 32, 32]), ((128, 192), [128, 64, 32, 32]),
                                       ((96, 96), [96, 48, 16, 16])])
def test_schedule_per_step_svd(shape, Ts):
    """Step t of the schedule acts on the Ts[t]-tiles of the current iterate:
    a generic (not block-diagonal) input, against the per-step SVD form."""
    X = rng(18).standard_normal(shape)
    got = tiled_ns_schedule(X, Ts, MIXED[:len(Ts)])
    want = _svd_step_schedule(X, Ts, MIXED[:len(Ts)])
    assert np.linalg.norm(got - want) <= 1e-11 * np.linalg.norm(want)
    # the input tells the sizes apart: the first size held for every step
    # gives a visibly different result
    coarse = _svd_step_schedule(X, [Ts[0]] * len(Ts), MIXED[:len(Ts)])
    assert np.linalg.norm(coarse - want) > 1e-2 * np.linalg.norm(want)


def test_schedule_rank_one_closed_form():
    """A rank-one 64-tile u v^T under the schedule 64 -> 32 (eps = 0).  After
    the coarse step the tile is p1(1) u v^T / (|u| |v|), so its 32-subtile
    (i, j) is rank one with singular value s_ij = p1(1) |u_i| |v_j| / (|u| |v|),
    and the fine step scales it by p2(s_ij) / s_ij."""
    r = rng(19)
    u, v = r.standard_normal(64), r.standard_normal(64)
    u[:32] *= 3.0   # unequal halves: the four subtiles get different s_ij
    v[32:] *= 0.25
    X = np.outer(u, v)
    c1, c2 = MIXED[0], MIXED[1]
    got = tiled_ns_schedule(X, [64, 32], [c1, c2], eps=0.0)
    p1 = scalar_poly(1.0, [c1])
    nu, nv = np.linalg.norm(u), np.linalg.norm(v)
    for i in (0, 32):
        for j in (0, 32):
            ui, vj = u[i:i + 32], v[j:j + 32]
            s = p1 * np.linalg.norm(ui) * np.linalg.norm(vj) / (nu * nv)
            want = scalar_poly(s, [c2]) / s * (p1 / (nu * nv)) * np.outer(ui, vj)
            np.testing.assert_allclose(got[i:i + 32, j:j + 32], want, rtol=0,
                                       atol=1e-13 * np.abs(want).max())


def test_muon_step_rank_one_closed_form():
    """M = u v^T, G = u w^T: the new momentum is u (mu v + w)^T, rank one, so
    with eps = 0 every T-tile (i, j) of the update is p(1) u_i z_j^T /
    (|u_i| |z_j|) with z = mu v + w; W moves by -eta times that."""
    r = rng(20)
    u, v, w = r.standard_normal(64), r.standard_normal(96), r.standard_normal(96)
    W0 = r.standard_normal((64, 96))
    mu, eta, T = 0.9, 0.05, 32
    Wn, Mn = muon_step(W0, np.outer(u, v), np.outer(u, w), mu=mu, eta=eta, T=T, coeffs=MIXED, eps=0.0)
    z = mu * v + w
    np.testing.assert_allclose(Mn, np.outer(u, z), rtol=0, atol=1e-13)
    p = scalar_poly(1.0, MIXED)
    for r0 in range(0, 64, T):
        for c0 in range(0, 96, T):
            ui, zj = u[r0:r0 + T], z[c0:c0 + T]
            upd = p * np.outer(ui, zj) / (np.linalg.norm(ui) * np.linalg.norm(zj))
            np.testing.assert_allclose(Wn[r0:r0 + T, c0:c0 + T], W0[r0:r0 + T, c0:c0 + T] - eta * upd,
                                       rtol=0, atol=1e-13)


def test_muon_step_composition():
    r = rng(17)
    W, M, G = (r.standard_normal((64, 96)) for _ in range(3))
    Wn, Mn = muon_step(W, M, G, mu=0.95, eta=0.02, T=32, coeffs=Q5)
    np.testing.assert_allclose(Mn, 0.95 * M + G, rtol=0, atol=1e-15)
    np.testing.assert_allclose((W - Wn) / 0.02, tiled_ns(0.95 * M + G, 32, Q5), rtol=0, atol=1e-11)


def test_page_constants_and_flop_model():
    g = json.load(open(os.path.join(GOLDEN, "alg1_page_constants.json")))
    assert EPS_DEFAULT == g["epsilon"]
    for case in g["cases"]:
        n, m = case["n"], case["m"]
        assert algorithmic_flops([(n, m)], T=max(n, m), K=1) == case["flops_per_iteration"]
        assert algorithmic_flops([(m, n)], T=max(n, m), K=1) == case["flops_per_iteration"]
    # for full square tiles the 6 H W T K count is exactly the page's count
    assert nominal_flops([(256, 512)], 64, 5) == algorithmic_flops([(256, 512)], 64, 5)


def test_tile_error_metric():
    ref = np.ones((64, 64))
    got = ref.copy()
    got[:32, :32] *= 1.01
    e = tile_rel_errors(got, ref, 32)
    np.testing.assert_allclose(e, [0.01, 0, 0, 0], atol=1e-15)
