"""GPU parity of the step path's 256 x 256 output blocks and its grouped block
order, on ragged tiles, for both the standard full-matrix map
(himuon_tiled_ns with T = max side) and the Gram iteration (himuon_gram_ns).

Moderate shapes are compared with the fp64 oracle element by element.  Shapes
too large for the oracle use an input with a closed-form map (SVD view of the
iteration, Gram Newton-Schulz page, section 3: each step applies one odd
polynomial to every singular value and keeps the singular vectors):
Y = U D W with
  U  2 x 2 rotations pairing row i with row i + r/2 (so X X^T has nonzero
     entries far off the diagonal, in blocks that are mirrored),
  D  singular values spread over [0.5, 1.5],
  W  rows of unit norm on disjoint column sets (+-1/sqrt(s/r) entries),
whose map is U p(D / (||Y||_F + eps)) W, p the composed step polynomial.
Bar: relative Frobenius error <= 3e-2 (bf16).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from oracle import diagnostics as OD
from oracle.gram_ns import gram_ns as oracle_gram
from workloads import COEFFS

TOL = 3e-2
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3), (3.0, -3.2, 1.2)]


def say(msg):
    print(msg, flush=True)


def rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def structured(r, s, seed):
    """(Y, E): a wide r x s input (s a multiple of r) and its exact map."""
    rng = np.random.default_rng([57, seed])
    per = s // r
    assert per * r == s and r % 2 == 0
    h = r // 2
    theta = rng.uniform(0.0, 2.0 * math.pi, h)
    c, sn = np.cos(theta), np.sin(theta)
    sig = rng.uniform(0.5, 1.5, r)
    owner = rng.permutation(s) % r                      # the W row each column belongs to: per columns each
    sign = rng.choice([-1.0, 1.0], s) / math.sqrt(per)
    W_rowval = np.zeros((r, s))
    W_rowval[owner, np.arange(s)] = sign                # W, rows of unit norm on disjoint supports

    def apply_u(M):                                     # U M for the pairwise rotation U
        out = np.empty_like(M)
        out[:h] = c[:, None] * M[:h] - sn[:, None] * M[h:]
        out[h:] = sn[:, None] * M[:h] + c[:, None] * M[h:]
        return out

    Y = apply_u(sig[:, None] * W_rowval)
    nrm = math.sqrt(float(np.sum(sig ** 2)))            # ||Y||_F
    p = np.array([OD.scalar_map(x, [COEFFS] * 5) for x in sig / (nrm + oracle.EPS_DEFAULT)])
    E = apply_u(p[:, None] * W_rowval)
    return Y, E


def run_std(m):
    H.himuon_tiled_ns([m], max(m.shape), 5, COEFFS)
    torch.cuda.synchronize()


def run_gram(m):
    H.himuon_gram_ns([m], 5, COEFFS)
    torch.cuda.synchronize()


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [(1000, 1500), (2000, 2100), (2100, 1880)])
def test_ragged_large_tiles_against_oracle(cuda, shape):
    """r = 1000: every product runs 128 x 128 blocks; r = 2000 and 1880: every
    product runs 256 x 256 blocks; none of the sides is a multiple of 256, so
    each ends in a partial workspace slab of 32 columns."""
    x = workloads.round_to(np.random.default_rng([58, shape[0]]).standard_normal(shape), "bf16")
    xd = x.double().numpy()
    ref = oracle.full_matrix_ns(xd, MIXED)
    g = x.cuda()
    H.himuon_tiled_ns([g], max(shape), 5, MIXED)
    torch.cuda.synchronize()
    e1 = rel(g.double().cpu().numpy(), ref)
    g = x.cuda()
    H.himuon_gram_ns([g], 5, MIXED)
    torch.cuda.synchronize()
    e2 = rel(g.double().cpu().numpy(), oracle_gram(xd, MIXED))
    say(f"{shape}: standard {e1:.3e}, gram {e2:.3e}")
    assert e1 <= TOL and e2 <= TOL


@pytest.mark.gpu
@pytest.mark.parametrize("shape,tall", [((4300, 8600), False), ((4300, 8600), True), ((1000, 5000), False)])
def test_closed_form_long_k(cuda, shape, tall):
    """k >= 4096 walks blocks in groups of block rows: 4300 x 8600 (apply and
    the symmetric products, all 256 x 256 blocks, r = 4300 ragged), its
    transpose (worked on transposed), and 1000 x 5000 (X X^T with k = 5000,
    grouped lower blocks of the 128 x 128 shape)."""
    Y, E = structured(shape[0], shape[1], seed=shape[0] + int(tall))
    if tall:
        Y, E = Y.T.copy(), E.T.copy()
    x = workloads.round_to(Y, "bf16")
    for name, fn in (("standard", run_std), ("gram", run_gram)):
        g = x.cuda()
        fn(g)
        e = rel(g.double().cpu().numpy(), E)
        say(f"{shape} tall={tall} {name}: {e:.3e}")
        assert e <= TOL, (name, e)


def test_structured_input_is_its_own_closed_form():
    """CPU check of the construction: E equals the fp64 oracle's map of Y on a
    size the oracle handles."""
    Y, E = structured(64, 256, seed=1)
    assert np.allclose(oracle.full_matrix_ns(Y, [COEFFS] * 5), E, atol=1e-10)
