"""GPU parity of himuon_gram_ns (Gram Newton-Schulz with a restart, "Gram
Newton-Schulz" page, section 6, Algorithm 3) against the fp64 oracle.

The bar is the library's: per-matrix relative Frobenius error <= 3e-2 for bf16
data and <= 1e-4 for fp32 data, against oracle.gram_ns (which equals the
standard full-matrix map to rounding in fp64).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from oracle.gram_ns import gram_ns as oracle_gram
from workloads import COEFFS, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = {"bf16": 3e-2, "fp32": 1e-4}
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3), (3.0, -3.2, 1.2)]


def say(msg):
    print(msg, flush=True)


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel(got, ref):
    return np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)


def gram_check(x_host, dt, K=5, abc=MIXED, restart=2, cap=None):
    ref = oracle_gram(x_host.double().numpy(), abc[:K] if K else [], restart=restart, K=K)
    g = x_host.cuda()
    H.himuon_gram_ns([g], K, abc[:K] if K else [], restart=restart, workspace_bytes=cap)
    torch.cuda.synchronize()
    return rel(to_np(g), ref), g


# Shapes: several 128-blocks with a ragged tail, both orientations, r below
# 32 (fp32 workspace), a row count that is not a multiple of 8, a square one.
BF16_SHAPES = [(300, 170), (170, 300), (256, 1024), (129, 600), (600, 129), (64, 64), (20, 700), (1, 1),
               (7, 300), (385, 1100)]


@pytest.mark.parametrize("restart", [0, 1, 2, 4])
def test_bf16_shapes_and_restarts(cuda, restart):
    rng = np.random.default_rng([71, restart])
    for (h, w) in BF16_SHAPES:
        x = workloads.round_to(rng.standard_normal((h, w)), "bf16")
        err, _ = gram_check(x, "bf16", restart=restart)
        say(f"gram bf16 {h}x{w} restart={restart}: {err:.3e}")
        assert err <= TOL["bf16"], (h, w, restart, err)


@pytest.mark.parametrize("restart", [0, 2])
def test_fp32_shapes(cuda, restart):
    rng = np.random.default_rng([72, restart])
    for (h, w) in [(1, 1), (33, 65), (200, 150), (300, 299), (129, 600), (20, 700)]:
        x = workloads.round_to(rng.standard_normal((h, w)), "fp32")
        err, _ = gram_check(x, "fp32", restart=restart)
        say(f"gram fp32 {h}x{w} restart={restart}: {err:.3e}")
        assert err <= TOL["fp32"], (h, w, restart, err)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("K", [0, 1, 2, 3, 5])
def test_step_counts(cuda, dt, K):
    """K = 2 with restart 2 never restarts; K = 3 restarts before its last
    step; K = 0 writes the normalised matrix."""
    rng = np.random.default_rng([73, K])
    x = workloads.round_to(rng.standard_normal((270, 520)), dt)
    err, _ = gram_check(x, dt, K=K, restart=2)
    say(f"gram {dt} K={K}: {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("restart", [2, 8])
def test_max_steps(cuda, restart):
    """K = 16 with a restart after two steps and after eight: five quintic
    steps, then eleven cubic ones (1.5, -0.5, 0), which draw the singular
    values to 1 (sixteen quintic steps compound bf16 rounding past 3e-2 on
    every route, the standard map's included)."""
    rng = np.random.default_rng([76, restart])
    x = workloads.round_to(rng.standard_normal((300, 900)), "bf16")
    steps = [COEFFS] * 5 + [(1.5, -0.5, 0.0)] * 11
    err, _ = gram_check(x, "bf16", K=16, abc=steps, restart=restart)
    say(f"gram K=16 restart={restart}: {err:.3e}")
    assert err <= TOL["bf16"]


def test_chunking_bit_exact(cuda):
    """A workspace that holds one matrix at a time gives the same bits as one
    chunk for all."""
    rng = np.random.default_rng(74)
    xs = [workloads.round_to(rng.standard_normal(s), "bf16").cuda() for s in [(600, 520), (257, 1300), (130, 40)]]
    full, mn = H.himuon_gram_ns_workspace(xs)
    assert full > mn > 0
    a = [x.clone() for x in xs]
    H.himuon_gram_ns(a, 5, COEFFS)
    b = [x.clone() for x in xs]
    H.himuon_gram_ns(b, 5, COEFFS, workspace_bytes=mn)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_transposed_view_and_batch(cuda):
    """A transposed view and a mixed batch in one call, each against the
    oracle on its own."""
    rng = np.random.default_rng(75)
    hosts = [workloads.round_to(rng.standard_normal(s), "bf16") for s in [(300, 900), (512, 256), (100, 333)]]
    devs = [hosts[0].cuda(), hosts[1].t().contiguous().cuda().t(), hosts[2].cuda()]
    assert devs[1].stride(0) == 1
    H.himuon_gram_ns(devs, 5, COEFFS)
    torch.cuda.synchronize()
    for x, d in zip(hosts, devs):
        err = rel(to_np(d), oracle_gram(x.double().numpy(), [COEFFS] * 5))
        say(f"gram batch {tuple(x.shape)}: {err:.3e}")
        assert err <= TOL["bf16"]


def test_layers24_d2048(cuda):
    """The 24-layer batch (d = 2048, 2048 x 2048, 2048 x 5632, 5632 x 2048)
    through the Gram iteration in one call: one matrix of each shape against
    the oracle, and every matrix against the standard full-matrix map on the
    GPU (both approximate the same exact map)."""
    w = WORKLOADS["layers24_d2048"]
    mats = workloads.device_tensors(w)
    std = [m.clone() for m in mats]
    idx = [3, 4, 6]
    host = {i: to_np(mats[i]) for i in idx}
    say("layers24 gram")
    H.himuon_gram_ns(mats, 5, COEFFS)
    H.himuon_tiled_ns(std, 5632, 5, COEFFS)
    torch.cuda.synchronize()
    for i in idx:
        e = rel(to_np(mats[i]), oracle_gram(host[i], [COEFFS] * 5))
        say(f"  matrix {i} {host[i].shape}: {e:.3e}")
        assert e <= TOL["bf16"]
    for a, b in zip(mats, std):
        d = (a.float() - b.float()).norm() / b.float().norm()
        assert d.item() <= 2 * TOL["bf16"]


def test_operand_past_2gib_closed_form(cuda):
    """16384 x 65536 bf16: the oriented operand is 2 GiB, past the DMA GEMM's
    32-bit offsets, so every product runs the register-staged GEMM.  Each row
    holds +-1 on four columns of its own (a random assignment), so the rows
    are orthogonal and of equal norm: R is a multiple of I, every matrix of
    the iteration stays diagonal, and the map sends each nonzero element to
    +-p(sigma) / sigma * x, with sigma = 2 / ||Y||_F (normalised) and p the
    composed step polynomial (SVD view of the iteration, Gram Newton-Schulz
    page, section 3).  Zeros must stay zero and signs must hold."""
    from oracle import diagnostics as OD
    Hh, Ww = 16384, 65536
    g = torch.Generator(device="cpu").manual_seed(77)
    owner = torch.randperm(Ww, generator=g) % Hh          # the row each column belongs to: four per row
    sign = (torch.randint(0, 2, (Ww,), generator=g) * 2 - 1).to(torch.bfloat16)
    m = torch.zeros((Hh, Ww), dtype=torch.bfloat16, device=cuda)
    cols = torch.arange(Ww)
    m[owner.to(cuda), cols.to(cuda)] = sign.to(cuda)
    full, _ = H.himuon_gram_ns_workspace([m])
    say(f"gram of {Hh}x{Ww} bf16, workspace {full / 2**30:.1f} GiB")
    H.himuon_gram_ns([m], 5, COEFFS)
    torch.cuda.synchronize()
    norm = math.sqrt(Ww)                                # ||Y||_F
    sigma = 2.0 / (norm + oracle.EPS_DEFAULT)           # every singular value of the normalised X
    p = float(OD.scalar_map(sigma, [COEFFS] * 5))
    want_mag = p / 2.0                                  # p(sigma) times y / ||row of y||, with ||row|| = 2
    # the nonzero elements
    got = m[owner.to(cuda), cols.to(cuda)].float()
    ratio = got / sign.to(cuda).float()
    err = (ratio - want_mag).abs().max().item() / want_mag
    say(f"  p(sigma) = {p:.6f}, element magnitude {want_mag:.6f}, worst relative error {err:.3e}")
    assert err <= 3e-2
    # every other element is zero
    m[owner.to(cuda), cols.to(cuda)] = 0
    assert torch.count_nonzero(m).item() == 0
    del m, got, ratio
    torch.cuda.empty_cache()
