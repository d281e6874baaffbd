"""GPU parity of the tiled-versus-full-map diagnostics against the fp64 oracle.

* himuon_pair_stats against oracle.diagnostics.pair_stats on host copies of the
  same inputs: products are exact in fp64 on both sides and only the summation
  order differs, so the bound is 1e-12 relative (to sum |a b| for the mixed
  sum, which can cancel).
* The distance and cosine reported for the library's own outputs against the
  oracle's formulas applied to host copies of those outputs: 1e-9.
* End to end against the oracle's fp64 maps: the bf16 path's per-tile error
  is at most 3e-2 of the tile norm (the parity bound), so by the triangle
  inequality ||tiled_gpu - full_gpu|| differs from ||tiled - full|| by at most
  3e-2 (||tiled|| + ||full||); the vector of singular values moves by at
  most the Frobenius error (Hoffman-Wielandt), which bounds the change of
  the spectral moments.
* The spectral moments the library computes with its own kernels against
  closed forms for matrices with known singular values (fp32: 1e-5).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import diagnostics as OD
import tiled_newton_schulz_amd as H
from tiled_newton_schulz_amd import diagnostics as GD
import workloads

pytestmark = pytest.mark.gpu

COEFFS = (3.4445, -4.7750, 2.0315)


def say(msg):
    print(msg, flush=True)


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_stats(a_list, b_list, got):
    got = got.cpu().numpy()
    for i, (a, b) in enumerate(zip(a_list, b_list)):
        A, B = host(a), host(b)
        want = OD.pair_stats(A, B)
        scale = (float(np.sum(np.abs(A * B))), want[1], want[2])
        for k in range(3):
            assert abs(got[i, k] - want[k]) <= 1e-12 * max(scale[k], 1e-300), (i, k, got[i, k], want[k])


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_pair_stats_shapes(cuda, dt):
    rng = np.random.default_rng([51, dt == "fp32"])
    shapes = [(1, 1), (3, 70000), (257, 129), (2048, 5632), (5632, 2048), (33, 7), (96, 160)]
    a = [workloads.round_to(rng.standard_normal(s), dt).to(cuda) for s in shapes]
    b = [workloads.round_to(rng.standard_normal(s), dt).to(cuda) for s in shapes]
    say(f"pair stats {dt}: {len(shapes)} pairs")
    st = H.himuon_pair_stats(a, b)
    torch.cuda.synchronize()
    check_stats(a, b, st)
    # a pair with itself: the three sums are equal
    st2 = H.himuon_pair_stats(a[:3], a[:3]).cpu().numpy()
    assert np.all(st2[:, 0] == st2[:, 1]) and np.all(st2[:, 1] == st2[:, 2])


def test_pair_stats_strided_views_and_many_pairs(cuda):
    """Column blocks of wider tensors (odd offsets: no 16-byte path), padded
    row strides, transposed views on both sides, and more pairs than one
    launch takes (300 > 128)."""
    rng = np.random.default_rng([52, 1])
    big_a = workloads.round_to(rng.standard_normal((300, 1031)), "bf16").to(cuda)
    big_b = workloads.round_to(rng.standard_normal((300, 1031)), "bf16").to(cuda)
    a = [big_a[:, 3:500], big_a[17:, 600:1031], big_a.t()[5:400, :200]]
    b = [big_b[:, 1:498], big_b[:283, 0:431], big_b.t()[100:495, 50:250]]
    say("pair stats on strided views")
    check_stats(a, b, H.himuon_pair_stats(a, b))
    with pytest.raises(ValueError):
        H.himuon_pair_stats([big_a[:100, :100]], [big_b.t()[:100, :100]])
    many_a = [workloads.round_to(rng.standard_normal((int(rng.integers(1, 90)), int(rng.integers(1, 90)))), "bf16")
              for _ in range(300)]
    many_b = [workloads.round_to(rng.standard_normal(x.shape), "bf16") for x in many_a]
    ga, gb = [x.to(cuda) for x in many_a], [x.to(cuda) for x in many_b]
    say("pair stats on 300 small pairs")
    check_stats(ga, gb, H.himuon_pair_stats(ga, gb))


def test_pair_stats_deterministic(cuda):
    rng = np.random.default_rng([53, 0])
    a = [workloads.round_to(rng.standard_normal((2048, 2048)), "bf16").to(cuda) for _ in range(3)]
    b = [x * 0.5 + 0.1 for x in a]
    s1 = H.himuon_pair_stats(a, b).cpu()
    s2 = H.himuon_pair_stats(a, b).cpu()
    assert torch.equal(s1, s2)


@pytest.mark.parametrize("shape,Ts", [((192, 320), [16, 32, 64, 128, 320]), ((300, 130), [32, 64, 100, 300])])
def test_tiled_vs_full_against_oracle(cuda, shape, Ts):
    rng = np.random.default_rng([54, shape[0]])
    x = workloads.round_to(rng.standard_normal(shape), "bf16")
    g = x.to(cuda)
    say(f"diagnostics {shape} T={Ts}")
    res = GD.tiled_vs_full([g], Ts, K=5, abc=COEFFS, spectrum=True)
    assert torch.equal(g.cpu(), x)                     # inputs untouched
    X = x.double().numpy()
    ref = OD.tiled_vs_full(X, Ts, [COEFFS] * 5, with_spectrum=True)
    full_ref = oracle.full_matrix_ns(X, [COEFFS] * 5)
    # the full map the library used, rebuilt for the exact checks
    full_gpu = g.clone()
    H.himuon_tiled_ns([full_gpu], res["full_T"], 5, COEFFS)
    F = host(full_gpu)
    for row, rr in zip(res["rows"], ref):
        T = row["T"]
        tg = g.clone()
        H.himuon_tiled_ns([tg], T, 5, COEFFS)
        Tm = host(tg)
        # exact: the measures of the library's own outputs
        assert row["distance"] == pytest.approx(OD.rel_distance(Tm, F), rel=1e-9, abs=1e-12)
        assert row["cosine"] == pytest.approx(OD.cosine(Tm, F), rel=1e-9)
        # end to end against the fp64 maps
        t_ref = oracle.tiled_ns(X, T, [COEFFS] * 5)
        slack = 3e-2 * (np.linalg.norm(t_ref) + np.linalg.norm(full_ref)) / np.linalg.norm(full_ref)
        say(f"  T={T}: distance {row['distance']:.4f} (oracle {rr['distance']:.4f}), cosine {row['cosine']:.4f}")
        assert abs(row["distance"] - rr["distance"]) <= slack + 3e-2
        check_moments(row["moments"][0], t_ref)
        if T >= max(shape):
            assert row["distance"] == 0.0 and row["cosine"] == pytest.approx(1.0, abs=1e-15)
    check_moments(res["full_moments"][0], full_ref)


def check_moments(got, ref_out):
    """Moments of a library output against those of the oracle's output: the
    singular values s (library) and t (oracle) satisfy ||s - t||_2 <= delta =
    3e-2 ||ref||_F, so |sum s^k - sum t^k| <= k M^(k-1) sqrt(r) delta."""
    want = OD.spectral_moments(ref_out)
    r = want[0]
    delta = 3e-2 * np.linalg.norm(ref_out)
    M = OD.spectrum(ref_out)[0] + delta
    assert got[0] == r
    for i, k in ((1, 2), (2, 4), (3, 6)):
        assert abs(got[i] - want[i]) <= k * M ** (k - 1) * math.sqrt(r) * delta, (k, got[i], want[i])


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_spectral_moments_closed_form(cuda, dt):
    """Matrices U diag(s) V^T with known s (several shapes in one call, a zero
    matrix among them): the library's moments against sum s^k, and its
    orthogonality residual against RMS(s^2 - 1)."""
    rng = np.random.default_rng([55, dt == "fp32"])
    mats, want = [], []
    for h, w in [(64, 96), (300, 130), (1, 40), (513, 512), (2048, 640)]:
        k = min(h, w)
        U, _ = np.linalg.qr(rng.standard_normal((h, k)))
        V, _ = np.linalg.qr(rng.standard_normal((w, k)))
        s = rng.uniform(0.3, 1.7, k)
        x = workloads.round_to((U * s) @ V.T, dt)
        mats.append(x.to(cuda))
        want.append(OD.spectral_moments(x.double().numpy()))   # of the rounded matrix
    mats.append(torch.zeros((40, 70), dtype=mats[0].dtype, device=cuda))
    want.append((40, 0.0, 0.0, 0.0))
    got = GD.spectral_moments(mats)
    for g_, w_ in zip(got, want):
        say(f"moments r={w_[0]}: {g_[1]:.6g} {g_[2]:.6g} {g_[3]:.6g} (want {w_[1]:.6g} {w_[2]:.6g} {w_[3]:.6g})")
        assert g_[0] == w_[0]
        for i in (1, 2, 3):
            assert abs(g_[i] - w_[i]) <= 1e-5 * max(w_[i], 1e-30)
        assert GD.orthogonality_residual(g_) == pytest.approx(OD.orthogonality_residual(w_), rel=1e-3, abs=1e-6)
