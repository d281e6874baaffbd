"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Per-tile relative Frobenius error, max over the tiles checked:
<= 3e-2 for bf16 data and <= 1e-4 for fp32 data.  Small cases are compared
tile by tile over the whole matrix; the full-size workloads are compared on
sampled tiles (edge tiles always included), with the input tiles copied to
the host before the in-place call.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from workloads import COEFFS, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = {"bf16": 3e-2, "fp32": 1e-4}
MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3), (3.0, -3.2, 1.2)]


def say(msg):
    print(msg, flush=True)


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run(mats, T, K=5, abc=COEFFS, cap=None):
    H.himuon_tiled_ns(mats, T, K, abc, workspace_bytes=cap)
    torch.cuda.synchronize()


def full_check(x_host, T, dt, K=5, abc=COEFFS, cap=None, device="cuda"):
    """Run one matrix on the GPU and compare every tile with the oracle."""
    ref = oracle.tiled_ns(x_host.double().numpy(), T, abc, K=K)
    g = x_host.to(device)
    run([g], T, K, abc, cap)
    err = oracle.tile_rel_errors(to_np(g), ref, T)
    return err.max(), g


def sample_tiles(H_, W_, T, n, rng):
    th, tw = math.ceil(H_ / T), math.ceil(W_ / T)
    pick = {(th - 1, tw - 1), (0, 0), (th - 1, 0), (0, tw - 1)}
    while len(pick) < min(n, th * tw):
        pick.add((int(rng.integers(th)), int(rng.integers(tw))))
    return sorted(pick)


def check_sampled(inputs_host_tiles, outputs, T, coeffs, K, tol):
    """inputs_host_tiles: list of (matrix index, ti, tj, tile float64)."""
    worst = 0.0
    for mi, ti, tj, tile in inputs_host_tiles:
        ref = oracle.ns_map(tile, coeffs, K=K)
        h, w = tile.shape
        got = to_np(outputs[mi][ti * T:ti * T + h, tj * T:tj * T + w])
        worst = max(worst, oracle.tile_rel_error(got, ref))
    assert worst <= tol, worst
    return worst


def grab(mats, T, per_matrix, rng, which=None):
    out = []
    for mi, m in enumerate(mats):
        if which is not None and mi not in which:
            continue
        Hh, Ww = m.shape
        for ti, tj in sample_tiles(Hh, Ww, T, per_matrix, rng):
            tile = to_np(m[ti * T:min(ti * T + T, Hh), tj * T:min(tj * T + T, Ww)])
            out.append((mi, ti, tj, tile))
    return out


# ---------------------------------------------------------------- small cases
@pytest.mark.parametrize("T", [64, 128])
def test_fp32_256x512_seed0(cuda, T):
    w = WORKLOADS["fp32_256x512"]
    x = workloads.host_tensors(w)[0]
    say(f"fp32 256x512 T={T}")
    err, _ = full_check(x, T, "fp32")
    say(f"  max err {err:.3e}")
    assert err <= TOL["fp32"]


SHAPES = [(1, 1), (7, 300), (300, 7), (33, 65), (128, 128), (200, 150), (129, 257), (300, 299)]


@pytest.mark.parametrize("T", [16, 32, 40, 64, 100, 128])
def test_bf16_on_chip_shapes(cuda, T):
    rng = np.random.default_rng([11, T])
    for (h, w) in SHAPES:
        x = workloads.round_to(rng.standard_normal((h, w)), "bf16")
        err, _ = full_check(x, T, "bf16")
        say(f"bf16 {h}x{w} T={T}: {err:.3e}")
        assert err <= TOL["bf16"], (h, w, T, err)


@pytest.mark.parametrize("T", [256, 4096])
def test_bf16_kernel_tile_256_shapes(cuda, T):
    """Tiles whose larger side is 129..256 (zero padded to 256 x 256 on chip),
    including thin, ragged and transposed shapes.  Short sides of 32..47
    (256 x 32, 32 x 256, 171 x 40) take the fp32 step path instead, and 256 x 48
    is the thinnest such tile on chip."""
    rng = np.random.default_rng([25, T])
    # (the shorter side <= 128 runs the narrow variant; a tall one is transposed)
    for (h, w) in [(256, 256), (256, 32), (32, 256), (200, 150), (130, 256), (256, 129), (171, 40), (97, 230),
                   (256, 48), (48, 200),
                   (128, 256), (256, 128), (129, 128), (128, 129)]:
        x = workloads.round_to(rng.standard_normal((h, w)), "bf16")
        err, _ = full_check(x, T, "bf16")
        say(f"bf16 {h}x{w} T={T}: {err:.3e}")
        assert err <= TOL["bf16"], (h, w, T, err)


@pytest.mark.parametrize("T", [160, 256, 512, 4096])
def test_bf16_large_tile_shapes(cuda, T):
    """bf16 tiles on the step path, whose workspace is laid out in 32-column
    slabs: padded row lengths of 304, 136, 264, 520 and 600/704 leave a last
    slab of 16, 8 or 24 columns (or none), tall tiles (600 x 130) are stored
    transposed, and T = 160 / 256 put the same shapes on chip for contrast."""
    rng = np.random.default_rng([12, T])
    for (h, w) in [(300, 299), (129, 600), (600, 130), (513, 257), (700, 520)]:
        x = workloads.round_to(rng.standard_normal((h, w)), "bf16")
        err, _ = full_check(x, T, "bf16")
        say(f"bf16 {h}x{w} T={T}: {err:.3e}")
        assert err <= TOL["bf16"], (h, w, T, err)


@pytest.mark.parametrize("T", [8, 32, 64, 128, 256, 1000])
def test_fp32_shapes(cuda, T):
    rng = np.random.default_rng([13, T])
    for (h, w) in [(1, 1), (33, 65), (200, 150), (300, 299), (129, 600)]:
        x = workloads.round_to(rng.standard_normal((h, w)), "fp32")
        err, _ = full_check(x, T, "fp32")
        say(f"fp32 {h}x{w} T={T}: {err:.3e}")
        assert err <= TOL["fp32"], (h, w, T, err)


@pytest.mark.parametrize("dt,T", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("fp32", 64)])
@pytest.mark.parametrize("K", [0, 1, 2, 5])
def test_step_counts_and_mixed_coefficients(cuda, dt, T, K):
    rng = np.random.default_rng([14, K, T])
    x = workloads.round_to(rng.standard_normal((2 * T + 17, T + 9)), dt)
    err, _ = full_check(x, T, dt, K=K, abc=MIXED[:K] if K else [])
    say(f"{dt} K={K} T={T}: {err:.3e}")
    assert err <= TOL[dt]


@pytest.mark.parametrize("eps", [0.0, 1e-3])
def test_eps_argument(cuda, eps):
    """eps is added to each tile's Frobenius norm: inputs scaled so that the
    tile norms are about 1e-2, where eps = 1e-3 changes the result by about
    10 %, on every route (kernel tiles 64, 128 and 256, the bf16 and fp32 step
    paths, the Gram iteration)."""
    rng = np.random.default_rng([39, int(eps * 1e4)])
    for shape, T, dt in [((200, 150), 64, "bf16"), ((300, 260), 128, "bf16"), ((300, 200), 256, "bf16"),
                         ((600, 520), 512, "bf16"), ((200, 150), 64, "fp32")]:
        x = workloads.round_to(rng.standard_normal(shape) * (1e-2 / min(T, shape[0])), dt)
        ref = oracle.tiled_ns(x.double().numpy(), T, COEFFS, eps=eps, K=5)
        g = x.cuda()
        H.himuon_tiled_ns([g], T, 5, COEFFS, eps=eps)
        torch.cuda.synchronize()
        err = oracle.tile_rel_errors(to_np(g), ref, T).max()
        off = oracle.tile_rel_errors(oracle.tiled_ns(x.double().numpy(), T, COEFFS, eps=1e-7 if eps else 1e-3, K=5),
                                     ref, T).max()
        say(f"eps={eps} {dt} {shape} T={T}: {err:.3e} (the other eps is {off:.3e} away)")
        assert err <= TOL[dt] and off > 3 * TOL[dt] * (eps > 0)
    from oracle.gram_ns import gram_ns
    x = workloads.round_to(rng.standard_normal((300, 900)) * (1e-2 / 300), "bf16")
    ref = gram_ns(x.double().numpy(), [COEFFS] * 5, restart=2, eps=eps)
    g = x.cuda()
    H.himuon_gram_ns([g], 5, COEFFS, restart=2, eps=eps)
    torch.cuda.synchronize()
    err = float(np.linalg.norm(to_np(g) - ref) / np.linalg.norm(ref))
    say(f"eps={eps} gram: {err:.3e}")
    assert err <= TOL["bf16"]


STEPS16 = [COEFFS] * 5 + [(1.5, -0.5, 0.0)] * 11


@pytest.mark.parametrize("shape,T,dt", [((300, 260), 128, "bf16"), ((300, 200), 256, "bf16"),
                                        ((600, 520), 512, "bf16"), ((130, 40), 64, "bf16"), ((300, 260), 32, "bf16"),
                                        ((300, 260), 64, "fp32"), ((300, 260), 128, "fp32")])
def test_max_steps(cuda, shape, T, dt):
    """K = 16, the largest step count, on every route (kernel tiles 32, 128
    and 256, the step path with bf16 and fp32 workspaces, split precision,
    fp32 tiles on chip and on the step path): five quintic steps, then eleven
    cubic ones (1.5, -0.5, 0), on a few tiles.  Over many tiles the bf16
    iterate of kernel tiles 64 and up exceeds the bound on a tail of them
    (test_gpu_precision.py pins that)."""
    rng = np.random.default_rng([37, T])
    x = workloads.round_to(rng.standard_normal(shape), dt)
    err, _ = full_check(x, T, dt, K=16, abc=STEPS16)
    say(f"K=16 {dt} {shape} T={T}: {err:.3e}")
    assert err <= TOL[dt]


# steps with c = 0 (the cubic iteration) mixed with quintic ones
CUBIC_MIX = [(1.5, -0.5, 0.0), (3.4445, -4.7750, 2.0315), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]


@pytest.mark.parametrize("dt,T", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("bf16", 512),
                                  ("fp32", 64)])
def test_steps_without_quintic_term(cuda, dt, T):
    rng = np.random.default_rng([26, T])
    x = workloads.round_to(rng.standard_normal((2 * T + 17, T + 9)), dt)
    err, _ = full_check(x, T, dt, K=5, abc=CUBIC_MIX)
    say(f"{dt} c=0 steps T={T}: {err:.3e}")
    assert err <= TOL[dt]


# One or two steps with other signs than the quintic's: c < 0, b = 0, b > 0,
# a = 0.  So few steps do not converge, so a wrong sign or scale of any term
# shows as an error of order one, not as a small change of a converged result.
SIGN_STEPS = [
    [(1.5, -0.7, -0.1)],
    [(1.5, -0.7, -0.1), (2.0, -1.2, 0.3)],
    [(1.2, 0.0, 0.4)],
    [(1.0, 0.5, 0.0)],
    [(0.0, 1.0, 0.0)],
    [(0.5, 0.3, -0.2), (1.5, -0.5, 0.0)],
]


@pytest.mark.parametrize("T", [8, 32, 64, 128, 256, 512])
def test_coefficient_signs(cuda, T):
    rng = np.random.default_rng([62, T])
    x = workloads.round_to(rng.standard_normal((2 * T + 17, T + 9)), "bf16")
    for steps in SIGN_STEPS:
        err, _ = full_check(x, T, "bf16", K=len(steps), abc=steps)
        say(f"T={T} steps {steps}: {err:.3e}")
        assert err <= 1e-2, (steps, err)


def test_steps_without_quintic_term_one_wave_kernel(cuda):
    """Enough 128-tiles that most run in the one-wave kernel (a small call runs
    in the eight-wave kernel only)."""
    rng = np.random.default_rng(27)
    x = workloads.round_to(rng.standard_normal((128 * 4, 128 * 400)), "bf16").cuda()
    sampled = grab([x], 128, 40, rng)
    run([x], 128, K=5, abc=CUBIC_MIX)
    worst = check_sampled(sampled, [x], 128, CUBIC_MIX, 5, TOL["bf16"])
    say(f"  max err {worst:.3e}")


def test_zero_and_tiny_tiles(cuda):
    for dt in ("bf16", "fp32"):
        for T in (32, 64, 256):
            x = torch.zeros(300, 200, dtype=torch.bfloat16 if dt == "bf16" else torch.float32)
            tw = min(T, 200)
            x[:T, :tw] = workloads.round_to(np.random.default_rng(3).standard_normal((T, tw)) * 1e-3, dt)
            err, g = full_check(x, T, dt)
            assert err <= TOL[dt]
            assert torch.count_nonzero(g[T:, :]) == 0 and torch.count_nonzero(g[:, tw:]) == 0


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("dt,T", [("bf16", 32), ("bf16", 128), ("bf16", 256), ("fp32", 64)])
def test_deterministic_and_tile_independent(cuda, dt, T):
    rng = np.random.default_rng([15, T])
    x = workloads.round_to(rng.standard_normal((3 * T + 5, 2 * T + 3)), dt).cuda()
    a, b = x.clone(), x.clone()
    run([a], T)
    run([b], T)
    assert torch.equal(a, b), "two runs differ"
    c = x.clone()
    c[T:2 * T, T:2 * T] *= -1.5
    c[T + 3, T + 4] = float("nan")
    run([c], T)
    mask = torch.zeros_like(c, dtype=torch.bool)
    mask[T:2 * T, T:2 * T] = True
    assert torch.equal(a[~mask], c[~mask]), "a change in one tile leaked into others"
    assert torch.isnan(c[mask]).all()


@pytest.mark.parametrize("dt,T", [("bf16", 64), ("bf16", 256), ("fp32", 64), ("fp32", 128)])
def test_transposed_view_and_batch(cuda, dt, T):
    rng = np.random.default_rng([16, T])
    xs = [workloads.round_to(rng.standard_normal(s), dt).cuda() for s in [(300, 170), (170, 300), (64, 64)]]
    ref = [x.clone() for x in xs]
    for r in ref:
        run([r], T)
    batch = [x.clone() for x in xs]
    run(batch, T)
    for r, b_ in zip(ref, batch):
        assert torch.equal(r, b_), "batched call differs from single calls"
    # a transposed view is processed as the transpose of its storage
    base = xs[0].clone()
    view = base.t()
    run([view], T)
    expect = xs[0].clone()
    run([expect], T)
    assert torch.equal(base, expect)


def test_column_blocks_of_fused_tensor(cuda):
    """Sub-matrix descriptors (functional blocks of a fused Q|K|V tensor) are
    processed as separate matrices, in one call."""
    rng = np.random.default_rng(17)
    fused = workloads.round_to(rng.standard_normal((256, 3 * 192)), "bf16").cuda()
    parts = [fused[:, i * 192:(i + 1) * 192] for i in range(3)]
    sep = [p.clone() for p in parts]
    run(sep, 64)
    run(parts, 64)
    for p, s_ in zip(parts, sep):
        assert torch.equal(p, s_)


@pytest.mark.parametrize("T", [256, 512])
@pytest.mark.parametrize("cap_tiles", [1, 3, 7])
def test_chunking_bit_exact(cuda, T, cap_tiles):
    rng = np.random.default_rng([18, cap_tiles])
    xs = [workloads.round_to(rng.standard_normal(s), "bf16").cuda() for s in [(600, 520), (257, 513), (1100, 1030)]]
    full, mn = H.himuon_workspace_size(xs, T, H.BF16)
    assert mn > 0
    a = [x.clone() for x in xs]
    run(a, T)
    b = [x.clone() for x in xs]
    run(b, T, cap=mn * cap_tiles)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ------------------------------------------------------------- Muon step
@pytest.mark.parametrize("dt,T,shape", [("bf16", 64, (300, 170)), ("bf16", 128, (300, 170)),
                                        ("bf16", 256, (300, 170)), ("bf16", 256, (250, 100)),
                                        ("fp32", 64, (300, 170)), ("fp32", 256, (300, 170))])
@pytest.mark.parametrize("K", [0, 5])
def test_muon_step(cuda, dt, T, shape, K):
    rng = np.random.default_rng([19, T, K])
    W = workloads.round_to(rng.standard_normal(shape), dt)
    M = workloads.round_to(rng.standard_normal(shape), dt)
    G = workloads.round_to(rng.standard_normal(shape), dt)
    mu, eta = 0.95, 0.02
    Wg, Mg, Gg = W.cuda(), M.cuda(), G.cuda()
    H.himuon_muon_step([Wg], [Mg], [Gg], T, K, COEFFS, mu=mu, eta=eta)
    torch.cuda.synchronize()
    # momentum: mu M + G rounded once to the dtype; the device evaluates the sum
    # in fp32, so allow one ulp of the result plus the fp32 evaluation error
    # (which matters where mu M and G nearly cancel)
    mM, gG = mu * M.double(), G.double()
    m_new = workloads.round_to((mM + gG).numpy(), dt).double()
    bound = m_new.abs() * (2.0 ** -7 if dt == "bf16" else 2.0 ** -23) + 2.0 ** -22 * (mM.abs() + gG.abs())
    assert bool(((Mg.cpu().double() - m_new).abs() <= bound).all()), "momentum differs beyond rounding"
    # weights: W - eta * tiledNS(M) with M as stored; per tile the difference
    # is bounded by W's own rounding plus eta times the map's tolerance
    U = oracle.tiled_ns(Mg.cpu().double().numpy(), T, COEFFS, K=K)
    want = W.double().numpy() - eta * U
    got = Wg.cpu().double().numpy()
    half_ulp = np.abs(want) * (2.0 ** -8 if dt == "bf16" else 2.0 ** -24)
    worst = 0.0
    for r0, r1, c0, c1 in oracle.tile_grid(*shape, T):
        d = np.linalg.norm(got[r0:r1, c0:c1] - want[r0:r1, c0:c1])
        bound = np.linalg.norm(half_ulp[r0:r1, c0:c1]) + eta * TOL[dt] * np.linalg.norm(U[r0:r1, c0:c1])
        worst = max(worst, d / bound)
    say(f"muon {dt} T={T} K={K}: worst difference / bound = {worst:.3f}")
    assert worst <= 1.0


def check_muon(W, M, G, Wg, Mg, dt, T, K, mu, eta, tiles=None):
    """Momentum within one rounding of mu M + G; weights within W's rounding
    plus eta times the map's tolerance per tile (tiles: (r0, r1, c0, c1)
    to check, default all).  Returns the worst difference / bound."""
    mM, gG = mu * M.double(), G.double()
    m_new = workloads.round_to((mM + gG).numpy(), dt).double()
    bound = m_new.abs() * (2.0 ** -7 if dt == "bf16" else 2.0 ** -23) + 2.0 ** -22 * (mM.abs() + gG.abs())
    assert bool(((Mg.cpu().double() - m_new).abs() <= bound).all()), "momentum differs beyond rounding"
    Mh = Mg.cpu().double().numpy()
    got = Wg.cpu().double().numpy()
    Wd = W.double().numpy()
    worst = 0.0
    for r0, r1, c0, c1 in (tiles if tiles is not None else oracle.tile_grid(*Mh.shape, T)):
        U = oracle.ns_map(Mh[r0:r1, c0:c1], COEFFS, K=K)
        want = Wd[r0:r1, c0:c1] - eta * U
        half_ulp = np.abs(want) * (2.0 ** -8 if dt == "bf16" else 2.0 ** -24)
        d = np.linalg.norm(got[r0:r1, c0:c1] - want)
        worst = max(worst, d / (np.linalg.norm(half_ulp) + eta * TOL[dt] * np.linalg.norm(U)))
    return worst


@pytest.mark.parametrize("K", [0, 1, 2])
@pytest.mark.parametrize("dt", ["bf16", "fp32", "bf16_precise"])
def test_step_path_short_runs(cuda, dt, K):
    """The step path with K = 0, 1 and 2.  The normalisation pass writes the
    tiles unscaled and the first Gram and apply products apply each tile's
    scale; with K = 1 both happen in the last step, whose apply writes the
    result in place (a tall matrix's tiles transposed back).  T = 512 (tiles
    with ragged edges) and T = 1024 (one tile per matrix), wide and tall;
    bf16_precise is bf16 storage on the fp32 workspace."""
    rng = np.random.default_rng([61, K, len(dt)])
    io = "fp32" if dt == "fp32" else "bf16"
    for (h, w) in [(700, 520), (520, 700)]:
        x = workloads.round_to(rng.standard_normal((h, w)) * 3.0, io)
        for T in (512, 1024):
            g = x.cuda()
            H.himuon_tiled_ns([g], T, K, MIXED[:K] if K else [], precise=(dt == "bf16_precise"))
            torch.cuda.synchronize()
            ref = oracle.tiled_ns(x.double().numpy(), T, MIXED[:K] if K else [], K=K)
            err = float(oracle.tile_rel_errors(to_np(g), ref, T).max())
            say(f"{dt} {h}x{w} T={T} K={K}: {err:.3e}")
            assert err <= TOL["fp32" if dt == "fp32" else "bf16"], (h, w, T, err)


@pytest.mark.parametrize("K", [1, 2])
def test_muon_step_on_step_path_short_runs(cuda, K):
    """The fused Muon step on the step path with K = 1 and 2: the momentum is
    written unscaled by the normalisation pass, and with K = 1 the first
    apply is also the one that writes W <- W - eta X."""
    rng = np.random.default_rng([62, K])
    shape = (700, 1100)
    W, M, G = (workloads.round_to(rng.standard_normal(shape), "bf16") for _ in range(3))
    Wg, Mg, Gg = W.cuda(), M.cuda(), G.cuda()
    mu, eta = 0.95, 0.02
    H.himuon_muon_step([Wg], [Mg], [Gg], 512, K, COEFFS, mu=mu, eta=eta)
    torch.cuda.synchronize()
    worst = check_muon(W, M, G, Wg, Mg, "bf16", 512, K, mu, eta)
    say(f"muon bf16 {shape} T=512 K={K}: worst difference / bound = {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("shape,T", [((1100, 1030), 512), ((2100, 2100), 2100), ((1030, 2100), 2100)])
def test_muon_step_on_step_path(cuda, shape, T):
    """The fused Muon step where the last product writes W <- W - eta X from
    the bf16 step GEMM: 512-tiles with edges (128 x 128 blocks) and
    whole-matrix tiles of side 2100, whose apply runs 256 x 256 blocks (a
    wide one, and a square one written back in place untransposed)."""
    rng = np.random.default_rng([29, T, shape[0]])
    W, M, G = (workloads.round_to(rng.standard_normal(shape), "bf16") for _ in range(3))
    Wg, Mg, Gg = W.cuda(), M.cuda(), G.cuda()
    mu, eta = 0.95, 0.02
    H.himuon_muon_step([Wg], [Mg], [Gg], T, 5, COEFFS, mu=mu, eta=eta)
    torch.cuda.synchronize()
    worst = check_muon(W, M, G, Wg, Mg, "bf16", T, 5, mu, eta)
    say(f"muon bf16 {shape} T={T}: worst difference / bound = {worst:.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("dt,T", [("bf16", 128), ("bf16", 512), ("fp32", 64)])
def test_muon_step_row_strides(cuda, dt, T):
    """W, M and G with different row strides (column blocks of wider buffers,
    at column offsets that break 16-byte alignment): the same bits as with
    contiguous matrices."""
    rng = np.random.default_rng([41, T])
    shape = (600, 530)
    W, M, G = (workloads.round_to(rng.standard_normal(shape), dt) for _ in range(3))
    a = [W.cuda(), M.cuda(), G.cuda()]
    H.himuon_muon_step([a[0]], [a[1]], [a[2]], T, 5, COEFFS, mu=0.9, eta=0.01)
    bw = torch.zeros((600, 700), dtype=W.dtype, device=cuda)
    bg = torch.zeros((600, 611), dtype=W.dtype, device=cuda)
    Wv, Gv = bw[:, 13:13 + 530], bg[:, 3:3 + 530]
    Wv.copy_(W.cuda())
    Gv.copy_(G.cuda())
    Mc = M.cuda()
    H.himuon_muon_step([Wv], [Mc], [Gv], T, 5, COEFFS, mu=0.9, eta=0.01)
    torch.cuda.synchronize()
    assert torch.equal(Wv, a[0]) and torch.equal(Mc, a[1]) and torch.equal(Gv, a[2])
    # outside the views the buffers are untouched
    assert bw[:, :13].abs().sum().item() == 0 and bw[:, 543:].abs().sum().item() == 0
    assert bg[:, :3].abs().sum().item() == 0 and bg[:, 533:].abs().sum().item() == 0


def test_muon_step_layer_d2048(cuda):
    """The fused Muon step on one transformer layer at d = 2048, T = 128 (the
    Muon variant of the one-wave kernel, one workgroup per tile), with 16
    sampled tiles per matrix checked."""
    w = WORKLOADS["layer_d2048"]
    Ms = workloads.host_tensors(w)
    rng = np.random.default_rng(31)
    Ws = [workloads.round_to(rng.standard_normal(tuple(m.shape)) * 0.02, "bf16") for m in Ms]
    Gs = [workloads.round_to(rng.standard_normal(tuple(m.shape)), "bf16") for m in Ms]
    Wg, Mg, Gg = [x.cuda() for x in Ws], [x.cuda() for x in Ms], [x.cuda() for x in Gs]
    mu, eta = 0.95, 0.02
    H.himuon_muon_step(Wg, Mg, Gg, 128, 5, COEFFS, mu=mu, eta=eta)
    torch.cuda.synchronize()
    worst = 0.0
    for i in range(len(Ms)):
        Hh, Ww = Ms[i].shape
        tiles = [(ti * 128, min(ti * 128 + 128, Hh), tj * 128, min(tj * 128 + 128, Ww))
                 for ti, tj in sample_tiles(Hh, Ww, 128, 16, rng)]
        worst = max(worst, check_muon(Ws[i], Ms[i], Gs[i], Wg[i], Mg[i], "bf16", 128, 5, mu, eta, tiles))
    say(f"muon layer_d2048 T=128: worst difference / bound = {worst:.3f}")
    assert worst <= 1.0


# ------------------------------------------------------------- workloads
def test_layer_d2048(cuda):
    """One transformer layer (Q, K, V, O, MLP x3) at T = 128, one launch."""
    w = WORKLOADS["layer_d2048"]
    mats = [t.cuda() for t in workloads.host_tensors(w)]
    rng = np.random.default_rng(21)
    sampled = grab(mats, 128, 40, rng)
    say(f"layer_d2048: {len(sampled)} sampled tiles")
    run(mats, 128)
    worst = check_sampled(sampled, mats, 128, COEFFS, 5, TOL["bf16"])
    say(f"  max err {worst:.3e}")


@pytest.mark.parametrize("T", [32, 64, 128, 256])
def test_layers24_d2048(cuda, T):
    w = WORKLOADS["layers24_d2048"]
    mats = workloads.device_tensors(w)
    rng = np.random.default_rng([22, T])
    which = set(int(i) for i in rng.choice(len(mats), 12, replace=False)) | {0, 6, 167}
    sampled = grab(mats, T, 12, rng, which)
    say(f"layers24 T={T}: {len(sampled)} sampled tiles")
    run(mats, T)
    worst = check_sampled(sampled, mats, T, COEFFS, 5, TOL["bf16"])
    say(f"  max err {worst:.3e}")


def test_layers24_full_matrix(cuda):
    """The full-matrix map (T = max dims) on the 24-layer batch; three
    matrices (one of each shape) are checked against the oracle."""
    w = WORKLOADS["layers24_d2048"]
    mats = workloads.device_tensors(w)
    idx = [3, 4, 6]
    host = {i: to_np(mats[i]) for i in idx}
    say("layers24 full-matrix")
    run(mats, 5632)
    for i in idx:
        ref = oracle.full_matrix_ns(host[i], COEFFS, K=5)
        e = oracle.tile_rel_error(to_np(mats[i]), ref)
        say(f"  matrix {i} {host[i].shape}: {e:.3e}")
        assert e <= TOL["bf16"]


def test_moe64_ragged(cuda):
    w = WORKLOADS["moe64"]
    mats = workloads.device_tensors(w)
    rng = np.random.default_rng(23)
    sampled = grab(mats, 256, 10, rng, {0, 1, 62, 127})
    assert any(t.shape != (256, 256) for _, _, _, t in sampled)
    say(f"moe64: {len(sampled)} sampled tiles")
    run(mats, 256)
    worst = check_sampled(sampled, mats, 256, COEFFS, 5, TOL["bf16"])
    say(f"  max err {worst:.3e}")


@pytest.mark.parametrize("T", [128, 256, 512])
def test_dense8192_cap(cuda, T):
    w = WORKLOADS["dense8192"]
    mats = workloads.device_tensors(w)
    rng = np.random.default_rng([24, T])
    sampled = grab(mats, T, 6, rng)
    say(f"dense8192 T={T}: {len(sampled)} sampled tiles, cap 4 GiB")
    ref_mats = [m.clone() for m in mats] if T == 512 else None
    run(mats, T, cap=4 << 30)
    worst = check_sampled(sampled, mats, T, COEFFS, 5, TOL["bf16"])
    say(f"  max err {worst:.3e}")
    if ref_mats is not None:
        # chunked (4 GiB) and a single chunk give the same bits
        run(ref_mats, T, cap=1 << 40)
        for a, b in zip(mats, ref_mats):
            assert torch.equal(a, b)


def test_full_map_operand_past_2gib(cuda):
    """The full-matrix map of a 16384 x 65536 bf16 matrix: its oriented operand
    is 2 GiB, past the 32-bit buffer offsets of the DMA GEMM, so the step path
    runs its register-staged GEMM with 64-bit addressing.  A rank-one input
    u v^T with +-1 entries has a closed-form result (SVD view of the iteration,
    Gram Newton-Schulz page, section 3): its one singular value, normalised to
    ||Y||_F / (||Y||_F + eps), goes through the step polynomial, so every output
    element is +-p(s) / ||Y||_F with the input's sign.  Random signs make any
    misplaced element show."""
    from oracle import diagnostics as OD
    Hh, Ww = 16384, 65536
    g = torch.Generator(device="cpu").manual_seed(61)
    u = (torch.randint(0, 2, (Hh,), generator=g) * 2 - 1).to(torch.float32).to(cuda)
    v = (torch.randint(0, 2, (Ww,), generator=g) * 2 - 1).to(torch.float32).to(cuda)
    m = torch.outer(u, v).to(torch.bfloat16)
    plan = H.himuon_plan([m], max(Hh, Ww), 5, H.BF16, 16 << 30)
    assert plan["chunks"] == 1 and plan["resident_launches"] == 0
    say(f"full map of {Hh}x{Ww} bf16 (operand {Hh * Ww * 2 / 2**30:.1f} GiB)")
    run([m], max(Hh, Ww))
    norm = math.sqrt(Hh * Ww)
    s = float(OD.scalar_map(norm / (norm + oracle.EPS_DEFAULT), [COEFFS] * 5))
    got = m.float() * (norm / s)            # should be the +-1 pattern
    want = torch.outer(u, v)
    rel = (got - want).abs().max().item()
    say(f"  p(s) = {s:.6f}, worst element relative error {rel:.3e}")
    assert rel <= 3e-2
    del got, want, m
    torch.cuda.empty_cache()


def test_tail_split_bit_exact(cuda):
    """The partial last round of kernel-tile-128 tiles runs eight waves per tile;
    its arithmetic is the one-wave kernel's, so a batched call (3,072 tiles
    one-wave + 64 eight-wave) equals matrix-by-matrix calls bit for bit."""
    w = WORKLOADS["layer_d2048"]
    base = [t.cuda() for t in workloads.host_tensors(w)]
    batched = [b.clone() for b in base]
    run(batched, 128)
    for b, m in zip(base, batched):
        single = b.clone()
        run([single], 128)
        assert torch.equal(single, m)


@pytest.mark.parametrize("K", [1, 2, 3])
def test_grid_stride_small_k_bit_exact(cuda, K):
    """K = 1, 2 and 3 on the grid-stride launch, where the folded first step is
    also the last one (K = 1, which then issues the next tile's loads) or comes
    right before it.  1,875 tiles of 128 in one call run one wave per tile;
    matrix-by-matrix calls (at most 256 tiles each) run eight waves per tile
    with the same arithmetic, so the two agree bit for bit.  Sampled tiles,
    edges included, against the oracle."""
    rng = np.random.default_rng([44, K])
    shapes = [(2048, 2048), (1000, 1500), (2048, 2048), (300, 2100), (2048, 2048), (2048, 700),
              (2048, 2048), (1500, 1000), (2048, 2048), (2048, 2048)]
    base = [workloads.round_to(rng.standard_normal(s), "bf16").cuda() for s in shapes]
    abc = MIXED[:K]
    picks = grab(base, 128, 6, rng)
    batched = [b.clone() for b in base]
    run(batched, 128, K=K, abc=abc)
    worst = check_sampled(picks, batched, 128, abc, K, TOL["bf16"])
    say(f"K={K}: worst sampled tile error {worst:.3e}")
    for i, (b, m) in enumerate(zip(base, batched)):
        single = b.clone()
        run([single], 128, K=K, abc=abc)
        assert torch.equal(single, m), i


def test_muon_tail_split_bit_exact(cuda):
    """The fused Muon step on one layer (3,136 tiles: 3,072 one-wave, the last 64
    eight-wave) against matrix-by-matrix Muon steps, which split the tiles
    between the two kernels differently (a 2048 x 2048 matrix alone is a partial
    round, all eight-wave; the last matrix's final 64 tiles run one-wave): W and
    M equal bit for bit."""
    w = WORKLOADS["layer_d2048"]
    rng = np.random.default_rng([45, 1])
    Ms = [t.cuda() for t in workloads.host_tensors(w)]
    Gs = [workloads.round_to(rng.standard_normal(tuple(m.shape)), "bf16").cuda() for m in Ms]
    Ws = [workloads.round_to(rng.standard_normal(tuple(m.shape)), "bf16").cuda() for m in Ms]
    Wb, Mb = [x.clone() for x in Ws], [x.clone() for x in Ms]
    H.himuon_muon_step(Wb, Mb, Gs, 128, 5, COEFFS, mu=0.9, eta=0.02)
    for i in range(len(Ms)):
        W1, M1 = Ws[i].clone(), Ms[i].clone()
        H.himuon_muon_step([W1], [M1], [Gs[i]], 128, 5, COEFFS, mu=0.9, eta=0.02)
        torch.cuda.synchronize()
        assert torch.equal(M1, Mb[i]) and torch.equal(W1, Wb[i]), i


def test_grid_stride_ragged_mix_bit_exact(cuda):
    """More kernel-tile-128 tiles than the device holds at once (1,875), full
    and ragged tile classes mixed: each workgroup then walks several tiles,
    loading the next full tile during the last step of the current one.
    Matrix-by-matrix calls (at most 256 tiles each) run one tile per
    workgroup.  The arithmetic is the same, so the results are equal bit for
    bit."""
    rng = np.random.default_rng([43, 1])
    shapes = [(2048, 2048), (1000, 1500), (2048, 2048), (300, 2100), (2048, 2048), (2048, 700),
              (2048, 2048), (1500, 1000), (2048, 2048), (2048, 2048)]
    base = [workloads.round_to(rng.standard_normal(s), "bf16").cuda() for s in shapes]
    batched = [b.clone() for b in base]
    say("batched call, 1,875 tiles of 128")
    run(batched, 128)
    for i, (b, m) in enumerate(zip(base, batched)):
        single = b.clone()
        say(f"single call {i}: {tuple(b.shape)}")
        run([single], 128)
        assert torch.equal(single, m), i


# ------------------------------------------------------------- tile-size schedule
@pytest.mark.parametrize("dt,Ts", [("bf16", [512, 256, 128, 64, 64]), ("bf16", [256, 256, 128, 128, 32]),
                                   ("fp32", [256, 128, 64])])
def test_tile_size_schedule(cuda, dt, Ts):
    """Per-step tile sizes inside one call against the oracle's schedule."""
    rng = np.random.default_rng([28, len(Ts), Ts[0]])
    x = workloads.round_to(rng.standard_normal((600, 520)), dt)
    abc = MIXED[:len(Ts)]
    ref = oracle.tiled_ns_schedule(x.double().numpy(), Ts, abc)
    g = x.cuda()
    H.himuon_tiled_ns_schedule([g], Ts, abc)
    torch.cuda.synchronize()
    err = oracle.tile_rel_errors(to_np(g), ref, Ts[0]).max()
    say(f"{dt} schedule {Ts}: {err:.3e}")
    assert err <= TOL[dt]


def test_schedule_of_one_size_is_the_plain_map(cuda):
    rng = np.random.default_rng(29)
    x = workloads.round_to(rng.standard_normal((300, 700)), "bf16").cuda()
    a, b = x.clone(), x.clone()
    H.himuon_tiled_ns([a], 128, 5, MIXED)
    H.himuon_tiled_ns_schedule([b], [128] * 5, MIXED)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dense8192_schedule(cuda):
    """The dense layer with the per-step schedule 512, 256, 128, 128, 128 under
    the 4 GiB cap; sampled 512-tiles checked with the oracle's schedule (a
    512-tile's result depends on that tile alone)."""
    w = WORKLOADS["dense8192"]
    mats = workloads.device_tensors(w)
    Ts = [512, 256, 128, 128, 128]
    rng = np.random.default_rng(30)
    sampled = grab(mats, 512, 4, rng)
    H.himuon_tiled_ns_schedule(mats, Ts, COEFFS, workspace_bytes=4 << 30)
    torch.cuda.synchronize()
    worst = 0.0
    for mi, ti, tj, tile in sampled:
        ref = oracle.tiled_ns_schedule(tile, Ts, COEFFS)
        h, w_ = tile.shape
        got = to_np(mats[mi][ti * 512:ti * 512 + h, tj * 512:tj * 512 + w_])
        worst = max(worst, oracle.tile_rel_errors(got, ref, 512).max())
    say(f"dense8192 schedule: {len(sampled)} tiles, max err {worst:.3e}")
    assert worst <= TOL["bf16"]


# ------------------------------------------------------------- input scale
@pytest.mark.parametrize("scale_exp", [50, -50])
def test_scale_extremes_tile128(cuda, scale_exp):
    """Inputs scaled by 2^50 and 2^-50 (exact in bf16) at T = 128, where the
    normalisation is folded into the first step (s^2 A formed from the fp32
    X X^T of the raw tile): one 300 x 520 matrix (15 tiles; its full tiles
    and 44 x 128 edge tiles form a partial round for the eight-wave kernel, its
    8-column edge tiles take other paths) and 600 full tiles on the one-wave
    kernel.  Every tile against the oracle, which normalises in fp64."""
    rng = np.random.default_rng([97, scale_exp + 100])
    f = 2.0 ** scale_exp
    # eps scales with the data, so that it stays as small against the tile
    # norm as at unit scale and the folded normalisation itself is exercised
    eps = 1e-7 * f
    small = [workloads.round_to(rng.standard_normal((300, 520)) * f, "bf16")]
    big = [workloads.round_to(rng.standard_normal((640, 640)) * f, "bf16") for _ in range(24)]
    for name, hosts in (("15 tiles", small), ("600 tiles", big)):
        devs = [x.cuda() for x in hosts]
        H.himuon_tiled_ns(devs, 128, 5, COEFFS, eps=eps)
        torch.cuda.synchronize()
        worst = 0.0
        for x, d in zip(hosts, devs):
            ref = oracle.tiled_ns(x.double().numpy(), 128, COEFFS, eps=eps, K=5)
            worst = max(worst, float(oracle.tile_rel_errors(to_np(d), ref, 128).max()))
        say(f"scale 2^{scale_exp}, {name}: worst per-tile error {worst:.3e}")
        assert worst <= TOL["bf16"]


# ------------------------------------------------------------- error tails
@pytest.mark.parametrize("T,N", [(32, 48), (64, 48), (128, 24)])
def test_error_tail_over_many_tiles(cuda, T, N):
    """Worst per-tile error over tens of thousands of random bf16 tiles (N
    matrices of 1024 x 1024, every tile checked with the batched oracle): the
    sampled workload tests do not reach the tail of the error distribution."""
    gen = torch.Generator(device="cuda").manual_seed(31 + T)
    mats = [torch.randn(1024, 1024, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(N)]
    nt = 1024 // T

    def tiles_of(ms):
        a = np.stack([to_np(m) for m in ms])
        return a.reshape(N, nt, T, nt, T).transpose(0, 1, 3, 2, 4).reshape(-1, T, T)

    ref = oracle.ns_map_stack(tiles_of(mats), COEFFS, K=5)
    run(mats, T)
    got = tiles_of(mats)
    err = np.linalg.norm((got - ref).reshape(len(ref), -1), axis=1) / np.linalg.norm(ref.reshape(len(ref), -1), axis=1)
    say(f"T={T}: {len(err)} tiles, worst {err.max():.3e}, mean {err.mean():.3e}")
    assert err.max() <= TOL["bf16"]
