"""The precision contract of include/himuon.h, on the GPU against the oracle.

- HIMUON_BF16_PRECISE (bf16 storage, fp32 arithmetic) holds the 3e-2 bound
  where the bf16 arithmetic does not: tiles of low numerical rank and sixteen
  quintic steps in a row.
- The bf16 path's errors on those cases are pinned in a band around what was
  measured, so that a regression (or a fix) shows.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from workloads import COEFFS

pytestmark = pytest.mark.gpu

MIXED = [(3.4445, -4.7750, 2.0315), (2.8, -3.1, 1.2), (1.9, -1.3, 0.4), (1.6, -0.9, 0.3), (3.0, -3.2, 1.2)]


def say(msg):
    print(msg, flush=True)


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def low_rank_matrix(rng, nt, T, rank):
    """An (nt T) x (nt T) matrix whose every T-tile has rank `rank` (random
    Gaussian factors), rounded to bf16."""
    x = np.zeros((nt * T, nt * T))
    for i in range(nt):
        for j in range(nt):
            x[i * T:(i + 1) * T, j * T:(j + 1) * T] = rng.standard_normal((T, rank)) @ rng.standard_normal((rank, T))
    return workloads.round_to(x, "bf16")


def tile_errors(host, dev, T, coeffs, K):
    ref = oracle.tiled_ns(host.double().numpy(), T, coeffs, K=K)
    return oracle.tile_rel_errors(to_np(dev), ref, T)


@pytest.mark.parametrize("rank", [1, 2, 4, 8, 16])
def test_low_rank_tiles(cuda, rank):
    """Rank-r 128-tiles (64 per rank): the precise mode within the bound, the
    bf16 path outside it, in the band measured for it."""
    rng = np.random.default_rng([41, rank])
    hosts = [low_rank_matrix(rng, 4, 128, rank) for _ in range(4)]
    worst = {}
    for precise in (True, False):
        devs = [h.cuda() for h in hosts]
        H.himuon_tiled_ns(devs, 128, 5, COEFFS, precise=precise)
        torch.cuda.synchronize()
        worst[precise] = max(float(tile_errors(h, d, 128, COEFFS, 5).max()) for h, d in zip(hosts, devs))
    say(f"rank {rank}: precise {worst[True]:.3e}, bf16 {worst[False]:.3e}")
    assert worst[True] <= 3e-2
    assert worst[True] <= 5e-3          # fp32 arithmetic: the final bf16 rounding dominates
    # the bf16 path's known limit (include/himuon.h); measured 0.175-0.291
    assert 3e-2 < worst[False] < 0.6


@pytest.mark.parametrize("T", [64, 128, 256])
def test_sixteen_quintic_steps(cuda, T):
    """Sixteen quintic steps in a row: the precise mode within the bound; the
    bf16 path outside it, in the band measured for it (0.041, 0.091, 0.176
    for kernel tiles 256, 64, 128)."""
    rng = np.random.default_rng([42, T])
    hosts = [workloads.round_to(rng.standard_normal((512, 768)), "bf16") for _ in range(2)]
    worst = {}
    for precise in (True, False):
        devs = [h.cuda() for h in hosts]
        H.himuon_tiled_ns(devs, T, 16, COEFFS, precise=precise)
        torch.cuda.synchronize()
        worst[precise] = max(float(tile_errors(h, d, T, COEFFS, 16).max()) for h, d in zip(hosts, devs))
    say(f"T={T} K=16 quintic: precise {worst[True]:.3e}, bf16 {worst[False]:.3e}")
    assert worst[True] <= 5e-3
    assert 3e-2 < worst[False] < 0.5


@pytest.mark.parametrize("T", [32, 64, 100, 128, 256, 512])
def test_precise_mixed_shapes(cuda, T):
    """Ragged, thin and wide matrices in one call, every tile against the
    oracle, with mixed per-step coefficients."""
    rng = np.random.default_rng([43, T])
    shapes = [(300, 260), (7, 300), (130, 40), (600, 520), (1, 1)]
    hosts = [workloads.round_to(rng.standard_normal(s), "bf16") for s in shapes]
    devs = [h.cuda() for h in hosts]
    H.himuon_tiled_ns(devs, T, 5, MIXED, precise=True)
    torch.cuda.synchronize()
    worst = max(float(tile_errors(h, d, T, MIXED, 5).max()) for h, d in zip(hosts, devs))
    say(f"precise T={T}: worst {worst:.3e}")
    assert worst <= 5e-3


def test_precise_muon_step_and_gram(cuda):
    """The fused Muon step and the Gram iteration also take the precise mode."""
    rng = np.random.default_rng([44, 0])
    W = workloads.round_to(rng.standard_normal((300, 520)), "bf16")
    M = workloads.round_to(rng.standard_normal((300, 520)), "bf16")
    G = workloads.round_to(rng.standard_normal((300, 520)), "bf16")
    Wg, Mg, Gg = W.cuda(), M.cuda(), G.cuda()
    mu, eta = 0.9, 0.05
    H.himuon_muon_step([Wg], [Mg], [Gg], 128, 5, COEFFS, mu=mu, eta=eta, precise=True)
    torch.cuda.synchronize()
    # momentum within one bf16 rounding of mu M + G (evaluated in fp32 on the device)
    mM, gG = mu * M.double(), G.double()
    m_new = workloads.round_to((mM + gG).numpy(), "bf16").double()
    bound = m_new.abs() * 2.0 ** -7 + 2.0 ** -22 * (mM.abs() + gG.abs())
    assert bool(((Mg.cpu().double() - m_new).abs() <= bound).all())
    # weights: within W's rounding plus eta times 5e-3 of the map, per tile
    Mh = to_np(Mg)
    got, Wd = to_np(Wg), W.double().numpy()
    worst = 0.0
    for r0, r1, c0, c1 in oracle.tile_grid(300, 520, 128):
        U = oracle.ns_map(Mh[r0:r1, c0:c1], COEFFS, K=5)
        want = Wd[r0:r1, c0:c1] - eta * U
        d = np.linalg.norm(got[r0:r1, c0:c1] - want)
        worst = max(worst, d / (np.linalg.norm(np.abs(want) * 2.0 ** -8) + eta * 5e-3 * np.linalg.norm(U)))
    say(f"precise muon: worst difference / bound {worst:.3f}")
    assert worst <= 1.0
    from oracle.gram_ns import gram_ns
    x = workloads.round_to(rng.standard_normal((260, 700)), "bf16")
    g = x.cuda()
    H.himuon_gram_ns([g], 5, COEFFS, restart=2, precise=True)
    torch.cuda.synchronize()
    ref = gram_ns(x.double().numpy(), [COEFFS] * 5, restart=2)
    e = oracle.tile_rel_error(to_np(g), ref)
    say(f"precise gram: {e:.3e}")
    assert e <= 5e-3


STEPS16 = [COEFFS] * 5 + [(1.5, -0.5, 0.0)] * 11


@pytest.mark.parametrize("T,N", [(32, 48), (64, 12), (128, 16)])
def test_damped_tail_many_tiles(cuda, T, N):
    """Five quintic steps then eleven cubic ones over thousands of random
    tiles.  Kernel tile 32 keeps the iterate in fp32 for such runs and stays
    within the bound; the bf16 iterate of kernel tiles 64 and 128 exceeds it on
    a tail of tiles whose small singular values the cubic steps keep
    amplifying (emulated: 1.7 % of 64-tiles, 2.5 % of 128-tiles, worst
    0.15-0.25), which the precise mode removes."""
    gen = torch.Generator(device="cuda").manual_seed(61 + T)
    mats = [torch.randn(1024, 1024, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(N)]
    nt = 1024 // T
    host = np.stack([to_np(m) for m in mats]).reshape(N, nt, T, nt, T).transpose(0, 1, 3, 2, 4).reshape(-1, T, T)
    ref = oracle.ns_map_stack_torch(host, STEPS16, K=16).numpy()
    worst = {}
    for precise in ((False,) if T == 32 else (False, True)):
        devs = [m.clone() for m in mats]
        H.himuon_tiled_ns(devs, T, 16, STEPS16, precise=precise)
        torch.cuda.synchronize()
        got = np.stack([to_np(m) for m in devs]).reshape(N, nt, T, nt, T).transpose(0, 1, 3, 2, 4).reshape(-1, T, T)
        e = np.linalg.norm((got - ref).reshape(len(ref), -1), axis=1) / np.linalg.norm(ref.reshape(len(ref), -1), axis=1)
        worst[precise] = float(e.max())
        say(f"T={T} damped K=16 {'precise' if precise else 'bf16'}: {len(e)} tiles, worst {e.max():.3e}, "
            f"over 3e-2: {(e > 3e-2).sum()}")
    if T == 32:
        assert worst[False] <= 3e-2
    else:
        assert 3e-2 < worst[False] < 0.6
        assert worst[True] <= 5e-3
