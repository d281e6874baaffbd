"""GPU parity of calls whose tile classes (one matrix's interior, right-edge,
bottom-edge or corner tiles) outnumber one launch's table of 256 entries, so
that a route runs several launch groups: the on-chip kernels, both step-path
workspaces, and the Gram iteration.  Every matrix is compared with the fp64
oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from oracle.gram_ns import gram_ns as oracle_gram
from workloads import COEFFS

pytestmark = pytest.mark.gpu

TOL = 3e-2


def say(msg):
    print(msg, flush=True)


def batch(shapes, seed):
    rng = np.random.default_rng([83, seed])
    return [workloads.round_to(rng.standard_normal(s), "bf16") for s in shapes]


def test_on_chip_groups(cuda):
    """300 matrices of 70 x 90 at T = 64: 300 interior classes on the plain
    kernel and 900 edge classes (a side of 6 or 26) on the split-precision
    one, in 2 and 4 launches."""
    hosts = batch([(70, 90)] * 300, 1)
    plan = H.himuon_plan([H.shape_descriptor(70, 90, ptr=(1 << 32) + i * (1 << 20)) for i in range(300)], 64, 5,
                         H.BF16)
    assert plan["resident_launches"] >= 6, plan
    devs = [x.cuda() for x in hosts]
    H.himuon_tiled_ns(devs, 64, 5, COEFFS)
    torch.cuda.synchronize()
    worst = 0.0
    for x, d in zip(hosts, devs):
        ref = oracle.tiled_ns(x.double().numpy(), 64, COEFFS, K=5)
        worst = max(worst, oracle.tile_rel_errors(d.double().cpu().numpy(), ref, 64).max())
    say(f"300 matrices, T=64: worst per-tile error {worst:.3e}")
    assert worst <= TOL


def test_step_path_groups(cuda):
    """600 matrices at T = 512: 300 of 64 x 300 (bf16 workspace) and 300 of
    300 x 40 (fp32 workspace: a short side below 64), two step groups each, in
    one call and in chunks of a small workspace cap; the two runs agree bit
    for bit."""
    shapes = [(64, 300), (300, 40)] * 300
    hosts = batch(shapes, 2)
    devs = [x.cuda() for x in hosts]
    full, mn = H.himuon_workspace_size(devs, 512)
    H.himuon_tiled_ns(devs, 512, 5, COEFFS)
    capped = [x.cuda() for x in hosts]
    H.himuon_tiled_ns(capped, 512, 5, COEFFS, workspace_bytes=max(mn, full // 7))
    torch.cuda.synchronize()
    worst = 0.0
    for x, d, c in zip(hosts, devs, capped):
        assert torch.equal(d, c)
        ref = oracle.tiled_ns(x.double().numpy(), 512, COEFFS, K=5)
        worst = max(worst, oracle.tile_rel_errors(d.double().cpu().numpy(), ref, 512).max())
    say(f"600 matrices, T=512: worst error {worst:.3e}")
    assert worst <= TOL


def test_gram_groups(cuda):
    """600 matrices through the Gram iteration, one class each: 300 with a
    short side of 96 (bf16 workspace) and 300 below 96 (fp32 workspace), two
    groups each."""
    hosts = batch([(96, 300), (40, 300), (300, 96), (300, 64)] * 150, 3)
    devs = [x.cuda() for x in hosts]
    H.himuon_gram_ns(devs, 5, COEFFS, restart=2)
    torch.cuda.synchronize()
    worst = 0.0
    for x, d in zip(hosts, devs):
        ref = oracle_gram(x.double().numpy(), [COEFFS] * 5, restart=2)
        got = d.double().cpu().numpy()
        worst = max(worst, float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    say(f"300 matrices, Gram: worst error {worst:.3e}")
    assert worst <= TOL
