"""Whole-workload parity: every tile of the one-layer workload, the 24-layer
batch (T = 32, 64, 128), the MoE batch (T = 256, ragged edges) and the dense
layer (T = 512 under the 4 GiB cap) against the oracle; the error tail of the
on-chip 256 kernel (square and narrow tiles) and of the 512 step path; and
functional-block splitting of a fused Q|K|V tensor (CMuon) against the oracle.

The oracle side of the large checks is ns_map_stack_torch (the per-tile map
in torch CPU float64, all host threads), in chunks of whole matrices so that
host memory stays bounded.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_newton_schulz_amd as H
import workloads
from workloads import COEFFS, WORKLOADS

pytestmark = pytest.mark.gpu

TOL = 3e-2


def say(msg):
    print(msg, flush=True)


def tiles(x, T):
    """(N, T, T) float64 CPU stack of the tiles of a matrix (T divides both
    sides), in row-major tile order."""
    h, w = x.shape
    return x.to("cpu", torch.float64).reshape(h // T, T, w // T, T).permute(0, 2, 1, 3).reshape(-1, T, T)


def stack_errors(got, ref):
    n = ref.shape[0]
    num = torch.linalg.vector_norm((got - ref).reshape(n, -1), dim=1)
    den = torch.linalg.vector_norm(ref.reshape(n, -1), dim=1)
    return torch.where(den > 0, num / den, num)


def check_every_tile(inputs, outputs, T, chunk_elems=64 << 20):
    """Every T-tile of every matrix: returns (tiles checked, worst error)."""
    worst, count, i = 0.0, 0, 0
    while i < len(inputs):
        j, el = i, 0
        while j < len(inputs) and (j == i or el + inputs[j].numel() <= chunk_elems):
            el += inputs[j].numel()
            j += 1
        x = torch.cat([tiles(m, T) for m in inputs[i:j]])
        g = torch.cat([tiles(m, T) for m in outputs[i:j]])
        e = stack_errors(g, oracle.ns_map_stack_torch(x, COEFFS, K=5))
        worst = max(worst, float(e.max()))
        count += e.numel()
        i = j
    return count, worst


def test_layer_d2048_every_tile(cuda):
    """The one-layer workload (7 matrices, 3,136 tiles of 128), every tile."""
    w = WORKLOADS["layer_d2048"]
    mats = [t.cuda() for t in workloads.host_tensors(w)]
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, 128, 5, COEFFS)
    torch.cuda.synchronize()
    n, worst = check_every_tile(inputs, mats, 128)
    say(f"layer_d2048 T=128: {n} tiles, worst {worst:.3e}")
    assert n == 3136 and worst <= TOL


@pytest.mark.parametrize("T,n_tiles", [(32, 1_204_224), (64, 301_056), (128, 75_264)])
def test_layers24_every_tile(cuda, T, n_tiles):
    """The 24-layer batch (168 matrices, 1.23 G elements) in one call; every
    tile against the oracle."""
    w = WORKLOADS["layers24_d2048"]
    mats = workloads.device_tensors(w)
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, T, 5, COEFFS)
    torch.cuda.synchronize()
    say(f"layers24 T={T}: comparing")
    n, worst = check_every_tile(inputs, mats, T)
    say(f"layers24 T={T}: {n} tiles, worst {worst:.3e}")
    assert n == n_tiles and worst <= TOL


def test_moe64_every_tile(cuda):
    """The MoE batch (64 experts, 4096 x 1408 and 1408 x 4096, T = 256): all
    12,288 tiles, 10,240 square and 2,048 ragged 128 x 256 / 256 x 128 edge
    tiles, against the oracle."""
    w = WORKLOADS["moe64"]
    mats = workloads.device_tensors(w)
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, 256, 5, COEFFS)
    torch.cuda.synchronize()
    say("moe64 T=256: comparing")
    worst, count = 0.0, 0
    for i in range(0, len(mats), 16):
        groups = {}
        for x, g in zip(inputs[i:i + 16], mats[i:i + 16]):
            h, w_ = x.shape
            for r0 in range(0, h, 256):
                for c0 in range(0, w_, 256):
                    key = (min(256, h - r0), min(256, w_ - c0))
                    groups.setdefault(key, ([], []))
                    groups[key][0].append(x[r0:r0 + 256, c0:c0 + 256])
                    groups[key][1].append(g[r0:r0 + 256, c0:c0 + 256])
        for key, (xs, gs) in groups.items():
            xt = torch.stack(xs).to("cpu", torch.float64)
            gt = torch.stack(gs).to("cpu", torch.float64)
            e = stack_errors(gt, oracle.ns_map_stack_torch(xt, COEFFS, K=5))
            worst = max(worst, float(e.max()))
            count += e.numel()
    say(f"moe64 T=256: {count} tiles, worst {worst:.3e}")
    assert count == 12288 and worst <= TOL


def test_dense8192_t512_every_tile(cuda):
    """The dense layer (8192 x 28672 and 28672 x 8192) at T = 512 under the
    4 GiB workspace cap: all 1,792 tiles against the oracle."""
    w = WORKLOADS["dense8192"]
    mats = workloads.device_tensors(w)
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, 512, 5, COEFFS, workspace_bytes=4 << 30)
    torch.cuda.synchronize()
    say("dense8192 T=512: comparing")
    n, worst = check_every_tile(inputs, mats, 512, chunk_elems=32 << 20)
    say(f"dense8192 T=512: {n} tiles, worst {worst:.3e}")
    assert n == 1792 and worst <= TOL


@pytest.mark.parametrize("kind", ["square", "wide", "tall"])
def test_error_tail_tile256(cuda, kind):
    """Over 2,000 tiles of the on-chip 256 kernel: square 256 x 256 tiles, and
    narrow 128 x 256 and 256 x 128 tiles (shorter side 128), all in bf16
    N(0, 1)."""
    gen = torch.Generator(device="cuda").manual_seed(57)
    shape, n = {"square": ((2048, 2048), 32), "wide": ((128, 65536), 8), "tall": ((65536, 128), 8)}[kind]
    mats = [torch.randn(shape, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(n)]
    plan = H.himuon_plan(mats, 256, 5, H.BF16)
    assert plan["chunks"] == 0 and plan["kernel_tile"] == 256
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, 256, 5, COEFFS)
    torch.cuda.synchronize()
    # tiles of the narrow shapes are whole rows (or columns) of 256 elements
    T = (128, 256) if kind == "wide" else (256, 128) if kind == "tall" else (256, 256)
    worst, count = 0.0, 0
    for x, g in zip(inputs, mats):
        h, w_ = x.shape
        xs = x.double().cpu().reshape(h // T[0], T[0], w_ // T[1], T[1]).permute(0, 2, 1, 3).reshape(-1, *T)
        gs = g.double().cpu().reshape(h // T[0], T[0], w_ // T[1], T[1]).permute(0, 2, 1, 3).reshape(-1, *T)
        e = stack_errors(gs, oracle.ns_map_stack_torch(xs, COEFFS, K=5))
        worst = max(worst, float(e.max()))
        count += e.numel()
    say(f"tile 256 {kind}: {count} tiles, worst {worst:.3e}")
    assert count >= 2048 and worst <= TOL


def test_error_tail_tile512(cuda):
    """200 tiles of 512 on the step path (25 matrices of 1024 x 2048)."""
    gen = torch.Generator(device="cuda").manual_seed(58)
    mats = [torch.randn((1024, 2048), device="cuda", generator=gen).to(torch.bfloat16) for _ in range(25)]
    inputs = [m.clone() for m in mats]
    H.himuon_tiled_ns(mats, 512, 5, COEFFS)
    torch.cuda.synchronize()
    n, worst = check_every_tile(inputs, mats, 512)
    say(f"tile 512: {n} tiles, worst {worst:.3e}")
    assert n == 200 and worst <= TOL


@pytest.mark.parametrize("widths", [(192, 192, 192), (130, 200, 246)])
def test_fused_qkv_column_blocks(cuda, widths):
    """Functional-block splitting (the CMuon article: fused Q|K|V weights are
    orthogonalised per block): a fused 256 x 576 bf16 tensor passed as its
    three column-block views, in one call, each against the oracle's map of
    that block.  Where T = 64 divides the split offsets, tiling the fused
    tensor as one matrix gives the same tiles, so the same bits."""
    rng = np.random.default_rng([59, widths[0]])
    host = workloads.round_to(rng.standard_normal((256, 576)), "bf16")
    fused = host.cuda()
    offs = np.cumsum((0,) + widths)
    views = [fused[:, offs[i]:offs[i + 1]] for i in range(3)]
    H.himuon_tiled_ns(views, 64, 5, COEFFS)
    torch.cuda.synchronize()
    out = fused.cpu().double().numpy()
    x = host.double().numpy()
    worst = 0.0
    for i in range(3):
        c0, c1 = offs[i], offs[i + 1]
        ref = oracle.tiled_ns(x[:, c0:c1], 64, COEFFS, K=5)
        worst = max(worst, float(oracle.tile_rel_errors(out[:, c0:c1], ref, 64).max()))
    say(f"fused Q|K|V {widths}: worst {worst:.3e}")
    assert worst <= TOL
    if all(o % 64 == 0 for o in offs):
        whole = host.cuda()
        H.himuon_tiled_ns([whole], 64, 5, COEFFS)
        torch.cuda.synchronize()
        assert torch.equal(whole, fused)
    else:
        # the fused tensor tiled as one matrix is a different map here
        whole = host.cuda()
        H.himuon_tiled_ns([whole], 64, 5, COEFFS)
        torch.cuda.synchronize()
        assert not torch.equal(whole, fused)
