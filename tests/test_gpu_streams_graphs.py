"""GPU tests of two properties of the C ABI that callers rely on: a call
allocates nothing, issues no memset and keeps no device state between calls.

- Graph capture: a call captured in a HIP graph (through torch.cuda.graph)
  and replayed several times, with the inputs restored by eager copies and
  the stream synchronised between replays, gives the eager result bit for
  bit on every replay (on-chip path with its tail launch, step path with a
  caller workspace, the Gram iteration).
- Streams: calls on two streams at once give the same bits as the same calls
  one after the other.
"""
import numpy as np
import pytest
import torch

import tiled_newton_schulz_amd as H
import workloads
from workloads import COEFFS

pytestmark = pytest.mark.gpu


def inputs(shapes, seed):
    rng = np.random.default_rng([81, seed])
    return [workloads.round_to(rng.standard_normal(s), "bf16").cuda() for s in shapes]


def workspace(mats, T):
    full, _ = H.himuon_workspace_size(mats, T)
    return torch.empty(max(full, 1), dtype=torch.uint8, device=mats[0].device), full


@pytest.mark.parametrize("case", ["onchip_tail", "step", "gram"])
def test_graph_capture_replays(cuda, case):
    if case == "onchip_tail":
        # one layer at d = 2048, T = 128: the one-wave launch plus the tail launch
        shapes, T = [(2048, 2048)] * 4 + [(2048, 5632), (2048, 5632), (5632, 2048)], 128
    elif case == "step":
        shapes, T = [(600, 520), (1100, 1030)], 512
    else:
        shapes, T = [(300, 900), (512, 256)], None
    x0 = inputs(shapes, len(case))
    if case == "gram":
        full, _ = H.himuon_gram_ns_workspace(x0)
        ws = torch.empty(max(full, 1), dtype=torch.uint8, device=cuda)
        call = lambda mats: H.himuon_gram_ns(mats, 5, COEFFS, workspace=ws, workspace_bytes=full)
    else:
        ws, full = workspace(x0, T)
        call = lambda mats: H.himuon_tiled_ns(mats, T, 5, COEFFS, workspace=ws, workspace_bytes=full)
    ref = [x.clone() for x in x0]
    call(ref)
    torch.cuda.synchronize()

    bufs = [x.clone() for x in x0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up call outside the capture
        call(bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(bufs)
    for rep in range(4):
        for b, x in zip(bufs, x0):
            b.copy_(x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (b, r) in enumerate(zip(bufs, ref)):
            assert torch.equal(b, r), (case, rep, i)
        # eager work of the program's own between replays
        scratch = torch.randn(1 << 16, device=cuda).sum()
        torch.cuda.synchronize()
        del scratch


def test_two_streams_at_once(cuda):
    a0 = inputs([(2048, 2048), (2048, 5632), (700, 520)], 1)
    b0 = inputs([(5632, 2048), (1100, 1030), (300, 260)], 2)
    T = 256
    ra, rb = [x.clone() for x in a0], [x.clone() for x in b0]
    wa, fa = workspace(ra, T)
    wb, fb = workspace(rb, T)
    H.himuon_tiled_ns(ra, T, 5, COEFFS, workspace=wa, workspace_bytes=fa)
    H.himuon_tiled_ns(rb, T, 5, COEFFS, workspace=wb, workspace_bytes=fb)
    torch.cuda.synchronize()

    ca, cb = [x.clone() for x in a0], [x.clone() for x in b0]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        for c, x in zip(ca + cb, a0 + b0):
            c.copy_(x)
        torch.cuda.synchronize()
        H.himuon_tiled_ns(ca, T, 5, COEFFS, workspace=wa, workspace_bytes=fa, stream=s1)
        H.himuon_tiled_ns(cb, T, 5, COEFFS, workspace=wb, workspace_bytes=fb, stream=s2)
        torch.cuda.synchronize()
        for c, r in zip(ca + cb, ra + rb):
            assert torch.equal(c, r)
