"""himuon_tiled_ns_noalloc: the tiled map with no device allocation, through
the library's own fixed scratch.  It must give exactly what himuon_tiled_ns
gives with a caller workspace, on consecutive calls that share the scratch
(the second smaller than the first, so stale contents from the first call lie
in the scratch), and reject work that does not fit before touching the
device."""
import ctypes

import numpy as np
import pytest

import oracle
import tiled_newton_schulz_amd as H
import workloads
from tiled_newton_schulz_amd import shape_descriptor as sd

COEFFS = workloads.COEFFS
SCRATCH = H.NOALLOC_SCRATCH_BYTES


def _noalloc_c(mats, T, K, dt):
    """Direct C-ABI call (no binding helpers beyond the descriptor array)."""
    import torch
    arr = (H.himuon_matrix_t * len(mats))(*[H.descriptor(m) for m in mats])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return H.lib.himuon_tiled_ns_noalloc(arr, len(mats), T, K, H.coeff_array(COEFFS, K), dt, 1e-7, stream)


def test_noalloc_rejects_oversize_before_device():
    """One tile beyond the scratch (a 6000 x 6000 fp32 full map needs four
    144 MB areas) is refused on the host; so are the usual bad arguments."""
    one = (H.himuon_matrix_t * 1)(sd(6000, 6000))
    abc = H.coeff_array(COEFFS, 5)
    assert H.lib.himuon_tiled_ns_noalloc(one, 1, 6000, 5, abc, H.FP32, 1e-7, None) == 5
    assert H.lib.himuon_tiled_ns_noalloc(one, 1, 6000, 17, abc, H.FP32, 1e-7, None) == 1
    assert H.lib.himuon_tiled_ns_noalloc(one, 1, 0, 5, abc, H.FP32, 1e-7, None) == 1
    bad = (H.himuon_matrix_t * 1)(H.himuon_matrix_t(None, 64, 64, 64))
    assert H.lib.himuon_tiled_ns_noalloc(bad, 1, 64, 5, abc, H.BF16, 1e-7, None) == 1
    assert H.lib.himuon_tiled_ns_noalloc(one, 0, 64, 5, abc, H.BF16, 1e-7, None) == 0
    # a 2500 x 2500 fp32 full map (four 25 MB areas) fits
    info = H.himuon_plan([sd(2500, 2500)], 2500, 5, H.FP32, SCRATCH)
    assert info["chunks"] == 1 and info["workspace_min"] <= SCRATCH


# (dtype, first call's shapes, second call's smaller shapes, T)
CASES = [
    ("bf16", [(4096, 4096), (700, 1100)], [(900, 1300)], 512),
    ("fp32", [(640, 960), (300, 500)], [(200, 330)], 256),
    ("bf16", [(2048, 3000)], [(1000, 700)], 3000),
]


@pytest.mark.gpu
@pytest.mark.parametrize("dt,first,second,T", CASES)
def test_noalloc_matches_workspace_entry(cuda, dt, first, second, T):
    import torch
    code = H.BF16 if dt == "bf16" else H.FP32
    tol = 3e-2 if dt == "bf16" else 1e-4
    rng = np.random.default_rng([77, T])
    plan = H.himuon_plan([sd(h, w, ptr=(i + 1) << 34) for i, (h, w) in enumerate(first)], T, 5, code, SCRATCH)
    assert plan["chunks"] >= 1, plan
    for call, shapes in enumerate((first, second)):
        print(f"noalloc: {dt} T={T} call {call} shapes {shapes}", flush=True)
        host = [workloads.round_to(rng.standard_normal(s), dt) for s in shapes]
        mine = [h.to(cuda) for h in host]
        ref = [h.to(cuda) for h in host]
        assert _noalloc_c(mine, T, 5, code) == 0
        H.himuon_tiled_ns(ref, T, 5, COEFFS)          # caller workspace through torch
        torch.cuda.synchronize()
        for g, r in zip(mine, ref):
            assert torch.equal(g.view(torch.int16 if dt == "bf16" else torch.int32),
                               r.view(torch.int16 if dt == "bf16" else torch.int32))
        # and against the oracle, on a few tiles of each matrix
        for h, g in zip(host, mine):
            x = h.double().numpy()
            out = g.cpu().double().numpy()
            nti, ntj = -(-x.shape[0] // T), -(-x.shape[1] // T)
            for ti, tj in {(0, 0), (nti - 1, ntj - 1), (nti // 2, ntj - 1)}:
                want = oracle.tiled_ns_tile(x, T, ti, tj, COEFFS, K=5)
                got = out[ti * T:ti * T + want.shape[0], tj * T:tj * T + want.shape[1]]
                assert oracle.tile_rel_error(got, want) <= tol


@pytest.mark.gpu
def test_noalloc_on_chip_only(cuda):
    """Work that never reaches the step path (kernel tiles 64 and 128) runs the
    same launches as himuon_tiled_ns."""
    import torch
    rng = np.random.default_rng([78, 1])
    host = [workloads.round_to(rng.standard_normal(s), "bf16") for s in [(300, 260), (128, 640)]]
    for T in (64, 128):
        mine = [h.to(cuda) for h in host]
        ref = [h.to(cuda) for h in host]
        H.himuon_tiled_ns_noalloc(mine, T, 5, COEFFS)
        H.himuon_tiled_ns(ref, T, 5, COEFFS)
        torch.cuda.synchronize()
        for g, r in zip(mine, ref):
            assert torch.equal(g.view(torch.int16), r.view(torch.int16))
