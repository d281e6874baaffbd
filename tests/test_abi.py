"""C-ABI checks that run without a GPU: the library loads, exports every
declared symbol, validates arguments before touching the device, and plans
chunks that respect the workspace cap.  No call here launches a kernel."""
import ctypes
import math
import os
import re

import pytest

import tiled_newton_schulz_amd as H
from tiled_newton_schulz_amd import shape_descriptor as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "himuon.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(himuon_\w+)\s*\(", txt)))


def test_header_symbols_exported():
    names = declared_functions()
    assert set(names) == set(H.EXPORTS)
    for n in names:
        assert hasattr(H.lib, n), n


def test_exports_via_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", H.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (himuon_\w+)", out))
    assert set(declared_functions()) <= syms


def test_status_strings_and_version():
    for code in range(7):
        assert H.himuon_status_string(code)
    assert H.himuon_status_string(99) == "unknown status"
    assert H.himuon_version() >= 10000
    assert H.himuon_last_hip_error() == 0


def call_ns(descs, T=128, K=5, abc=None, dt=H.BF16, eps=1e-7, ws=None, ws_bytes=0):
    arr = (H.himuon_matrix_t * max(1, len(descs)))(*descs)
    if abc is None:
        abc = H.coeff_array((3.4445, -4.775, 2.0315), K) if K > 0 else None
    return H.lib.himuon_tiled_ns(arr, len(descs), T, K, abc, dt, eps, ws, ws_bytes, None)


def test_validation_errors_before_any_launch():
    good = sd(64, 64)
    assert call_ns([], T=128) == 0                      # n == 0 is a no-op
    assert call_ns([H.himuon_matrix_t(None, 64, 64, 64)]) == 1
    assert call_ns([sd(0, 64)]) == 1
    assert call_ns([sd(64, 0)]) == 1
    assert call_ns([sd(64, 64, ld=63)]) == 1
    assert call_ns([good], T=0) == 1
    assert call_ns([good], K=-1, abc=H.coeff_array([], 0)) == 1
    assert call_ns([good], K=17, abc=(ctypes.c_float * 51)(*([1.0] * 51))) == 1
    arr = (H.himuon_matrix_t * 1)(good)
    assert H.lib.himuon_tiled_ns(arr, 1, 128, 2, None, H.BF16, 1e-7, None, 0, None) == 1
    nanabc = (ctypes.c_float * 3)(3.4, float("nan"), 2.0)
    assert H.lib.himuon_tiled_ns(arr, 1, 128, 1, nanabc, H.BF16, 1e-7, None, 0, None) == 1
    assert call_ns([good], eps=-1.0) == 1
    assert call_ns([good], eps=float("inf")) == 1
    assert call_ns([good], dt=7) == 2
    assert call_ns([H.himuon_matrix_t((1 << 20) + 1, 64, 64, 64)]) == 3   # misaligned bf16
    assert call_ns([H.himuon_matrix_t((1 << 20) + 2, 64, 64, 64)], dt=H.FP32, T=256) == 3
    # the step path needs a workspace
    assert call_ns([sd(1024, 1024)], T=512) == 5
    assert call_ns([sd(1024, 1024)], T=512, ws=None, ws_bytes=1 << 20) == 5
    assert call_ns([sd(1024, 1024)], T=512, ws=ctypes.c_void_p(1 << 30), ws_bytes=1000) == 5


def test_overlap_detection():
    base = 1 << 30
    # identical or overlapping row ranges
    assert call_ns([sd(64, 64, ptr=base), sd(64, 64, ptr=base)]) == 4
    assert call_ns([sd(64, 64, ptr=base), sd(64, 64, ptr=base + 2 * 64 * 63)]) == 4
    # adjacent row blocks of one tensor
    assert H.himuon_plan([sd(64, 64, ptr=base), sd(64, 64, ptr=base + 2 * 64 * 64)], 128, 5, H.BF16)["tiles"] == 2
    # column blocks of one fused tensor: same ld, disjoint columns -> allowed
    ld = 192
    q = sd(64, 64, ld=ld, ptr=base)
    k = sd(64, 64, ld=ld, ptr=base + 2 * 64)
    v = sd(64, 64, ld=ld, ptr=base + 2 * 128)
    info = H.himuon_plan([q, k, v], 128, 5, H.BF16)
    assert info["tiles"] == 3
    # overlapping columns -> rejected
    k2 = sd(64, 64, ld=ld, ptr=base + 2 * 32)
    with pytest.raises(H.HimuonError) as e:
        H.himuon_plan([q, k2], 128, 5, H.BF16)
    assert e.value.code == 4


def test_muon_step_validation():
    P = ctypes.POINTER(H.himuon_matrix_t)
    W = (H.himuon_matrix_t * 1)(sd(64, 64, ptr=1 << 30))
    M = (H.himuon_matrix_t * 1)(sd(64, 64, ptr=1 << 31))
    G = (H.himuon_matrix_t * 1)(sd(64, 64, ptr=1 << 32))
    G_bad = (H.himuon_matrix_t * 1)(sd(64, 32, ptr=1 << 32))
    G_alias = (H.himuon_matrix_t * 1)(sd(64, 64, ptr=1 << 31))
    abc = H.coeff_array((3.4445, -4.775, 2.0315), 5)
    f = H.lib.himuon_muon_step
    assert f(W, M, G_bad, 1, 128, 5, abc, 0.9, 0.02, H.BF16, 1e-7, None, 0, None) == 1
    assert f(W, M, G_alias, 1, 128, 5, abc, 0.9, 0.02, H.BF16, 1e-7, None, 0, None) == 4
    assert f(W, M, G, 1, 128, 5, abc, float("nan"), 0.02, H.BF16, 1e-7, None, 0, None) == 1
    assert f(ctypes.cast(None, P), M, G, 1, 128, 5, abc, 0.9, 0.02, H.BF16, 1e-7, None, 0, None) == 1


def layer_descs(ptr0=1 << 30):
    shapes = [(2048, 2048)] * 4 + [(2048, 5632), (2048, 5632), (5632, 2048)]
    out, p = [], ptr0
    for h, w in shapes:
        out.append(sd(h, w, ptr=p))
        p += h * w * 4 + 4096
    return out


def test_plan_layer_on_chip():
    info = H.himuon_plan(layer_descs(), 128, 5, H.BF16)
    assert info["tiles"] == 3136
    assert info["resident_launches"] == 1 and info["chunks"] == 0 and info["kernel_tile"] == 128
    assert info["workspace_full"] == 0
    info = H.himuon_plan(layer_descs(), 32, 5, H.BF16)
    assert info["tiles"] == 4 * 64 * 64 + 3 * 64 * 176 and info["kernel_tile"] == 32


def test_plan_fp32_on_chip():
    """fp32 tiles of up to 64 x 64 run in one on-chip launch with no workspace;
    larger fp32 tiles take the step path."""
    x = sd(256, 512, ptr=1 << 32)
    info = H.himuon_plan([x], 64, 5, H.FP32)
    assert info["tiles"] == 32 and info["resident_launches"] == 1 and info["chunks"] == 0
    assert info["kernel_tile"] == 64 and info["workspace_full"] == 0
    info = H.himuon_plan([sd(100, 70, ptr=1 << 32)], 48, 3, H.FP32)   # 48 and 22/4-wide edges
    assert info["resident_launches"] == 1 and info["chunks"] == 0
    info = H.himuon_plan([x], 128, 5, H.FP32, 1 << 30)
    assert info["resident_launches"] == 0 and info["chunks"] >= 1 and info["workspace_full"] > 0
    # bf16 storage with fp32 arithmetic keeps the step path
    info = H.himuon_plan([sd(256, 512, ptr=1 << 32)], 64, 5, H.BF16_PRECISE, 1 << 30)
    assert info["resident_launches"] == 0 and info["chunks"] >= 1


def test_plan_cross_layer_groups():
    descs = layer_descs() * 1
    many = []
    p = 1 << 32
    for _ in range(24):
        for d in layer_descs(p):
            many.append(d)
        p += 200 << 20
    info = H.himuon_plan(many, 128, 5, H.BF16)
    assert info["tiles"] == 24 * 3136
    assert info["resident_launches"] == math.ceil(168 / 256)


def moe_descs():
    descs, p = [], 1 << 32
    for _ in range(64):
        for h, w in ((4096, 1408), (1408, 4096)):
            descs.append(sd(h, w, ptr=p))
            p += h * w * 2 + 4096
    return descs


def test_plan_moe_ragged_on_chip():
    descs = moe_descs()
    info = H.himuon_plan(descs, 256, 5, H.BF16)
    # 10,240 full tiles and 2,048 ragged 256x128 / 128x256 edge tiles, all on
    # chip (kernel tile 256): one launch for the 128 interior classes and one
    # for the 128 narrow edge classes (shorter side <= 128)
    assert info["tiles"] == 64 * 2 * 16 * 6
    assert info["kernel_tile"] == 256 and info["chunks"] == 0 and info["workspace_full"] == 0
    assert info["resident_launches"] == 2


def test_plan_moe_chunking():
    descs = moe_descs()
    full, mn = H.himuon_workspace_size(descs, 512, H.BF16)
    assert full > mn > 0
    info = H.himuon_plan(descs, 512, 5, H.BF16, full)
    # at T = 512 every tile takes the step path: 512x512 and 512x384 / 384x512
    assert info["tiles"] == 64 * 2 * 8 * 3 and info["resident_launches"] == 0
    assert info["chunks"] == math.ceil(2 * len(descs) / 256)
    # a small cap forces many chunks, each within the cap
    cap = 64 << 20
    info2 = H.himuon_plan(descs, 512, 5, H.BF16, cap)
    assert info2["chunks"] > info["chunks"] and info2["workspace_full"] <= cap
    with pytest.raises(H.HimuonError) as e:
        H.himuon_plan(descs, 512, 5, H.BF16, mn - 1)
    assert e.value.code == 5


def test_plan_dense_cap():
    d = [sd(8192, 28672, ptr=1 << 34), sd(28672, 8192, ptr=1 << 36)]
    for T in (128, 256, 512):
        full, mn = H.himuon_workspace_size(d, T, H.BF16)
        info = H.himuon_plan(d, T, 5, H.BF16, 4 << 30)
        assert info["workspace_full"] <= 4 << 30
        assert info["tiles"] == 2 * (8192 // T) * (28672 // T)
        if T <= 256:
            assert info["resident_launches"] == 1 and info["chunks"] == 0 and info["kernel_tile"] == T
        else:
            assert info["chunks"] >= math.ceil(full / (4 << 30))


def test_plan_full_matrix_and_fp32():
    d = layer_descs()
    info = H.himuon_plan(d, 5632, 5, H.BF16, 1 << 40)
    assert info["tiles"] == 7 and info["resident_launches"] == 0 and info["chunks"] == 1
    # fp32 tiles larger than 64 take the step path
    info = H.himuon_plan([sd(256, 512)], 128, 5, H.FP32, 1 << 30)
    assert info["tiles"] == 8 and info["chunks"] == 1 and info["launches"] == 2 + 15
    # a bf16 matrix smaller than 128 at T = 256 stays on chip
    info = H.himuon_plan([sd(100, 90)], 256, 5, H.BF16)
    assert info["resident_launches"] == 1 and info["kernel_tile"] == 128


def route(th, tw):
    mn, mx = min(th, tw), max(th, tw)
    if mx <= 256 and (mn >= 48 or (mn >= 32 and mx <= 128)):
        return "chip"
    if mx <= 64:
        return "chip-precise"
    return "step-bf16" if mn >= 64 else "step-fp32"


def test_workspace_layout_closed_form():
    """The planner's workspace equals, per workspace dtype, the sum over the
    step-path tiles of r * round8(s) + r * round8(r) (brute force over the tile
    grid, with each edge class routed by its shape)."""
    al = lambda x: (x + 255) // 256 * 256
    for (h, w, T) in [(300, 170, 64), (4096, 1408, 256), (1408, 4096, 256), (70, 45, 256), (513, 1025, 512),
                      (700, 20, 256), (100, 300, 200)]:
        full, _ = H.himuon_workspace_size([sd(h, w)], T, H.BF16)
        acc = {"step-bf16": [0, 0, 0], "step-fp32": [0, 0, 0]}
        for r0 in range(0, h, T):
            for c0 in range(0, w, T):
                a, b = min(T, h - r0), min(T, w - c0)
                k = route(a, b)
                if k in acc:
                    r, s_ = min(a, b), max(a, b)
                    acc[k][0] += r * ((s_ + 7) // 8 * 8)
                    acc[k][1] += r * ((r + 7) // 8 * 8)
                    acc[k][2] += 1
        want = 0
        for k, es in (("step-bf16", 2), ("step-fp32", 4)):
            x, a_, n = acc[k]
            if n:
                want = max(want, 2 * al(es * x) + 2 * al(es * a_) + al(n * 32 * 4))
        assert full == want, (h, w, T, full, want)


def test_routes_in_plan():
    # 513 x 1025 at T = 512: two 512x512 tiles (bf16 step path), a 512x1 column
    # and two 1x512 rows (fp32 step path), a 1x1 corner (on chip, precise)
    info = H.himuon_plan([sd(513, 1025)], 512, 5, H.BF16, 1 << 30)
    assert info["tiles"] == 6 and info["resident_launches"] == 1 and info["chunks"] == 2
    # T = 16: every tile is 16 x 16 and runs on chip with hi/lo splitting
    info = H.himuon_plan([sd(64, 64)], 16, 5, H.BF16)
    assert info["tiles"] == 16 and info["resident_launches"] == 1 and info["kernel_tile"] == 32


def test_schedule_validation():
    """The per-step tile-size schedule rejects sizes that increase or do not
    nest, K outside 1..16 and a null size array, before any launch."""
    d = (H.himuon_matrix_t * 1)(sd(600, 520))
    abc = H.coeff_array((3.4445, -4.775, 2.0315), 3)
    f = H.lib.himuon_tiled_ns_schedule

    def ts(*v):
        return (ctypes.c_int32 * len(v))(*v)

    assert f(d, 1, ts(256, 512, 512), 3, abc, H.BF16, 1e-7, None, 0, None) == 1   # increasing
    assert f(d, 1, ts(256, 96, 32), 3, abc, H.BF16, 1e-7, None, 0, None) == 1     # 96 does not divide 256
    assert f(d, 1, ts(256, 128, 0), 3, abc, H.BF16, 1e-7, None, 0, None) == 1     # size < 1
    assert f(d, 1, ts(256), 0, abc, H.BF16, 1e-7, None, 0, None) == 1             # K = 0
    assert f(d, 1, None, 3, abc, H.BF16, 1e-7, None, 0, None) == 1                # no sizes
    # a pass that needs a workspace (T = 512: step path) without one
    assert f(d, 1, ts(512, 256, 128), 3, abc, H.BF16, 1e-7, None, 0, None) == 5


def test_pair_stats_workspace_and_validation():
    """Pair statistics: workspace size from the shapes (one partial of three
    doubles per band of about 64k elements), and every argument error found on
    the host before any launch (placeholder pointers are never read)."""
    P = ctypes.POINTER
    shapes = [(2048, 5632), (5632, 2048), (1, 1), (3, 70000)]
    a = (H.himuon_matrix_t * len(shapes))(*[sd(r, c) for r, c in shapes])
    want = 0
    for r, c in shapes:
        R = max(1, min(-(-65536 // c), r))
        want += -(-r // R)
    assert H.himuon_pair_stats_workspace(a) == want * 24
    assert H.himuon_pair_stats_workspace([]) == 0
    nb = ctypes.c_size_t(0)
    assert H.lib.himuon_pair_stats_workspace(a, len(shapes), None) == 1
    assert H.lib.himuon_pair_stats_workspace(None, 1, ctypes.byref(nb)) == 1
    bad = (H.himuon_matrix_t * 1)(sd(0, 5))
    assert H.lib.himuon_pair_stats_workspace(bad, 1, ctypes.byref(nb)) == 1

    ws, out = ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 26)
    big = 1 << 40

    def call(x, y, n=1, dt=H.BF16, o=out, w=ws, wb=big):
        return H.lib.himuon_pair_stats(x, y, n, dt, o, w, wb, None)

    x = (H.himuon_matrix_t * 1)(sd(64, 96))
    y = (H.himuon_matrix_t * 1)(sd(64, 96, ptr=1 << 22))
    assert call(x, y, n=0) == 0                                   # no-op
    assert call(x, y, dt=7) == 2                                  # dtype
    assert call(x, y, n=-1) == 1
    assert call(None, y) == 1 and call(x, None) == 1
    assert call(x, y, o=None) == 1
    assert call(x, (H.himuon_matrix_t * 1)(sd(64, 95, ptr=1 << 22))) == 1   # shapes differ
    assert call(x, (H.himuon_matrix_t * 1)(sd(64, 96, ld=90, ptr=1 << 22))) == 1   # ld < cols
    assert call(x, (H.himuon_matrix_t * 1)(sd(64, 96, ptr=(1 << 22) + 1))) == 3   # misaligned
    assert call(x, y, o=ctypes.c_void_p((1 << 26) + 4)) == 3      # out not 8-byte aligned
    assert call(x, y, w=None) == 5
    need = H.himuon_pair_stats_workspace(x)
    assert call(x, y, wb=need - 1) == 5
    assert call(x, y, w=ctypes.c_void_p((1 << 24) + 4)) == 3


def test_one_hip_runtime_after_import():
    """Importing the binding first (as this file does, before any GPU test)
    must leave one HIP runtime in the process: the library binds to torch's,
    which owns the device memory and streams it is handed."""
    import subprocess
    import sys
    code = ("import os, tiled_newton_schulz_amd, torch\n"
            "m = open(f'/proc/{os.getpid()}/maps').read()\n"
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip() == "1"


def test_gram_ns_workspace_and_validation():
    """himuon_gram_ns: every matrix is one tile on the step path with two
    oriented X areas and four r x r areas (R, the step polynomial, the running
    product, a spare) plus the norm partials; bf16 keeps a bf16 workspace when
    both sides are >= 96, else fp32.  Errors come before any launch."""
    al = lambda x: (x + 255) // 256 * 256
    r8 = lambda x: (x + 7) // 8 * 8
    for h, w, dt in [(2048, 5632, H.BF16), (5632, 2048, H.BF16), (300, 170, H.FP32), (20, 700, H.BF16),
                     (64, 64, H.BF16)]:
        r, s_ = min(h, w), max(h, w)
        es = 4 if dt == H.FP32 or r < 96 else 2
        want = 2 * al(es * r * r8(s_)) + 4 * al(es * r * r8(r)) + al(32 * 4)
        assert H.himuon_gram_ns_workspace([sd(h, w)], dt) == (want, want), (h, w)
    # several matrices: one chunk holds them all; min is the largest single one
    full, mn = H.himuon_gram_ns_workspace([sd(1024, 4096), sd(512, 512, ptr=1 << 34)], H.BF16)
    one = lambda r, s_: 2 * al(2 * r * s_) + 4 * al(2 * r * r) + al(32 * 4)
    assert mn == one(1024, 4096)
    assert full == 2 * al(2 * (1024 * 4096 + 512 * 512)) + 4 * al(2 * (1024 * 1024 + 512 * 512)) + al(2 * 32 * 4)

    def call(descs, K=5, restart=2, ws=None, nbytes=0, dt=H.BF16):
        arr = (H.himuon_matrix_t * max(1, len(descs)))(*descs)
        abc = H.coeff_array((3.4445, -4.775, 2.0315), K)
        return H.lib.himuon_gram_ns(arr, len(descs), K, abc, restart, dt, 1e-7, ws, nbytes, None)

    assert call([]) == 0
    assert call([sd(256, 512)], restart=-1) == 1
    assert call([H.himuon_matrix_t(None, 64, 64, 64)]) == 1
    assert call([sd(256, 512)], K=17) == 1
    assert call([sd(256, 512)]) == 5                                         # no workspace
    assert call([sd(256, 512)], ws=ctypes.c_void_p(1 << 30), nbytes=1000) == 5
    assert call([sd(1, (1 << 31) + 8)]) == 3                                 # side past the int32 grid
    assert call([H.himuon_matrix_t((1 << 20) + 1, 64, 64, 64)]) == 3
