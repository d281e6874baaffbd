"""Python binding of libhimuon (MI355X tiled Newton-Schulz).

Argument marshalling only: every function here forwards to the C entry point
of the same name in include/himuon.h, taking torch tensors for device memory
and torch's current stream.  All arithmetic runs in the library's HIP kernels;
importing this module fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhimuon.so")

BF16 = 0
FP32 = 1
BF16_PRECISE = 2   # bf16 storage, fp32 arithmetic throughout
MAX_STEPS = 16

STATUS = {0: "HIMUON_OK", 1: "HIMUON_ERR_INVALID_ARGUMENT", 2: "HIMUON_ERR_UNSUPPORTED",
          3: "HIMUON_ERR_LAYOUT", 4: "HIMUON_ERR_OVERLAP", 5: "HIMUON_ERR_WORKSPACE", 6: "HIMUON_ERR_HIP"}
NOALLOC_SCRATCH_BYTES = 128 << 20
EXPORTS = ["himuon_plan", "himuon_workspace_size", "himuon_tiled_ns", "himuon_tiled_ns_noalloc",
           "himuon_tiled_ns_schedule",
           "himuon_muon_step", "himuon_gram_ns", "himuon_gram_ns_workspace", "himuon_pair_stats",
           "himuon_pair_stats_workspace", "himuon_status_string",
           "himuon_last_hip_error", "himuon_version"]


class himuon_matrix_t(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


class himuon_plan_info_t(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_int64), ("resident_launches", ctypes.c_int64),
                ("chunks", ctypes.c_int64), ("launches", ctypes.c_int64),
                ("kernel_tile", ctypes.c_int64), ("workspace_full", ctypes.c_size_t),
                ("workspace_min", ctypes.c_size_t), ("tail_tiles", ctypes.c_int64)]


class HimuonError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = STATUS.get(code, str(code))
        if code == 6:
            msg += f" (hipError {lib.himuon_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    # torch first: it brings its own HIP runtime (same soname as the system
    # one), and the library must bind to that instance, the one that owns the
    # device memory and streams it is handed.  Loaded the other way round, the
    # process would hold two HIP runtimes and the library's would see no device.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python tiled_newton_schulz_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.himuon_plan.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                              ctypes.c_int, ctypes.c_size_t, P(himuon_plan_info_t)]
    L.himuon_plan.restype = ctypes.c_int
    L.himuon_workspace_size.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                        P(ctypes.c_size_t), P(ctypes.c_size_t)]
    L.himuon_workspace_size.restype = ctypes.c_int
    L.himuon_tiled_ns.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  P(ctypes.c_float), ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
    L.himuon_tiled_ns.restype = ctypes.c_int
    L.himuon_tiled_ns_noalloc.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          P(ctypes.c_float), ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
    L.himuon_tiled_ns_noalloc.restype = ctypes.c_int
    L.himuon_tiled_ns_schedule.argtypes = [P(himuon_matrix_t), ctypes.c_int32, P(ctypes.c_int32), ctypes.c_int32,
                                           P(ctypes.c_float), ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
    L.himuon_tiled_ns_schedule.restype = ctypes.c_int
    L.himuon_muon_step.argtypes = [P(himuon_matrix_t), P(himuon_matrix_t), P(himuon_matrix_t), ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, P(ctypes.c_float), ctypes.c_float,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    L.himuon_muon_step.restype = ctypes.c_int
    L.himuon_gram_ns.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int32, P(ctypes.c_float),
                                 ctypes.c_int32, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    L.himuon_gram_ns.restype = ctypes.c_int
    L.himuon_gram_ns_workspace.argtypes = [P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int,
                                           P(ctypes.c_size_t), P(ctypes.c_size_t)]
    L.himuon_gram_ns_workspace.restype = ctypes.c_int
    L.himuon_pair_stats.argtypes = [P(himuon_matrix_t), P(himuon_matrix_t), ctypes.c_int32, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.himuon_pair_stats.restype = ctypes.c_int
    L.himuon_pair_stats_workspace.argtypes = [P(himuon_matrix_t), ctypes.c_int32, P(ctypes.c_size_t)]
    L.himuon_pair_stats_workspace.restype = ctypes.c_int
    L.himuon_status_string.argtypes = [ctypes.c_int]
    L.himuon_status_string.restype = ctypes.c_char_p
    L.himuon_last_hip_error.argtypes = []
    L.himuon_last_hip_error.restype = ctypes.c_int32
    L.himuon_version.argtypes = []
    L.himuon_version.restype = ctypes.c_int32
    return L


lib = _load()


# ---- marshalling helpers -------------------------------------------------
def _dtype_code(t, precise: bool = False) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16_PRECISE if precise else BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def descriptor(t) -> himuon_matrix_t:
    """Descriptor of a 2-D tensor.  Row-major views pass as they are; a
    transposed view (unit stride along dim 0) is passed as its row-major
    transpose, which is exact because the tiled map commutes with transposition
    under the (0, 0)-anchored tiling."""
    if t.dim() != 2:
        raise ValueError("matrices must be 2-D")
    H, W = t.shape
    s0, s1 = t.stride()
    if s1 == 1 or W == 1:
        return himuon_matrix_t(t.data_ptr(), H, W, s0 if H > 1 else max(W, 1))
    if s0 == 1 or H == 1:
        return himuon_matrix_t(t.data_ptr(), W, H, s1 if W > 1 else max(H, 1))
    raise ValueError("matrix must have unit stride along one dimension")


def shape_descriptor(rows: int, cols: int, ld: int | None = None, ptr: int = 1 << 20) -> himuon_matrix_t:
    """Descriptor with a placeholder address, for planning queries only."""
    return himuon_matrix_t(ptr, rows, cols, cols if ld is None else ld)


def _descs(ts) -> ctypes.Array:
    arr = (himuon_matrix_t * max(len(ts), 1))()
    for i, t in enumerate(ts):
        arr[i] = t if isinstance(t, himuon_matrix_t) else descriptor(t)
    return arr


def coeff_array(abc, K: int):
    """(a, b, c) per step as a float array of 3K entries.  `abc` is one triple
    (used for every step), a flat list of 3K numbers, or K triples."""
    if K == 0:
        return (ctypes.c_float * 3)()
    flat = []
    items = list(abc)
    if len(items) == 3 and not hasattr(items[0], "__len__"):
        flat = [float(x) for x in items] * K
    elif items and hasattr(items[0], "__len__"):
        for tri in items:
            flat.extend(float(x) for x in tri)
    else:
        flat = [float(x) for x in items]
    if len(flat) != 3 * K:
        raise ValueError("need one (a, b, c) triple per step")
    return (ctypes.c_float * (3 * K))(*flat)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(code: int, where: str):
    if code != 0:
        raise HimuonError(code, where)


# ---- entry points ----------------------------------------------------------
def himuon_plan(mats: Sequence, T: int, K: int, dtype: int, workspace_bytes: int = 0) -> dict:
    d = _descs(mats)
    info = himuon_plan_info_t()
    _check(lib.himuon_plan(d, len(mats), T, K, dtype, workspace_bytes, ctypes.byref(info)), "himuon_plan")
    return {f: getattr(info, f) for f, _ in himuon_plan_info_t._fields_}


def himuon_workspace_size(mats: Sequence, T: int, dtype: int | None = None) -> tuple[int, int]:
    if dtype is None:
        dtype = _dtype_code(mats[0])
    d = _descs(mats)
    full, mn = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.himuon_workspace_size(d, len(mats), T, dtype, ctypes.byref(full), ctypes.byref(mn)),
           "himuon_workspace_size")
    return full.value, mn.value


def _workspace(mats, T, dtype, workspace, workspace_bytes, device):
    import torch
    if workspace is not None:
        nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
        return workspace, workspace.data_ptr(), nbytes
    full, mn = himuon_workspace_size(mats, T, dtype)
    if full == 0:
        return None, None, 0
    cap = full if workspace_bytes is None else max(min(full, workspace_bytes), 0)
    buf = torch.empty(max(cap, 1), dtype=torch.uint8, device=device)
    return buf, buf.data_ptr(), cap


def himuon_tiled_ns(mats: Sequence, T: int, K: int, abc=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
                    workspace=None, workspace_bytes: int | None = None, stream=None, precise: bool = False):
    """Tiled Newton-Schulz in place on a list of 2-D bf16 or fp32 CUDA tensors.

    workspace: optional uint8 device tensor; if omitted the binding allocates
    one through torch (capped at workspace_bytes when given).  precise: bf16
    data with fp32 arithmetic throughout (HIMUON_BF16_PRECISE)."""
    if len(mats) == 0:
        return
    dtype = _dtype_code(mats[0], precise)
    d = _descs(mats)
    ws, ptr, nbytes = _workspace(mats, T, dtype, workspace, workspace_bytes, mats[0].device)
    code = lib.himuon_tiled_ns(d, len(mats), T, K, coeff_array(abc, K), dtype, eps,
                               ctypes.c_void_p(ptr), nbytes, _stream_handle(stream))
    _check(code, "himuon_tiled_ns")
    return ws


def himuon_tiled_ns_noalloc(mats: Sequence, T: int, K: int, abc=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
                            stream=None):
    """Tiled Newton-Schulz in place, with no device allocation: the step path
    runs through the library's own 128 MiB scratch on the device.  Calls that
    overlap in time on one device race on that scratch."""
    if len(mats) == 0:
        return
    dtype = _dtype_code(mats[0])
    d = _descs(mats)
    code = lib.himuon_tiled_ns_noalloc(d, len(mats), T, K, coeff_array(abc, K), dtype, eps,
                                       _stream_handle(stream))
    _check(code, "himuon_tiled_ns_noalloc")


def himuon_tiled_ns_schedule(mats: Sequence, Ts: Sequence[int], abc=(3.4445, -4.7750, 2.0315), eps: float = 1e-7,
                             workspace=None, workspace_bytes: int | None = None, stream=None, precise: bool = False):
    """len(Ts) Newton-Schulz steps in place, step k on the Ts[k] x Ts[k] tiles
    (non-increasing, nested sizes; one normalisation, on the first size)."""
    if len(mats) == 0:
        return
    dtype = _dtype_code(mats[0], precise)
    d = _descs(mats)
    K = len(Ts)
    ts = (ctypes.c_int32 * max(1, K))(*[int(t) for t in Ts])
    if workspace is None:
        # the largest need of any pass, capped
        need = max(himuon_workspace_size(mats, int(t), dtype)[0] for t in set(Ts)) if K else 0
        if need:
            import torch
            need = need if workspace_bytes is None else max(min(need, workspace_bytes), 0)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=mats[0].device)
            workspace_bytes = need
    ptr = workspace.data_ptr() if workspace is not None else None
    nbytes = 0 if workspace is None else (workspace.numel() if workspace_bytes is None else workspace_bytes)
    code = lib.himuon_tiled_ns_schedule(d, len(mats), ts, K, coeff_array(abc, K), dtype, eps,
                                        ctypes.c_void_p(ptr), nbytes, _stream_handle(stream))
    _check(code, "himuon_tiled_ns_schedule")
    return workspace


def himuon_muon_step(W: Sequence, M: Sequence, G: Sequence, T: int, K: int, abc=(3.4445, -4.7750, 2.0315),
                     mu: float = 0.95, eta: float = 0.02, eps: float = 1e-7, workspace=None,
                     workspace_bytes: int | None = None, stream=None, precise: bool = False):
    """Fused Muon step M <- mu M + G, W <- W - eta tiledNS(M), in place."""
    n = len(M)
    if not (len(W) == len(G) == n):
        raise ValueError("W, M, G must have equal length")
    if n == 0:
        return
    dtype = _dtype_code(M[0], precise)
    dW, dM, dG = _descs(W), _descs(M), _descs(G)
    ws, ptr, nbytes = _workspace(M, T, dtype, workspace, workspace_bytes, M[0].device)
    code = lib.himuon_muon_step(dW, dM, dG, n, T, K, coeff_array(abc, K), mu, eta, dtype, eps,
                                ctypes.c_void_p(ptr), nbytes, _stream_handle(stream))
    _check(code, "himuon_muon_step")
    return ws


def himuon_gram_ns_workspace(mats: Sequence, dtype: int | None = None) -> tuple[int, int]:
    """(full, min) workspace bytes of himuon_gram_ns for these matrices."""
    if dtype is None:
        dtype = _dtype_code(mats[0])
    d = _descs(mats)
    full, mn = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.himuon_gram_ns_workspace(d, len(mats), dtype, ctypes.byref(full), ctypes.byref(mn)),
           "himuon_gram_ns_workspace")
    return full.value, mn.value


def himuon_gram_ns(mats: Sequence, K: int, abc=(3.4445, -4.7750, 2.0315), restart: int = 2, eps: float = 1e-7,
                   workspace=None, workspace_bytes: int | None = None, stream=None, precise: bool = False):
    """Full-matrix Newton-Schulz of each matrix, in place, through its Gram
    matrix with a restart before step restart + 1 (0: none)."""
    if len(mats) == 0:
        return
    dtype = _dtype_code(mats[0], precise)
    d = _descs(mats)
    if workspace is None:
        full = himuon_gram_ns_workspace(mats, dtype)[0]
        cap = full if workspace_bytes is None else max(min(full, workspace_bytes), 0)
        if cap:
            import torch
            workspace = torch.empty(cap, dtype=torch.uint8, device=mats[0].device)
        workspace_bytes = cap
    elif workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    ptr = workspace.data_ptr() if workspace is not None else None
    code = lib.himuon_gram_ns(d, len(mats), K, coeff_array(abc, K), restart, dtype, eps,
                              ctypes.c_void_p(ptr), workspace_bytes, _stream_handle(stream))
    _check(code, "himuon_gram_ns")
    return workspace


def himuon_pair_stats_workspace(a: Sequence) -> int:
    """Workspace bytes himuon_pair_stats needs for pairs shaped like `a`."""
    d = _descs(a)
    nbytes = ctypes.c_size_t(0)
    _check(lib.himuon_pair_stats_workspace(d, len(a), ctypes.byref(nbytes)), "himuon_pair_stats_workspace")
    return nbytes.value


def _row_major(t) -> bool:
    return t.stride(1) == 1 or t.shape[1] == 1


def himuon_pair_stats(a: Sequence, b: Sequence, out=None, workspace=None, stream=None):
    """(n, 3) float64 device tensor: sum a*b, sum a*a, sum b*b for each pair.

    a[i] and b[i] are equal-shaped bf16 or fp32 tensors with the same memory
    orientation (both row-major, or both transposed views); `out` and
    `workspace` are optional device tensors (float64 of 3n elements, uint8)."""
    import torch
    n = len(a)
    if len(b) != n:
        raise ValueError("a and b must have equal length")
    if n == 0:
        return torch.empty((0, 3), dtype=torch.float64)
    dtype = _dtype_code(a[0])
    for x, y in zip(a, b):
        if x.shape != y.shape:
            raise ValueError("pairs must have equal shapes")
        if _row_major(x) != _row_major(y):
            raise ValueError("both matrices of a pair must have the same orientation")
    da, db = _descs(a), _descs(b)
    dev = a[0].device
    if out is None:
        out = torch.empty((n, 3), dtype=torch.float64, device=dev)
    if workspace is None:
        workspace = torch.empty(max(himuon_pair_stats_workspace(a), 8), dtype=torch.uint8, device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    code = lib.himuon_pair_stats(da, db, n, dtype, ctypes.c_void_p(out.data_ptr()),
                                 ctypes.c_void_p(workspace.data_ptr()), nbytes, _stream_handle(stream))
    _check(code, "himuon_pair_stats")
    return out


def himuon_status_string(code: int) -> str:
    return lib.himuon_status_string(code).decode()


def himuon_last_hip_error() -> int:
    return lib.himuon_last_hip_error()


def himuon_version() -> int:
    return lib.himuon_version()
