"""fp64 reference implementation of tiled Newton-Schulz (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use this
module.  See the package docstring for the passages it follows.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

# Algorithm 1 of the "Gram Newton-Schulz" summary page normalises with
# ||X||_F + epsilon, epsilon = 1e-7.
EPS_DEFAULT = 1e-7
# The pages name per-step coefficients (a_t, b_t, c_t) but print no values; this
# widely used quintic triple is the one the workloads use for every step.
QUINTIC_COEFFS = (3.4445, -4.7750, 2.0315)


def _coeff_list(coeffs, K=None):
    """Normalise coefficients to a list of K (a, b, c) triples."""
    if K == 0:
        return []
    arr = np.asarray(coeffs, dtype=np.float64)
    if arr.size == 0 and K is None:
        return []
    if arr.ndim == 1:
        if arr.shape[0] != 3:
            raise ValueError("a single coefficient triple must have 3 entries")
        if K is None:
            raise ValueError("K is required with a single triple")
        return [tuple(arr)] * int(K)
    if arr.ndim != 2 or arr.shape[1] != 3:
        raise ValueError("coefficients must be (K, 3)")
    if K is not None and arr.shape[0] != K:
        raise ValueError("need one triple per step")
    return [tuple(r) for r in arr]


def ns_map(Y, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """The per-tile Newton-Schulz map, Algorithm 1 of the Gram Newton-Schulz page.

    Y: an h x w block (any real dtype; computed in float64).
    coeffs: (K, 3) per-step (a_t, b_t, c_t), or one triple with K given.
    Returns the h x w float64 result.

    Steps, in the page's order: X = Y / (||Y||_F + eps); transpose if the block
    is tall so that A = X X^T is the smaller Gram matrix; for each step
    A = X X^T, B = b A + c A A, X = a X + B X; undo the transpose.
    """
    steps = _coeff_list(coeffs, K)
    X = np.array(Y, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("ns_map takes a 2-D block")
    norm = math.sqrt(float(np.sum(X * X)))
    X = X / (norm + eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    for a, b, c in steps:
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if transposed:
        X = X.T
    return np.ascontiguousarray(X)


def ns_map_stack(Ys, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """ns_map applied to every block of an (N, h, w) stack.

    The same arithmetic as ns_map, with each matmul taken over the stack; blocks
    do not interact.  Used to time and check many equal-shaped tiles.
    """
    steps = _coeff_list(coeffs, K)
    X = np.array(Ys, dtype=np.float64, copy=True)
    if X.ndim != 3:
        raise ValueError("ns_map_stack takes an (N, h, w) stack")
    norms = np.sqrt(np.sum(X * X, axis=(1, 2)))
    X = X / (norms + eps)[:, None, None]
    transposed = X.shape[1] > X.shape[2]
    if transposed:
        X = np.swapaxes(X, 1, 2)
    for a, b, c in steps:
        A = X @ np.swapaxes(X, 1, 2)
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    if transposed:
        X = np.swapaxes(X, 1, 2)
    return np.ascontiguousarray(X)


def ns_map_stack_torch(Ys, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """ns_map on every block of an (N, h, w) stack, with torch CPU float64
    batched products in place of numpy's (same steps and order as ns_map;
    torch runs the batch on all host threads).  Takes and returns a torch
    float64 CPU tensor; used to check whole workloads of 10^5 - 10^6 tiles."""
    import torch
    steps = _coeff_list(coeffs, K)
    X = torch.as_tensor(Ys, dtype=torch.float64, device="cpu").clone()
    if X.dim() != 3:
        raise ValueError("ns_map_stack_torch takes an (N, h, w) stack")
    norms = torch.sqrt(torch.sum(X * X, dim=(1, 2)))
    X = X / (norms + eps)[:, None, None]
    transposed = X.shape[1] > X.shape[2]
    if transposed:
        X = X.transpose(1, 2)
    for a, b, c in steps:
        A = torch.bmm(X, X.transpose(1, 2))
        B = b * A + c * torch.bmm(A, A)
        X = a * X + torch.bmm(B, X)
    if transposed:
        X = X.transpose(1, 2)
    return X.contiguous()


def full_matrix_ns(M, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """Full-matrix Newton-Schulz, written independently of ns_map.

    It uses the right-hand Gram form for tall matrices: with G = X^T X,
    X <- a X + X (b G + c G^2), which equals the left form because each step is
    an odd polynomial in X.  Used to pin tiled_ns at T >= max(H, W).
    """
    steps = _coeff_list(coeffs, K)
    X = np.asarray(M, dtype=np.float64)
    X = X / (np.linalg.norm(X, "fro") + eps)
    tall = X.shape[0] > X.shape[1]
    for a, b, c in steps:
        if tall:
            G = X.T @ X
            X = a * X + X @ (b * G + c * np.linalg.matrix_power(G, 2))
        else:
            G = X @ X.T
            X = a * X + (b * G + c * np.linalg.matrix_power(G, 2)) @ X
    return X


def tile_grid(H: int, W: int, T: int):
    """Tile boxes (r0, r1, c0, c1) of an H x W matrix cut into T x T tiles.

    Tiles are anchored at (0, 0); the last row/column of tiles holds the
    remainder, so a matrix has ceil(H/T) * ceil(W/T) tiles, in row-major order.
    """
    if H < 1 or W < 1 or T < 1:
        raise ValueError("H, W, T must be positive")
    boxes = []
    for r0 in range(0, H, T):
        for c0 in range(0, W, T):
            boxes.append((r0, min(r0 + T, H), c0, min(c0 + T, W)))
    return boxes


def tiled_ns(X, T: int, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """HiMuon tiled Newton-Schulz on one matrix (abstract of the HiMuon paper).

    Every T x T tile (edge tiles at their own size) gets ns_map on its own and
    the results are reassembled into an H x W float64 array.
    """
    X = np.asarray(X)
    H, W = X.shape
    out = np.empty((H, W), dtype=np.float64)
    for r0, r1, c0, c1 in tile_grid(H, W, T):
        out[r0:r1, c0:c1] = ns_map(X[r0:r1, c0:c1], coeffs, eps, K)
    return out


def tiled_ns_tile(X, T: int, ti: int, tj: int, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """The (ti, tj) tile of tiled_ns(X, T, ...), computed on its own."""
    X = np.asarray(X)
    H, W = X.shape
    r0, c0 = ti * T, tj * T
    if not (0 <= r0 < H and 0 <= c0 < W):
        raise IndexError("tile index out of range")
    return ns_map(X[r0:min(r0 + T, H), c0:min(c0 + T, W)], coeffs, eps, K)


def tiled_ns_schedule(X, Ts: Sequence[int], coeffs, eps: float = EPS_DEFAULT):
    """Coarse-to-fine tile schedule inside one call: step t uses tile size Ts[t].

    Reading of the abstract's "runtime tile-size schedules" as a per-step tile
    size: normalise once, on the tiles of the first (largest) size, then run
    step t on the tiles of size Ts[t].  Sizes must not increase and each must
    divide the one before, so every finer tile lies inside one coarser tile.
    """
    steps = _coeff_list(coeffs, len(Ts))
    Ts = [int(t) for t in Ts]
    for t0, t1 in zip(Ts, Ts[1:]):
        if t1 > t0 or t0 % t1 != 0:
            raise ValueError("tile sizes must be non-increasing and nested")
    X = np.array(X, dtype=np.float64, copy=True)
    H, W = X.shape
    for r0, r1, c0, c1 in tile_grid(H, W, Ts[0]):
        blk = X[r0:r1, c0:c1]
        X[r0:r1, c0:c1] = blk / (math.sqrt(float(np.sum(blk * blk))) + eps)
    for (a, b, c), T in zip(steps, Ts):
        for r0, r1, c0, c1 in tile_grid(H, W, T):
            Y = X[r0:r1, c0:c1]
            tall = Y.shape[0] > Y.shape[1]
            if tall:
                Y = Y.T
            A = Y @ Y.T
            B = b * A + c * (A @ A)
            Y = a * Y + B @ Y
            X[r0:r1, c0:c1] = Y.T if tall else Y
    return X


def muon_step(W, M, G, mu: float, eta: float, T: int, coeffs, eps: float = EPS_DEFAULT, K: int | None = None):
    """One Muon update with tiled orthogonalisation (Muon recap of the Gram
    Newton-Schulz page, with polar() replaced by the tiled map):
    M_new = mu M + G;  W_new = W - eta * tiled_ns(M_new).

    Returns (W_new, M_new) in float64.  The caller may round M_new to the
    storage dtype before passing it to tiled_ns to mirror a stored momentum.
    """
    M_new = mu * np.asarray(M, dtype=np.float64) + np.asarray(G, dtype=np.float64)
    U = tiled_ns(M_new, T, coeffs, eps, K)
    return np.asarray(W, dtype=np.float64) - eta * U, M_new


def tile_rel_error(got, ref):
    """Relative Frobenius error ||got - ref||_F / ||ref||_F of one block
    (absolute error when ref is exactly zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm(got - ref))
    den = float(np.linalg.norm(ref))
    return num / den if den > 0 else num


def tile_rel_errors(got, ref, T: int):
    """Per-tile relative Frobenius errors between two H x W arrays."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    H, W = ref.shape
    return np.array([tile_rel_error(got[r0:r1, c0:c1], ref[r0:r1, c0:c1])
                     for r0, r1, c0, c1 in tile_grid(H, W, T)])


def nominal_flops(shapes: Iterable[tuple[int, int]], T: int, K: int) -> float:
    """Useful work as the workload metric counts it: sum of 6 H W T K."""
    return float(sum(6.0 * H * W * T * K for H, W in shapes))


def algorithmic_flops(shapes: Iterable[tuple[int, int]], T: int, K: int) -> float:
    """Per-tile work of Algorithm 1 as the Gram Newton-Schulz page's runtime
    section counts it (X X^T: 2 m n^2, A^2: 2 n^3, B X: 2 m n^2 for an n x m
    block with n <= m), summed over all tiles and K steps."""
    tot = 0.0
    for H, W in shapes:
        for r0, r1, c0, c1 in tile_grid(H, W, T):
            n, m = sorted((r1 - r0, c1 - c0))
            tot += (2.0 * m * n * n + 2.0 * n ** 3 + 2.0 * m * n * n) * K
    return tot
