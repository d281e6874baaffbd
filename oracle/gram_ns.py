"""fp64 reference for Gram Newton-Schulz (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use this
module; it shares no code with the HIP library.

Source: the "Gram Newton-Schulz" summary page.
* Section 5, Algorithm 2 (naive Gram Newton-Schulz): normalise X, then iterate
  on the small symmetric Gram matrix R = X X^T and a running product Q, and
  apply Q to X once at the end.
* Section 6, Algorithm 3 (stabilised): the same iteration with the identity
  terms added explicitly, and a restart part-way (the page restarts at step 3,
  after two steps): X <- Q X, R <- X X^T, Q <- I.

Per step t with (a, b, c) = (a_t, b_t, c_t):
    Z   = b R + c R^2
    Q   = Q Z + a Q
    RZ  = R Z + a R
    R   = Z RZ + a RZ
In exact arithmetic this is the standard map of the same page's Algorithm 1:
with X_t = (a I + b R + c R^2) X_{t-1}, Q_t X_0 = X_t and R_t = X_t X_t^T.

Readings of points the page leaves open:
* After its five-step loop, Algorithm 3 applies the running product with the
  index of step four.  The product of all steps run is applied here (step five's
  for five steps), the only reading under which the iteration equals
  Algorithm 1.
* A tall block is transposed first so that R is the smaller Gram matrix (the
  page's input has n <= m); the result is transposed back.
* restart = k restarts before step k + 1 (the page's t = 3 is restart = 2);
  restart = 0 never restarts (Algorithm 2's naive form).

Parity status: pinned by tests/test_oracle_gram.py against full_matrix_ns (an
independent form of the standard map) for several shapes, step counts and
restart points.
"""
from __future__ import annotations

import numpy as np

from .tiled_ns import EPS_DEFAULT, _coeff_list


def gram_ns(M, coeffs, restart: int = 2, eps: float = EPS_DEFAULT, K: int | None = None,
            return_parts: bool = False):
    """Full-matrix Newton-Schulz of M through its Gram matrix (Algorithm 3).

    With return_parts the result is (out, Q, X): the running product and the
    base it is applied to at the end, both in the short orientation (X is the
    normalised input advanced by the steps before the last restart)."""
    steps = _coeff_list(coeffs, K)
    X = np.array(M, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("gram_ns takes a 2-D matrix")
    X = X / (np.linalg.norm(X, "fro") + eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    n = X.shape[0]
    eye = np.eye(n)
    R = X @ X.T
    Q = eye.copy()
    for t, (a, b, c) in enumerate(steps, start=1):
        if restart > 0 and t == restart + 1:
            X = Q @ X
            R = X @ X.T
            Q = eye.copy()
        Z = b * R + c * (R @ R)
        Q = Q @ Z + a * Q
        RZ = R @ Z + a * R
        R = Z @ RZ + a * RZ
    out = Q @ X
    if transposed:
        out = out.T
    out = np.ascontiguousarray(out)
    return (out, Q, X) if return_parts else out
