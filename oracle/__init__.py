"""Plain fp64 CPU oracle for the HiMuon tiled Newton-Schulz step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library in
``tiled_newton_schulz_amd/``; the two meet only through the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

Sources (cited by page title and section):

* "Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
  Optimization" (arXiv 2606.27216), abstract: each momentum-gradient matrix is
  partitioned into T x T tiles, the same finite Newton-Schulz map is applied to
  every tile independently, and the results are reassembled.
* "Gram Newton-Schulz" summary page, section 3 (Muon recap): the update rule
  M_k = mu M_{k-1} + G_k, W_{k+1} = W_k - eta polar(M_k); Algorithm 1
  (standard Newton-Schulz): Frobenius normalisation with epsilon 1e-7, optional
  transpose so the Gram matrix is the small one, then per step
  A = X X^T, B = b_t A + c_t A^2, X = a_t X + B X.  The same section's SVD view:
  the iteration applies a scalar odd polynomial to the singular values and keeps
  the singular vectors.

Readings of points the pages leave open:

* ragged edges: tiles are anchored at (0, 0); the last tile row/column holds the
  remainder and is processed at its own h x w size;
* orientation: the pages give a transpose only as a cost trick; since every
  step is an odd matrix polynomial, X q(X^T X) = q(X X^T) X, so the result does
  not depend on it.  The oracle transposes tall tiles so its Gram matrix is the
  short side, min(h, w)^2;
* epsilon is added to the norm, not to its square;
* the pages give no numeric (a, b, c); callers pass one triple per step.

The submodule ``oracle.diagnostics`` holds the tiled-versus-full-map measures
(distance, cosine, output spectrum), pinned by
``tests/test_oracle_diagnostics.py``.

``ns_map_stack_torch`` runs the same steps with torch CPU float64 batched
products, for checks over whole workloads; it is pinned against ``ns_map``
and the SVD closed form.

Parity status: every function below is pinned by ``tests/test_oracle.py``
(SVD closed form, independent full-matrix form, exact rational brute force,
tile independence, transpose symmetry, zero padding, closed forms for rank-1,
scaled-orthogonal and diagonal tiles).  No function here is "parity unpinned".
"""
from .tiled_ns import (  # noqa: F401
    EPS_DEFAULT,
    QUINTIC_COEFFS,
    ns_map,
    ns_map_stack,
    ns_map_stack_torch,
    full_matrix_ns,
    tile_grid,
    tiled_ns,
    tiled_ns_tile,
    tiled_ns_schedule,
    muon_step,
    tile_rel_errors,
    tile_rel_error,
    algorithmic_flops,
    nominal_flops,
)
from . import diagnostics  # noqa: F401,E402
