"""Seeded synthetic inputs shared by the tests, the bench and smoke().

This module holds shapes, seeds and random-number draws only; it contains none
of the Newton-Schulz arithmetic, so neither the HIP path nor the oracle
depends on the other through it.

Workloads (sizes as the tiled Newton-Schulz workloads state them):

* ``fp32_256x512``: one fp32 256 x 512 matrix, iid N(0, 1) from numpy seed 0;
  T = 64 (32 tiles; T = 128 gives 8 tiles); K = 5.
* ``layer_d2048``: one transformer layer at d = 2048 in bf16, iid N(0, 1):
  Q, K, V, O 2048 x 2048 and MLP 2048 x 5632, 2048 x 5632, 5632 x 2048;
  T = 128, K = 5; one batched launch.
* ``layers24_d2048``: 24 such layers (168 matrices, 1,233,125,376 elements),
  bf16 N(0, 0.02^2) times a per-matrix scale drawn log-uniform in [0.1, 10];
  T in {32, 64, 128, 256}, plus the full-matrix comparison.
* ``moe64``: 64 experts, each a 4096 x 1408 up and a 1408 x 4096 down matrix,
  bf16 N(0, 1); T = 256 leaves ragged 128-wide edge tiles.
* ``dense8192``: 8192 x 28672 and 28672 x 8192, bf16 N(0, 1); T = 512 with a
  4 GiB workspace cap; tile sizes 128, 256 and 512 chosen at run time.

Seeds: the fp32 workload uses numpy ``default_rng(0)`` as stated; every other
matrix i of workload c uses its own stream seeded with (c, i) so that any
single matrix can be regenerated alone.  Host generation draws float64 with
numpy PCG64 and rounds to the storage dtype (round to nearest even); device
generation (for the multi-GB workloads) uses torch's Philox generator on the
GPU seeded the same way, and the checks copy the sampled inputs back to the
host before the call that overwrites them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

COEFFS = (3.4445, -4.7750, 2.0315)


@dataclass
class Workload:
    name: str
    shapes: list            # [(H, W), ...]
    dtype: str              # "bf16" | "fp32"
    T: int
    K: int = 5
    std: float = 1.0
    log_uniform_scale: tuple | None = None   # (lo, hi) per-matrix scale range
    seed_id: int = 0
    Ts: tuple = ()
    workspace_cap: int | None = None
    note: str = ""

    @property
    def elements(self) -> int:
        return sum(h * w for h, w in self.shapes)


def _layer_shapes(d=2048, f=5632):
    return [(d, d)] * 4 + [(d, f), (d, f), (f, d)]


WORKLOADS = {
    "fp32_256x512": Workload("fp32_256x512", [(256, 512)], "fp32", 64, seed_id=1, Ts=(64, 128)),
    "layer_d2048": Workload("layer_d2048", _layer_shapes(), "bf16", 128, seed_id=2),
    "layers24_d2048": Workload("layers24_d2048", _layer_shapes() * 24, "bf16", 128, std=0.02,
                               log_uniform_scale=(0.1, 10.0), seed_id=3, Ts=(32, 64, 128, 256)),
    "moe64": Workload("moe64", [(4096, 1408), (1408, 4096)] * 64, "bf16", 256, seed_id=4),
    "dense8192": Workload("dense8192", [(8192, 28672), (28672, 8192)], "bf16", 512, seed_id=5,
                          Ts=(128, 256, 512), workspace_cap=4 << 30),
}


def matrix_scale(w: Workload, i: int) -> float:
    """Per-matrix multiplier: std times, where requested, a log-uniform scale."""
    s = w.std
    if w.log_uniform_scale is not None:
        lo, hi = w.log_uniform_scale
        u = np.random.default_rng([w.seed_id, i, 7]).random()
        s *= math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return s


def host_matrix(w: Workload, i: int, shape=None) -> np.ndarray:
    """Matrix i of workload w drawn on the host as float64 (before rounding)."""
    H, W = shape if shape is not None else w.shapes[i]
    if w.name == "fp32_256x512" and i == 0 and shape is None:
        x = np.random.default_rng(0).standard_normal((H, W))
    else:
        x = np.random.default_rng([w.seed_id, i]).standard_normal((H, W))
    return x * matrix_scale(w, i)


def round_to(x: np.ndarray, dtype: str):
    """Round float64 values to the storage dtype (nearest even); returns a torch
    CPU tensor of that dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.float32 if dtype == "fp32" else torch.bfloat16)


def host_tensors(w: Workload, idx=None):
    """Host (CPU) torch tensors of the workload, rounded to its dtype."""
    idx = range(len(w.shapes)) if idx is None else idx
    return [round_to(host_matrix(w, i), w.dtype) for i in idx]


def device_tensors(w: Workload, device="cuda", idx=None):
    """Device tensors generated on the GPU with torch's seeded Philox stream
    (used for workloads too large to draw on the host)."""
    import torch
    idx = range(len(w.shapes)) if idx is None else idx
    out = []
    dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    for i in idx:
        H, W = w.shapes[i]
        g = torch.Generator(device=device)
        g.manual_seed(1_000_003 * w.seed_id + i)
        x = torch.randn((H, W), generator=g, device=device, dtype=torch.float32)
        x.mul_(matrix_scale(w, i))
        out.append(x.to(dt))
        del x
    return out


def random_shapes(n, lo, hi, seed):
    """n random (H, W) pairs with each side uniform in [lo, hi]."""
    rng = np.random.default_rng([99, seed])
    return [(int(a), int(b)) for a, b in rng.integers(lo, hi + 1, size=(n, 2))]
