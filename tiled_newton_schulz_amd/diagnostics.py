"""How far the tiled map lies from the full-matrix map, on the GPU.

The HiMuon abstract presents the tiled Newton-Schulz map as a local stand-in
for the full-matrix one: each tile is orthogonalised on its own, where the full
map couples all rows and columns.  The pages give no measure of the gap; this
module reports the plain ones, per matrix and over the whole batch:

* relative Frobenius distance  ||tiled - full||_F / ||full||_F;
* cosine similarity            <tiled, full>_F / (||tiled||_F ||full||_F);
* optionally the spectral moments of each output, sum s^2, s^4 and s^6 over
  its singular values s, and from them the orthogonality residual
  RMS(s^2 - 1) = sqrt(||G - I||_F^2 / r), G the Gram matrix of the shorter
  side (the "Gram Newton-Schulz" page, section 3: each step moves every
  singular value through the same odd polynomial, so an orthogonalised
  update has them near 1).

Both maps run in libhimuon (himuon_tiled_ns; the full map is the same call
with one tile per matrix), and the three sums behind the two measures come
from himuon_pair_stats.  The moments come from the library too: with
Xn = X / ||X||_F and Y = Xn Xn^T Xn (one step of the map with coefficients
(0, 1, 0) at T = max(H, W), on an fp32 copy), the pair sums of (Y, X) are
<Y, X> = m4 / ||X||^3, <Y, Y> = m6 / ||X||^6 and <X, X> = m2.

The outputs are the library's bf16 (or fp32) results, so the distance carries
their rounding: about 2^-9 per element for bf16.
"""
from __future__ import annotations

import math
from typing import Sequence

from . import himuon_pair_stats, himuon_tiled_ns

QUINTIC = (3.4445, -4.7750, 2.0315)


def measures(stats) -> tuple[float, float]:
    """(distance, cosine) from one row (sum g*f, sum g*g, sum f*f) of pair
    sums, g the tiled output and f the full map."""
    gf, gg, ff = (float(x) for x in stats)
    dist = math.sqrt(max(gg + ff - 2.0 * gf, 0.0) / ff) if ff > 0 else float("nan")
    cos = gf / math.sqrt(gg * ff) if gg > 0 and ff > 0 else float("nan")
    return dist, cos


def spectral_moments(mats: Sequence) -> list[tuple[int, float, float, float]]:
    """(r, sum s^2, sum s^4, sum s^6) per matrix, s its r = min(H, W)
    singular values, computed by the library's kernels in fp32 (relative
    error about 1e-6)."""
    import torch

    out = [(min(m.shape), 0.0, 0.0, 0.0) for m in mats]
    idx = [i for i, m in enumerate(mats) if m.numel() > 0]
    if not idx:
        return out
    xs = [mats[i].to(torch.float32).contiguous() for i in idx]
    st = himuon_pair_stats(xs, xs).cpu().tolist()
    live = [j for j, row in enumerate(st) if row[2] > 0.0]
    if live:
        xl = [xs[j] for j in live]
        ys = [x.clone() for x in xl]
        himuon_tiled_ns(ys, max(max(x.shape) for x in xl), 1, [(0.0, 1.0, 0.0)], eps=0.0)
        ps = himuon_pair_stats(ys, xl).cpu().tolist()
        for j, (yx, yy, xx) in zip(live, ps):
            n2 = st[j][2]
            out[idx[j]] = (min(xs[j].shape), n2, yx * n2 ** 1.5, yy * n2 ** 3)
    return out


def orthogonality_residual(moments) -> float:
    """RMS of s^2 - 1 over the singular values: sqrt((m4 - 2 m2 + r) / r)."""
    r, m2, m4, _ = moments
    return math.sqrt(max(m4 - 2.0 * m2 + r, 0.0) / r) if r > 0 else 0.0


def tiled_vs_full(mats: Sequence, Ts: Sequence[int], K: int = 5, abc=QUINTIC, eps: float = 1e-7,
                  spectrum: bool = False) -> dict:
    """Compare tiledNS_T(M) with the full-matrix map for each T in Ts.

    mats: 2-D bf16 or fp32 CUDA tensors (read only; the maps run on copies).
    Returns {"full_T": T used for the full map, "rows": [...]} where each row
    holds T, the batch distance and cosine, and per-matrix (distance, cosine);
    with spectrum=True each row also holds the outputs' spectral moments
    ("moments") and the result holds the full map's ("full_moments").
    """
    if len(mats) == 0:
        return {"full_T": 0, "rows": []}
    full_T = max(max(m.shape) for m in mats)
    full = [m.clone() for m in mats]
    himuon_tiled_ns(full, full_T, K, abc, eps)
    result = {"full_T": full_T, "rows": []}
    if spectrum:
        result["full_moments"] = spectral_moments(full)
    for T in Ts:
        tiled = [m.clone() for m in mats]
        himuon_tiled_ns(tiled, int(T), K, abc, eps)
        st = himuon_pair_stats(tiled, full).cpu()
        per = [measures(r) for r in st.tolist()]
        dist, cos = measures(st.sum(dim=0).tolist())
        row = {"T": int(T), "distance": dist, "cosine": cos, "per_matrix": per, "stats": st}
        if spectrum:
            row["moments"] = spectral_moments(tiled)
        result["rows"].append(row)
        del tiled
    return result


def _main():
    import argparse

    import torch

    ap = argparse.ArgumentParser(description="tiled versus full-matrix Newton-Schulz on synthetic matrices")
    ap.add_argument("--shapes", default="2048x2048,2048x5632,5632x2048",
                    help="comma-separated HxW of bf16 N(0,1) matrices")
    ap.add_argument("--T", type=int, nargs="+", default=[32, 64, 128, 256, 512])
    ap.add_argument("--K", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--spectrum", action="store_true")
    args = ap.parse_args()
    g = torch.Generator(device="cpu").manual_seed(args.seed)
    mats = []
    for s in args.shapes.split(","):
        h, w = (int(x) for x in s.lower().split("x"))
        mats.append(torch.randn(h, w, generator=g).to(torch.bfloat16).cuda())
    res = tiled_vs_full(mats, args.T, K=args.K, spectrum=args.spectrum)
    print(f"full map: T = {res['full_T']}")
    print("T      distance   cosine    " + "  ".join(f"m{i}:dist" for i in range(len(mats))))
    for r in res["rows"]:
        per = "  ".join(f"{d:8.4f}" for d, _ in r["per_matrix"])
        print(f"{r['T']:<6d} {r['distance']:9.5f}  {r['cosine']:8.5f}  {per}")
        if args.spectrum:
            for i, m in enumerate(r["moments"]):
                print(f"       m{i}: mean s^2 {m[1] / m[0]:.4f}, RMS(s^2 - 1) {orthogonality_residual(m):.4f}")
    if args.spectrum:
        for i, m in enumerate(res["full_moments"]):
            print(f"full   m{i}: mean s^2 {m[1] / m[0]:.4f}, RMS(s^2 - 1) {orthogonality_residual(m):.4f}")


if __name__ == "__main__":
    _main()
