"""Throughput of the HiMuon tiled Newton-Schulz step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]

A step is one himuon_tiled_ns call over the whole workload (all matrices of
the batch, every tile, all K Newton-Schulz steps), with the inputs already
resident in HBM.  The default workload is one transformer layer at d = 2048
in bf16 (Q, K, V, O 2048 x 2048, MLP 2048 x 5632, 2048 x 5632, 5632 x 2048),
T = 128, K = 5, one batched launch.  Each timed step runs on the previous
step's output; the work does not depend on the values.

Prints one JSON line: useful TFLOP/s counted as sum 6 H W T K (value),
matrices/s, % of the bf16 MFMA peak, the roofline of the dominant kernel
(algorithmic flops per launch over the launch time measured with HIP events
on the launch stream), and the fp64 CPU oracle timed on a bounded sample on
the host cores.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def algorithmic_flops(shapes, T, K):
    """Sum over tiles of 2 r^2 (2 s + r) K, by tile shape class."""
    tot = 0.0
    for H, W in shapes:
        fh, rh = divmod(H, T)
        fw, rw = divmod(W, T)
        for nh, h in ((fh, T), (1 if rh else 0, rh)):
            for nw, w in ((fw, T), (1 if rw else 0, rw)):
                if nh and nw:
                    r, s = min(h, w), max(h, w)
                    tot += nh * nw * 2.0 * r * r * (2 * s + r) * K
    return tot


def cpu_baseline(w, T, K, min_seconds=10.0, max_seconds=30.0):
    """The fp64 oracle, as it stands, on whole matrices of the workload drawn on
    the host, repeated until at least min_seconds have passed."""
    import numpy as np

    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    mats = []
    for i in range(len(w.shapes)):
        mats.append(workloads.round_to(workloads.host_matrix(w, i), w.dtype).double().numpy())
    done_shapes = []
    t0 = time.perf_counter()
    i = 0
    while True:
        oracle.tiled_ns(mats[i % len(mats)], T, w_coeffs(), K=K)
        done_shapes.append(mats[i % len(mats)].shape)
        i += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el >= max_seconds:
            break
    flops = sum(6.0 * h * ww * T * K for h, ww in done_shapes)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(done_shapes)} whole matrices of the workload ({i} oracle calls, fp64 numpy, "
                      f"{el:.1f} s), same T and K",
            "matrices_per_s": len(done_shapes) / el}


def w_coeffs():
    import workloads
    return workloads.COEFFS


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="layer_d2048")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--K", type=int, default=5)
    ap.add_argument("--cap", type=int, default=None, help="workspace cap in bytes")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times (used to "
                         "calibrate the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the tiled map has no "
              "cross-GPU exchange and this build measures one GPU's share", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return

    import tiled_newton_schulz_amd as H
    import workloads

    w = workloads.WORKLOADS[args.workload]
    T = args.T or w.T
    K = args.K
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.elements > 200_000_000:
        mats = workloads.device_tensors(w, device=dev)
    else:
        mats = [t.to(dev) for t in workloads.host_tensors(w)]
    shapes = [tuple(m.shape) for m in mats]
    cap = args.cap if args.cap is not None else w.workspace_cap
    full, mn = H.himuon_workspace_size(mats, T)
    ws = None
    ws_bytes = 0
    if full:
        ws_bytes = min(full, cap) if cap else full
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    plan = H.himuon_plan(mats, T, K, H.BF16 if w.dtype == "bf16" else H.FP32, ws_bytes)
    stream = torch.cuda.current_stream()

    def step():
        H.himuon_tiled_ns(mats, T, K, workloads.COEFFS, workspace=ws, workspace_bytes=ws_bytes, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / args.steps

    nominal = sum(6.0 * h * ww * T * K for h, ww in shapes)
    alg = algorithmic_flops(shapes, T, K)
    tflops = nominal / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    launches = plan["launches"]
    # the dominant kernel: the on-chip kernel when the whole step is one launch
    per_launch_ms = ms_per_step / max(1, launches)
    achieved = alg / launches / (per_launch_ms * 1e-3) / 1e12 if launches else 0.0
    io_bytes = 2.0 * sum(h * ww for h, ww in shapes) * (2 if w.dtype == "bf16" else 4)
    out = {
        "metric": "tiled-NS TFLOP/s (6*H*W*T*K) and % bf16 MFMA peak; matrices/s per step",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) bf16, transformer-layer shapes)",
        "config": {"workload": w.name, "matrices": len(shapes), "T": T, "K": K,
                   "elements": sum(h * ww for h, ww in shapes), "launches_per_step": launches,
                   "tiles": plan["tiles"], "chunks": plan["chunks"], "workspace_bytes": ws_bytes,
                   "parallelism": "single GPU"},
        "matrices_per_s": round(len(shapes) / (ms_per_step * 1e-3), 1),
        "pct_bf16_peak": round(100.0 * tflops / peak, 2),
        "algorithmic_tflops": round(alg / (ms_per_step * 1e-3) / 1e12, 3),
        "hbm_gbs_io": round(io_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, T, K)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
