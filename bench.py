"""Throughput of the HiMuon tiled Newton-Schulz step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--T T]
    python bench.py --gram [--restart 2] --workload NAME   # full map through the Gram iteration

A step is one himuon_tiled_ns call over the whole workload (all matrices of
the batch, every tile, all K Newton-Schulz steps), with the inputs already
resident in HBM.  The default workload is the cross-layer batch of 24
transformer layers at d = 2048 in bf16 (per layer Q, K, V, O 2048 x 2048 and
MLP 2048 x 5632, 2048 x 5632, 5632 x 2048: 168 matrices, 1.23 G elements),
T = 128, K = 5, batched into one on-chip launch plus a launch for the partial
last round.  Each timed step runs on the previous step's output; the work does
not depend on the values.  Warm-up runs at least --warmup steps and at least
--warmup-seconds.

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

METRIC = "tiled-NS TFLOP/s (6\u00b7H\u00b7W\u00b7T\u00b7K) and % bf16 MFMA peak; matrices/s per step"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# Context only (another method on another machine): the Gram Newton-Schulz
# page reports its Gram iteration cutting orthogonalisation-step time by
# 40-50 % against standard Newton-Schulz on Hopper/Blackwell-class GPUs
# (contributions; speed-up table).
CONTEXT = {"gram_ns_page_cut": "40-50 % less orthogonalisation-step time for Gram Newton-Schulz vs standard "
                               "Newton-Schulz on Hopper/Blackwell-class GPUs, as the Gram Newton-Schulz page "
                               "reports it (context only: different method and hardware; the in-run comparison "
                               "here is bench.py --gram)",
           "gram_ns_page_cut_pct": [40, 50]}


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


CPU_SHARE = 16   # host cores of one GPU's share of the box
_CPU_MATS = []    # the sampled matrices, drawn before the workers fork


def _oracle_bands(job):
    """Worker: the oracle on whole T-row bands of the sampled matrices (a band
    is tiled exactly as inside its matrix), with BLAS held to one thread."""
    from threadpoolctl import threadpool_limits

    import oracle
    bands, T, K = job
    with threadpool_limits(limits=1):
        t0 = time.time()
        for i, r0 in bands:
            oracle.tiled_ns(_CPU_MATS[i][r0:r0 + T], T, w_coeffs(), K=K)
        return t0, time.time()


def _device_fds():
    """Open file descriptors of this process on GPU device nodes."""
    out = []
    try:
        for fd in os.listdir("/proc/self/fd"):
            try:
                tgt = os.readlink(f"/proc/self/fd/{fd}")
            except OSError:
                continue
            if tgt.startswith("/dev/kfd") or tgt.startswith("/dev/dri"):
                out.append(tgt)
    except OSError:
        pass
    return out


def cpu_baseline(w, T, K, target_s=10.0):
    """The fp64 oracle, as it stands, timed on the host cores: one worker
    process per core (BLAS one thread each) with the tiles split between them
    as whole T-row bands, plus a single-core figure.  Runs before this process
    touches the GPU, so the forked workers hold no device state.  The sample is
    the workload's first (up to) 7 matrices, taken as many times as fill about
    target_s seconds at the single-core rate times the worker count; the
    oracle's time does not depend on the values."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import oracle
    import workloads
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, CPU_SHARE))
    _CPU_MATS.clear()
    nm = min(7, len(w.shapes))
    for i in range(nm):
        _CPU_MATS.append(workloads.round_to(workloads.host_matrix(w, i), w.dtype).double().numpy())
    # single core: bands of the first matrix for about 2 s
    x0 = _CPU_MATS[0]
    done, t0 = [], time.perf_counter()
    with threadpool_limits(limits=1):
        for r0 in range(0, x0.shape[0], T):
            oracle.tiled_ns(x0[r0:r0 + T], T, w_coeffs(), K=K)
            done.append(r0)
            if time.perf_counter() - t0 >= 2.0:
                break
    t1 = time.perf_counter() - t0
    single = algorithmic_flops([tuple(x0[r0:r0 + T].shape) for r0 in done], T, K) / t1
    # all cores
    bands = [(i, r0) for i in range(nm) for r0 in range(0, _CPU_MATS[i].shape[0], T)]
    per_pass = sum(algorithmic_flops([tuple(_CPU_MATS[i][r0:r0 + T].shape)], T, K) for i, r0 in bands)
    reps = max(1, int(round(single * cores * target_s / per_pass)))
    bands = bands * reps
    res = {"unit": "TFLOP/s", "kind": "oracle", "single_core_tflops": round(single / 1e12, 6),
           "single_core_sample": f"{len(done)} T-row bands of matrix 0 {tuple(x0.shape)}, {t1:.1f} s, "
                                 "one BLAS thread",
           "affinity_cores": affinity}
    held = _device_fds()
    if held:
        # never fork a process that holds the GPU: report the single core only
        res.update({"value": round(single / 1e12, 6), "cores": 1,
                    "sample": res["single_core_sample"] + f" (workers not started: {len(held)} device fds open)"})
        _CPU_MATS.clear()
        return res
    jobs = [(bands[k::cores], T, K) for k in range(cores)]
    with mp.get_context("fork").Pool(cores) as pool:
        spans = pool.map(_oracle_bands, jobs, chunksize=1)
    wall = max(e for _, e in spans) - min(b for b, _ in spans)
    flops = per_pass * reps
    elems = sum(m.size for m in _CPU_MATS)
    _CPU_MATS.clear()
    res.update({"value": round(flops / wall / 1e12, 5), "cores": cores,
                "sample": f"{reps} pass(es) over the workload's first {nm} matrices ({elems:,} elements, "
                          f"{len(bands)} T-row bands) on {cores} worker processes, one BLAS thread each, fp64 "
                          f"numpy, {wall:.1f} s; same T and K",
                "matrices_per_s": round(nm * reps / wall, 3), "gflops_fp64": round(flops / wall / 1e9, 2),
                "wall_s": round(wall, 2)})
    return res


KERNEL_SOURCES = {
    "resident32_kernel": ["resident32.hip", "device_util.h", "common.h"],
    "resident_kernel<64>": ["resident.hip", "device_util.h", "common.h"],
    "resident_kernel<128>": ["resident.hip", "device_util.h", "common.h"],
    "resident_f32_kernel": ["resident_f32.hip", "common.h"],
    "resident256_kernel": ["resident256.hip", "device_util.h", "common.h"],
    "pair_stats": ["pair_stats.hip", "pair_stats.h"],
}
KERNEL_OF_TILE = {32: "resident32_kernel", 64: "resident_kernel<64>", 128: "resident_kernel<128>",
                  256: "resident256_kernel"}


def sources_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "tiled_newton_schulz_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload, T, tiles):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this kernel and workload, if the kernel sources are unchanged
    since the counters were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("workload") != workload or rec.get("T") != T or rec.get("tiles") != tiles:
        return None
    if rec.get("sources_sha256") != sources_sha(kernel):
        return None
    return rec.get("traffic_bytes")


def trim_tail(mats, T, tail):
    """Views of the matrices with `tail` full tiles removed (whole T-row bands
    from the bottom of one matrix), or None if no matrix allows it."""
    for i in range(len(mats) - 1, -1, -1):
        h, w = mats[i].shape
        per_band = -(-w // T)
        if h % T == 0 and w % T == 0 and tail % per_band == 0 and tail // per_band < h // T:
            out = list(mats)
            out[i] = mats[i][:h - (tail // per_band) * T]
            return out
    return None


def dominant_kernel_roofline(H, torch, mats, shapes, T, K, plan, stream, ms_per_step, alg, peak, w, steps):
    """Roofline of the kernel that takes most of a step, timed with HIP events
    on the launch stream.  A step that is one launch is timed as a whole; when a
    step is one on-chip launch plus a tail launch, the main launch alone is
    timed on the same matrices with the tail's tiles cut off (whole row bands),
    which gives the same kernel the same tile count it runs in the step.  The
    bound is the roofline with the longer floor for that work: MFMA (its
    algorithmic flops at the dtype's peak) or HBM (one read and one write of
    every element at 8 TB/s)."""
    dsize = 2 if w.dtype == "bf16" else 4
    nbytes = 2.0 * dsize * sum(h * ww for h, ww in shapes)
    kernel_tile = plan["kernel_tile"]
    main = "resident_f32_kernel" if w.dtype == "fp32" and kernel_tile == 64 else KERNEL_OF_TILE.get(kernel_tile)
    one_launch = plan["chunks"] == 0 and plan["resident_launches"] == 1
    if one_launch and plan["tail_tiles"] == 0 and main:
        kernel, tiles, ms, flops = main, plan["tiles"], ms_per_step, alg
    elif one_launch and main and trim_tail(mats, T, plan["tail_tiles"]) is not None:
        sub = trim_tail(mats, T, plan["tail_tiles"])
        sub_plan = H.himuon_plan(sub, T, K, H.BF16)
        assert sub_plan["launches"] == 1 and sub_plan["tiles"] == plan["tiles"] - plan["tail_tiles"]
        import workloads
        n = max(20, steps // 2)
        for _ in range(5):
            H.himuon_tiled_ns(sub, T, K, workloads.COEFFS, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            H.himuon_tiled_ns(sub, T, K, workloads.COEFFS, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        kernel, tiles, ms = main, sub_plan["tiles"], e0.elapsed_time(e1) / n
        flops = algorithmic_flops([tuple(m.shape) for m in sub], T, K)
        nbytes = 2.0 * dsize * sum(m.shape[0] * m.shape[1] for m in sub)
    else:
        kernel = f"whole step ({plan['launches']} launches)"
        tiles, ms, flops = plan["tiles"], ms_per_step, alg
    traffic = recorded_traffic(kernel, w.name, T, tiles) if kernel in KERNEL_SOURCES else None
    if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12):
        achieved = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kernel, "tiles": tiles,
                "launch_ms": round(ms, 5)}
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel, "tiles": tiles,
            "launch_ms": round(ms, 5)}


def pair_stats_bench(H, torch, w, mats, steps, warmup, no_cpu):
    """Time himuon_pair_stats over (matrix, copy) pairs of the workload: the
    three sums behind the tiled-versus-full distance and cosine.  A step is
    one call (per-workgroup partials, then the fixed-order finish); it reads
    every element of both matrices once, so the bound is HBM bandwidth."""
    a = mats
    b = [m.clone() for m in mats]
    es = 2 if w.dtype == "bf16" else 4
    nbytes = 2.0 * sum(m.numel() for m in mats) * es
    out = torch.empty((len(a), 3), dtype=torch.float64, device=a[0].device)
    ws = torch.empty(max(H.himuon_pair_stats_workspace(a), 8), dtype=torch.uint8, device=a[0].device)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        H.himuon_pair_stats(a, b, out=out, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        H.himuon_pair_stats(a, b, out=out, workspace=ws, stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "pair statistics GB/s (both matrices read once)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded normal entries, transformer-layer shapes)",
        "config": {"workload": w.name + " pair statistics", "pairs": len(a),
                   "elements": sum(m.numel() for m in mats), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": recorded_traffic("pair_stats", w.name, None, len(a)),
                     "kernel": "pair_partial_kernel + pair_final_kernel (whole call)", "launch_ms": round(ms, 5)},
    }
    if not no_cpu:
        import numpy as np

        from oracle import diagnostics as OD
        hx = [m.cpu().to(torch.float64).numpy() for m in mats[:2]]
        hy = [x.copy() for x in hx]
        n_el, t0, reps = 0, time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0 or reps == 0:
            for x, y in zip(hx, hy):
                OD.pair_stats(x, y)
                n_el += x.size
            reps += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(2.0 * n_el * es / dt / 1e9, 2), "unit": "GB/s (same byte count)",
                               "cores": 1, "kind": "oracle",
                               "sample": f"oracle pair_stats on the first {len(hx)} matrices, {reps} passes"}
        del np
    return res


def gram_flops(shapes, K, restart):
    """Full-product flops of the Gram iteration per call, summed over the
    matrices (r = shorter side, s = longer): R = X X^T and the final Q X
    (2 r^2 s each), per step R^2 (2 r^3), the running product (2 r^3, not on
    the first step after a start or restart) and the R update (4 r^3, not after
    the last step nor before a restart), and per restart Q X and X X^T."""
    tot = 0.0
    for h, w in shapes:
        r, s_ = float(min(h, w)), float(max(h, w))
        f = 4.0 * r * r * s_
        ident = True
        for t in range(1, K + 1):
            if restart and t == restart + 1:
                f += 4.0 * r * r * s_
                ident = True
            f += 2.0 * r ** 3 + (0.0 if ident else 2.0 * r ** 3)
            ident = False
            if t < K and not (restart and t == restart):
                f += 4.0 * r ** 3
        tot += f
    return tot


def muon_bench(H, torch, w, mats, T, K, steps, warmup, warmup_seconds, cap):
    """Time himuon_muon_step (M <- mu M + G, W <- W - eta tiledNS(M), fused)
    on the workload's matrices as M, with seeded G and W of the same shapes.
    The flops are the tiled map's; the HBM bytes are five passes over the
    elements (M, G and W read, M and W written).  M and W change from call to
    call, as they would over optimiser steps."""
    import workloads
    shapes = [tuple(m.shape) for m in mats]
    gen = torch.Generator(device=mats[0].device).manual_seed(12345)
    G = [(torch.randn(sh, device=mats[0].device, generator=gen) * 0.01).to(mats[0].dtype) for sh in shapes]
    W = [(torch.randn(sh, device=mats[0].device, generator=gen) * 0.02).to(mats[0].dtype) for sh in shapes]
    full, _ = H.himuon_workspace_size(mats, T)
    ws_bytes = (min(full, cap) if cap else full) if full else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=mats[0].device) if ws_bytes else None
    stream = torch.cuda.current_stream()

    def step():
        H.himuon_muon_step(W, mats, G, T, K, workloads.COEFFS, workspace=ws, workspace_bytes=ws_bytes,
                           stream=stream)

    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t0 < warmup_seconds:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    alg = algorithmic_flops(shapes, T, K)
    nominal = sum(6.0 * h * ww * T * K for h, ww in shapes)
    es = 2 if w.dtype == "bf16" else 4
    io_bytes = 5.0 * sum(h * ww for h, ww in shapes) * es
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = alg / (ms * 1e-3) / 1e12
    return {
        "metric": "fused Muon step (M <- mu M + G, W <- W - eta tiledNS(M)) TFLOP/s (6*H*W*T*K)",
        "value": round(nominal / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded normal M, G and W)",
        "config": {"workload": w.name, "matrices": len(shapes), "T": T, "K": K, "mu": 0.95, "eta": 0.02,
                   "elements": sum(h * ww for h, ww in shapes), "workspace_bytes": ws_bytes,
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "hbm_gbs_io": round(io_bytes / (ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None, "kernel": "whole step",
                     "hbm_floor_ms": round(io_bytes / 8e12 * 1e3, 4)},
        "warmup_steps_run": n_warm,
    }


def gram_bench(H, torch, w, mats, K, restart, steps, warmup, cap, no_cpu):
    """Time himuon_gram_ns (the full-matrix map through the Gram iteration)
    against himuon_tiled_ns with T = max(rows, cols) (the standard full map)
    on the same matrices, each with its own workspace.  The value is the
    standard map's algorithmic flops over the Gram call's time, so it compares
    directly with the standard map's rate; the roofline is the Gram
    iteration's own flops over its time."""
    import workloads
    shapes = [tuple(m.shape) for m in mats]
    Tf = max(max(sh) for sh in shapes)
    stream = torch.cuda.current_stream()
    gfull, _ = H.himuon_gram_ns_workspace(mats)
    gbytes = min(gfull, cap) if cap else gfull
    gws = torch.empty(max(gbytes, 1), dtype=torch.uint8, device=mats[0].device)
    sfull, _ = H.himuon_workspace_size(mats, Tf)
    sbytes = min(sfull, cap) if cap else sfull
    sws = torch.empty(max(sbytes, 1), dtype=torch.uint8, device=mats[0].device)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_gram = timed(lambda: H.himuon_gram_ns(mats, K, workloads.COEFFS, restart=restart, workspace=gws,
                                             workspace_bytes=gbytes, stream=stream))
    ms_std = timed(lambda: H.himuon_tiled_ns(mats, Tf, K, workloads.COEFFS, workspace=sws,
                                             workspace_bytes=sbytes, stream=stream))
    alg_std = algorithmic_flops(shapes, Tf, K)
    alg_gram = gram_flops(shapes, K, restart)
    eff = alg_std / (ms_gram * 1e-3) / 1e12
    own = alg_gram / (ms_gram * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    res = {
        "metric": "full-matrix NS through the Gram iteration, standard-map TFLOP/s (2 r^2 (2s + r) K per matrix)",
        "value": round(eff, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_gram, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded normal entries, transformer-layer shapes)",
        "config": {"workload": w.name + " full-matrix map, Gram iteration", "matrices": len(shapes), "K": K,
                   "restart": restart, "workspace_bytes": gbytes, "parallelism": "single GPU"},
        "standard_full_map_ms": round(ms_std, 5),
        "speedup_vs_standard": round(ms_std / ms_gram, 3),
        "flop_ratio_gram_over_standard": round(alg_gram / alg_std, 4),
        "roofline": {"bound": "mfma", "achieved": round(own, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(own / peak, 4), "traffic": None,
                     "kernel": "whole call (step GEMMs of the Gram iteration)", "launch_ms": round(ms_gram, 5)},
    }
    if not no_cpu:
        from oracle.gram_ns import gram_ns
        i = max(range(len(shapes)), key=lambda k: min(shapes[k]) * max(shapes[k]))
        h, w_ = shapes[i]
        if min(h, w_) > 2048:
            # a 2048-row (or -column) crop with the matrix's aspect ratio keeps
            # the sample to seconds
            f = 2048.0 / min(h, w_)
            h, w_ = int(round(h * f)), int(round(w_ * f))
        x = mats[i][:h, :w_].cpu().to(torch.float64).numpy()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0 or n == 0:
            gram_ns(x, [workloads.COEFFS] * K, restart=restart)
            n += 1
        dt = (time.perf_counter() - t0) / n
        try:
            from threadpoolctl import threadpool_info
            threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
        except Exception:
            threads = os.cpu_count() or 1
        res["cpu_baseline"] = {"value": round(algorithmic_flops([(h, w_)], max(h, w_), K) / dt / 1e12, 5),
                               "unit": "TFLOP/s (standard-map count)", "cores": threads, "kind": "oracle",
                               "sample": f"oracle gram_ns on the leading {h}x{w_} block of matrix {i} "
                                         f"{shapes[i]}, {n} calls"}
    return res


def w_coeffs():
    import workloads
    return workloads.COEFFS


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up until at least this long has passed (and --warmup steps have run)")
    ap.add_argument("--workload", default="layers24_d2048")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--K", type=int, default=5)
    ap.add_argument("--cap", type=int, default=None, help="workspace cap in bytes")
    ap.add_argument("--schedule", default=None,
                    help="per-step tile sizes, e.g. 512,256,128,128,128 (non-increasing, nested); "
                         "replaces --T and --K")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--pair-stats", action="store_true",
                    help="time the pair statistics (tiled-versus-full diagnostics) instead of the map")
    ap.add_argument("--gram", action="store_true",
                    help="time the full-matrix map through the Gram iteration (himuon_gram_ns) against the "
                         "standard full map instead of the tiled map")
    ap.add_argument("--restart", type=int, default=2, help="Gram iteration restart point (0: none)")
    ap.add_argument("--muon", action="store_true",
                    help="time the fused Muon step (himuon_muon_step) on the workload instead of the map")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 5 times (used to "
                         "calibrate the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the tiled map has no "
              "exchange between GPUs, so one GPU's share is what is measured", file=sys.stderr)
        sys.exit(2)

    # the CPU oracle first, before anything touches the GPU
    cpu = None
    if not (args.no_cpu or args.schedule or args.pair_stats or args.gram or args.muon or args.copy_mib):
        import workloads
        wl = workloads.WORKLOADS[args.workload]
        cpu = cpu_baseline(wl, args.T or wl.T, args.K)

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
    if args.pair_stats:
        print(json.dumps(pair_stats_bench(H, torch, w, mats, args.steps, args.warmup, args.no_cpu)), flush=True)
        return
    cap = args.cap if args.cap is not None else w.workspace_cap
    if args.gram:
        print(json.dumps(gram_bench(H, torch, w, mats, args.K, args.restart, args.steps, args.warmup, cap,
                                    args.no_cpu)), flush=True)
        return
    if args.muon:
        print(json.dumps(muon_bench(H, torch, w, mats, T, K, args.steps, args.warmup, args.warmup_seconds, cap)),
              flush=True)
        return
    full, mn = H.himuon_workspace_size(mats, T)
    ws = None
    ws_bytes = 0
    if full:
        ws_bytes = min(full, cap) if cap else full
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    plan = H.himuon_plan(mats, T, K, H.BF16 if w.dtype == "bf16" else H.FP32, ws_bytes)
    stream = torch.cuda.current_stream()

    sched = [int(x) for x in args.schedule.split(",")] if args.schedule else None
    if sched:
        T, K = sched[0], len(sched)
        need = max(H.himuon_workspace_size(mats, t)[0] for t in set(sched))
        ws_bytes = min(need, cap) if cap else need
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
        plan = H.himuon_plan(mats, sched[-1], 0, H.BF16 if w.dtype == "bf16" else H.FP32, ws_bytes)

    def step():
        if sched:
            H.himuon_tiled_ns_schedule(mats, sched, workloads.COEFFS, workspace=ws, workspace_bytes=ws_bytes,
                                       stream=stream)
        else:
            H.himuon_tiled_ns(mats, T, K, workloads.COEFFS, workspace=ws, workspace_bytes=ws_bytes, stream=stream)

    # warm-up: at least --warmup steps and at least --warmup-seconds, so that
    # a short --warmup still times the steady state (clocks up, code loaded)
    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t0 < args.warmup_seconds:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
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

    if sched:
        nominal = sum(6.0 * h * ww * t for h, ww in shapes for t in sched)
        alg = sum(algorithmic_flops(shapes, t, 1) for t in sched)
    else:
        nominal = sum(6.0 * h * ww * T * K for h, ww in shapes)
        alg = algorithmic_flops(shapes, T, K)
    tflops = nominal / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    if sched:
        roof = {"bound": "mfma", "achieved": round(alg / (ms_per_step * 1e-3) / 1e12, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(alg / (ms_per_step * 1e-3) / 1e12 / peak, 4), "traffic": None,
                "kernel": "whole schedule", "tiles": None, "launch_ms": round(ms_per_step, 5)}
    else:
        roof = dominant_kernel_roofline(H, torch, mats, shapes, T, K, plan, stream, ms_per_step, alg, peak,
                                        w, args.steps)
    io_bytes = 2.0 * sum(h * ww for h, ww in shapes) * (2 if w.dtype == "bf16" else 4)
    out = {
        "metric": METRIC,
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
        "data": "synthetic (seeded normal entries, transformer-layer shapes)",
        "config": {"workload": w.name, "matrices": len(shapes), "T": sched if sched else T, "K": K,
                   "elements": sum(h * ww for h, ww in shapes), "launches_per_step": plan["launches"],
                   "tiles": plan["tiles"], "tail_tiles": plan["tail_tiles"], "chunks": plan["chunks"],
                   "workspace_bytes": ws_bytes, "parallelism": "single GPU"},
        "matrices_per_s": round(len(shapes) / (ms_per_step * 1e-3), 1),
        # from the algorithmic count, which equals 6 H W T K for full tiles and
        # stays meaningful for ragged tiles and T above the matrix size
        "pct_bf16_peak": round(100.0 * alg / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "algorithmic_tflops": round(alg / (ms_per_step * 1e-3) / 1e12, 3),
        "hbm_gbs_io": round(io_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "roofline": roof,
        "warmup_steps_run": n_warm,
        "context": CONTEXT,
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
