"""Benchmark: 3x3x3 submanifold convolution, neighbour-cache build + forward + both backward passes, one GPU.

One step runs the whole path over one resident batch: build_neighbor_map
(hash insert, probes, mask/z-order sort, pair lists), the forward masked
implicit GEMM, the input-gradient GEMM and the Split-K weight gradient with
dbias.  The headline value is effective TFLOP/s counting valid-neighbour MACs
only (3 passes x 2 P Ci Co flops per step); voxels/s is reported beside it,
and so are the three passes on a built plan alone and the plan build alone
(medians and minima over at least 20 event-timed repetitions).

The default workload is the C = 1024 one (1 x 128^3 grid, every cell active
with p = 0.3, bf16): the largest by valid work.  The roofline object covers
the dominant kernel (the masked implicit GEMM, timed on the input-gradient
call, which enqueues nothing but its launches) against the dense bf16 MFMA
peak, or, when a workload's arithmetic intensity sits below the ridge,
against HBM bandwidth with algorithmic bytes.  The oracle (CPU, float64) is
timed on the host on a bounded sample of the same workload as a reported
baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (valid MACs) + voxels/s, subm conv3d fwd+bwd, 1 MI355X"
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0}
DEFAULT_CONFIG = 5


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=DEFAULT_CONFIG, choices=[1, 2, 3, 4, 5])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="time eagerly launched steps instead of replaying one captured HIP graph per step")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--phase-reps", type=int, default=20,
                   help="event-timed repetitions of each call (median and min); profiling runs cut this down")
    p.add_argument("--copy-calib", type=int, default=0,
                   help="only run a device copy of this many MiB (HBM counter calibration)")
    p.add_argument("--serialize", action="store_true",
                   help="only time encode_seq + decode_seq (z-order and Hilbert) on the workload's "
                        "coordinates; prints its own JSON line")
    p.add_argument("--sparse-conv", action="store_true",
                   help="only time the strided sparse convolution (output sites, map build, fwd, dgrad, wgrad) "
                        "over the workload's voxels; prints its own JSON line")
    p.add_argument("--ks", type=int, default=2, help="--sparse-conv kernel side")
    p.add_argument("--stride", type=int, default=2, help="--sparse-conv stride")
    p.add_argument("--pad", type=int, default=0, help="--sparse-conv padding")
    p.add_argument("--grid-sample", action="store_true",
                   help="only time sparse grid sampling (fwd + feature gradient) at one point per voxel of "
                        "the workload; prints its own JSON line")
    return p.parse_args()


# the sources the masked implicit GEMM's work depends on: its translation unit, the plan builder that
# orders its rows, and the headers they include
GEMM_SOURCES = ("sparse_submanifold_convolution_amd/csrc/conv.hip", "sparse_submanifold_convolution_amd/csrc/ssc_internal.h",
                "sparse_submanifold_convolution_amd/csrc/plan.hip", "include/ssc.h")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(os.path.basename(rel).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per call (all launches of one call) from the committed counter summary, if it matches the
    current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}|{workload}")
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_call")


def measured_counters(kernel: str, workload: str):
    """MFMA counters of the kernel's launches (profiles/counters.json), if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}|{workload}")
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec


def copy_calibration(mib: int) -> None:
    import torch
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "launches": 5, "bytes_read_per_launch": mib << 20,
                      "bytes_written_per_launch": mib << 20}), flush=True)


def host_cpu() -> dict:
    """CPU model, the cores this process may run on and the BLAS thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    blas_threads = cores
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        if blas:
            blas_threads = int(blas[0]["num_threads"])
    except Exception:  # threadpoolctl missing: BLAS uses the affinity set
        pass
    return {"cpu_model": model, "cores": cores, "blas_threads": blas_threads}


def _oracle_step(O, coords, shape, X, W, b, dY) -> dict:
    """One pass of the oracle over a voxel set: map, permutation, fwd, dgrad, wgrad + dbias (seconds)."""
    t = {}
    t0 = time.perf_counter()
    nm = O.neighbor_map(coords, shape)
    t["nmap"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.sort_perm(coords, nm, shape)
    t["perm"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.fwd(X, W, b, nm)
    t["fwd"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.dgrad(dY, W, nm)
    t["dgrad"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.wgrad(X, dY, nm)
    O.dbias(dY)
    t["wgrad"] = time.perf_counter() - t0
    t["pairs"] = int((nm != O.SENTINEL).sum())
    return t


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle as it stands (float64, numpy + BLAS), timed on the host on a bounded sample.

    The sample is the workload's own voxels in the slab x < t of every batch entry (a whole
    sub-problem of the same distribution: map, sort and all three passes over those voxels, with
    the same rounded values).  A thin slab is timed first; the slab is then widened so that one
    pass of the oracle takes about `budget_s` (the whole workload when it fits), and that pass is
    the reported figure, in the metric's unit (valid-MAC TFLOP/s of the sample).
    """
    import numpy as np
    import torch
    from oracle import subm as O
    X_dim = int(w.shape[1])
    x = w.coords[:, 1]

    def slab(t):
        sel = np.nonzero(x < t)[0]
        idx = torch.from_numpy(sel)
        return (np.ascontiguousarray(w.coords[sel]), w.feats.index_select(0, idx), w.dout.index_select(0, idx),
                int(sel.size))

    t0 = max(1, X_dim // 64)
    c, Xs, dYs, n0 = slab(t0)
    first = _oracle_step(O, c, w.shape, Xs, w.weight, w.bias, dYs)
    sec0 = sum(v for k, v in first.items() if k != "pairs")
    t1 = X_dim if sec0 <= 0 else int(min(X_dim, max(t0, t0 * budget_s / sec0)))
    if t1 > t0:
        c, Xs, dYs, n1 = slab(t1)
        res = _oracle_step(O, c, w.shape, Xs, w.weight, w.bias, dYs)
    else:
        t1, n1, res = t0, n0, first
    sec = sum(v for k, v in res.items() if k != "pairs")
    flops = 3 * 2.0 * res["pairs"] * w.ci * w.co
    whole = t1 >= X_dim
    host = host_cpu()
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": ("whole workload" if whole else f"slab x < {t1} of {X_dim} in every batch entry")
                      + f": {n1} of {w.n} voxels, {res['pairs']} valid pairs; neighbour map, permutation, "
                        f"fwd, dgrad, wgrad + dbias, one pass, float64 numpy/BLAS",
            "cpu_model": host["cpu_model"], "affinity_cores": host["cores"],
            "seconds_per_sample_step": sec, "voxels_per_s": n1 / sec,
            "stage_seconds": {k: v for k, v in res.items() if k != "pairs"}}


def serialize_bench(args) -> None:
    """encode_seq + decode_seq in both modes on the workload's coordinates, inputs resident in HBM.

    Each measured sequence is captured once in a HIP graph and replayed, so host-side
    marshalling stays out of the timed region.
    """
    import torch
    import sparse_submanifold_convolution_amd as ssc
    from sparse_submanifold_convolution_amd import workloads as WL

    dev = torch.device("cuda:0")
    w = WL.make_workload(args.config)
    coords = torch.from_numpy(w.coords).to(dev)
    width = ssc.seq_code_width(w.shape)
    reps = 20
    side = torch.cuda.Stream(dev)

    def timed(fn):
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()  # warm the allocator outside capture
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        best = 1e30
        for _ in range(args.steps):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / reps)
        return best

    per, results = {}, {}
    for mode in ("z_order", "hilbert"):
        codes = ssc.encode_seq(coords, w.shape, mode)
        results[mode] = ssc.decode_seq(codes, w.shape, mode)
        per[f"{mode}_encode"] = timed(lambda m=mode: ssc.encode_seq(coords, w.shape, m))
        per[f"{mode}_decode"] = timed(lambda m=mode, c=codes: ssc.decode_seq(c, w.shape, m))
    torch.cuda.synchronize()
    ok = all(torch.equal(v, coords) for v in results.values())
    ms = sum(per.values())
    # algorithmic bytes per launch: 16-byte rows in and a 4- or 8-byte code out (or the reverse)
    bytes_per_launch = w.n * (16 + width // 8)
    dom = max(per, key=per.get)
    ach = bytes_per_launch / (per[dom] * 1e-3) / 1e9
    print(json.dumps({
        "metric": "voxels/s, encode_seq + decode_seq (z-order and Hilbert), 1 MI355X",
        "value": 4 * w.n / (ms * 1e-3), "unit": "voxels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"int{width}", "data": "synthetic",
        "config": {"workload": f"config {args.config}: {w.desc}", "voxels": w.n, "code_width": width,
                   "step": "encode + decode, z-order and Hilbert (four launches)",
                   "launch": f"graph of {reps} calls per launch kind, best replay",
                   "parallelism": "single GPU"},
        "per_call_ms": per, "round_trip_exact": ok,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": None, "kernel": f"seq_{dom}",
                     "avg_launch_ms": per[dom], "alg_bytes_per_launch": bytes_per_launch},
    }), flush=True)


def grid_sample_bench(args) -> None:
    """Sparse trilinear grid sampling, forward + feature gradient, inputs resident in HBM.

    Points: one per voxel of the workload, 90 % within a cell of an active voxel and 10 % anywhere
    in the box; dout ~ N(0, 1).  Each pass is captured in a HIP graph of `reps` calls and replayed.
    """
    import numpy as np
    import torch
    import sparse_submanifold_convolution_amd as ssc
    from sparse_submanifold_convolution_amd import workloads as WL

    dev = torch.device("cuda:0")
    w = WL.make_workload(args.config)
    m = w.n
    pts_np = WL.sample_points(w.coords, w.shape, m, args.config)
    plan = ssc.build_neighbor_map(torch.from_numpy(w.coords).to(dev), w.shape, key_bits=w.key_bits)
    F = w.feats.to(dev)
    P = torch.from_numpy(pts_np).to(dev)
    dout = WL.normal(np.random.default_rng(1000 + args.config), (m, w.ci), w.dtype).to(dev)
    out = torch.empty((m, w.ci), dtype=F.dtype, device=dev)
    dF = torch.empty_like(F)
    ws = torch.empty(ssc.grid_sample_workspace_bytes(w.n, m), dtype=torch.uint8, device=dev)
    reps = 10
    side = torch.cuda.Stream(dev)

    def timed(fn):
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        best = 1e30
        for _ in range(args.steps):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / reps)
        return best

    t_fwd = timed(lambda: ssc.grid_sample_fwd(plan, F, P, out=out))
    t_bwd = timed(lambda: ssc.grid_sample_bwd(plan, P, dout, dfeats=dF, ws=ws))
    ms = t_fwd + t_bwd
    s = F.element_size()
    slot = 16 if plan_key_width(w) == 64 else 8
    # gs_fwd, algorithmic bytes per launch: the points, the output rows, every voxel row once and
    # one hash slot per corner lookup
    fwd_bytes = m * 16 + s * w.ci * m + s * w.ci * w.n + 8 * slot * m
    ach = fwd_bytes / (t_fwd * 1e-3) / 1e9
    res = {
        "metric": "points/s, sparse trilinear grid_sample fwd + feature gradient, 1 MI355X",
        "value": m / (ms * 1e-3), "unit": "points/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"config {args.config} voxels: {w.desc}; one point per voxel",
                   "voxels": w.n, "points": m, "channels": w.ci,
                   "launch": f"graph of {reps} calls per pass, best replay", "parallelism": "single GPU"},
        "per_pass_ms": {"fwd": t_fwd, "bwd": t_bwd},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": None, "kernel": "gs_fwd",
                     "avg_launch_ms": t_fwd, "alg_bytes_per_launch": fwd_bytes},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = grid_sample_cpu_baseline(w, pts_np, dout.cpu(), args.cpu_budget_s)
    print(json.dumps(res), flush=True)


def sparse_conv_bench(args) -> None:
    """Strided sparse convolution over a workload's voxel set, inputs resident in HBM.

    Phases: output sites (count, host read, emit), map build, forward, input gradient, weight
    gradient + dbias.  The map build and each pass are captured in a HIP graph of `reps` calls and
    replayed; the output sites include the count's host read.  Values are seeded (strided_values).
    """
    import numpy as np
    import torch
    import sparse_submanifold_convolution_amd as ssc
    from sparse_submanifold_convolution_amd import workloads as WL

    dev = torch.device("cuda:0")
    L = ssc.lib()
    P_ = ssc.binding._ptr
    w = WL.make_workload(args.config, values=False)
    ks, st, pd = args.ks, args.stride, args.pad
    coords = torch.from_numpy(w.coords).to(dev)
    print(f"[bench] strided conv on workload {args.config} ({w.n} voxels), ks={ks} s={st} p={pd}",
          file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_sites = 1e30
    for _ in range(max(3, args.steps // 4)):
        torch.cuda.synchronize()
        e0.record()
        oc = ssc.sparse_out_coords(coords, w.shape, ks, st, pd)
        e1.record()
        torch.cuda.synchronize()
        best_sites = min(best_sites, e0.elapsed_time(e1))
    plan = ssc.build_sparse_map(coords, w.shape, ks, st, pd, out_coords=oc, key_bits=w.key_bits)
    n_in, n_out, V, C = plan.n_in, plan.n_out, ks ** 3, w.ci
    P = int((plan.nmap != -1).sum())
    X, W, b, dY = (t.to(dev) for t in WL.strided_values(1000 + args.config, n_in, n_out, ks, C, C, w.dtype))
    out = torch.empty((n_out, C), dtype=X.dtype, device=dev)
    dX = torch.empty((n_in, C), dtype=X.dtype, device=dev)
    dW = torch.empty((V, C, C), dtype=X.dtype, device=dev)
    db = torch.empty((C,), dtype=X.dtype, device=dev)
    ws = ssc.sparse_workspace(plan, C, C, X.dtype)
    B_, Xd, Yd, Zd = w.shape

    def build():
        r = L.ssc_build_sparse_map(P_(coords), n_in, B_, Xd, Yd, Zd, P_(oc), n_out, ks, st, pd, w.key_bits,
                                   P_(plan.nmap), P_(plan.perm), P_(plan.buf), plan.buf.numel(),
                                   ssc.binding._stream(dev))
        if r:
            raise ssc.SSCError("ssc_build_sparse_map", r)

    reps = 10
    side = torch.cuda.Stream(dev)

    def timed(fn):
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = 1e30
        for _ in range(args.steps):
            a.record()
            g.replay()
            c.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(c) / reps)
        return best

    per = {
        "map_build": timed(build),
        "fwd": timed(lambda: ssc.sparse_conv3d_fwd(plan, X, W, b, out=out, ws=ws)),
        "dgrad": timed(lambda: ssc.sparse_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(dX, None, None))),
        "wgrad": timed(lambda: ssc.sparse_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(None, dW, db))),
    }
    conv_ms = per["fwd"] + per["dgrad"] + per["wgrad"]
    flops_pass = 2.0 * P * C * C
    s = X.element_size()
    # input-gradient GEMM: one index per valid pair, each dY row read once, each dX row written once, W
    alg_bytes = 4.0 * P + s * (n_out * C + n_in * C) + s * V * C * C
    ai = flops_pass / alg_bytes
    peak_f = PEAK_TFLOPS[w.dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    t_k = per["dgrad"] * 1e-3
    if ai >= ridge:
        ach = flops_pass / t_k / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak_f, "unit": "TFLOP/s", "frac": ach / peak_f}
    else:
        ach = alg_bytes / t_k / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    roof.update({"traffic": None, "kernel": "igemm (input-gradient launch, transposed map)",
                 "avg_launch_ms": per["dgrad"], "flops_per_launch": flops_pass, "alg_bytes_per_launch": alg_bytes,
                 "arith_intensity": ai, "ridge": ridge})
    res = {
        "metric": "effective TFLOP/s (valid MACs), strided sparse conv3d fwd+bwd, 1 MI355X",
        "value": 3 * flops_pass / (conv_ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": conv_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"config {args.config} voxels: {w.desc}; strided conv ks={ks} stride={st} pad={pd}",
                   "in_voxels": n_in, "out_voxels": n_out, "valid_pairs": P, "ci": C, "co": C,
                   "step": "fwd + dgrad + wgrad + dbias on a built map",
                   "launch": f"graph of {reps} calls per phase, best replay", "parallelism": "single GPU"},
        "out_voxels_per_s": n_out / (conv_ms * 1e-3),
        "plan_ms": {"out_sites_incl_host_read": best_sites, "map_build": per["map_build"]},
        "per_pass_ms": {k: per[k] for k in ("fwd", "dgrad", "wgrad")},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = sparse_conv_cpu_baseline(w, ks, st, pd, X.cpu(), W.cpu(), b.cpu(), dY.cpu(),
                                                       args.cpu_budget_s)
    print(json.dumps(res), flush=True)


def sparse_conv_cpu_baseline(w, ks, st, pd, X, W, b, dY, budget_s: float) -> dict:
    """The strided-conv oracle (float64 numpy + BLAS) on the whole workload, on the host."""
    from oracle import sparse_conv as SC
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        cores = int(blas[0]["num_threads"]) if blas else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    reps, t_total, flops = 0, 0.0, 0.0
    while reps == 0 or (t_total < budget_s / 2 and reps < 3):
        t0 = time.perf_counter()
        oc = SC.out_coords(w.coords, w.shape, ks, st, pd)
        nm = SC.neighbor_map(w.coords, w.shape, oc, ks, st, pd)
        SC.fwd(X, W, b, nm)
        SC.dgrad(dY, W, nm, len(w.coords))
        SC.wgrad(X, dY, nm, ks ** 3)
        SC.dbias(dY)
        t_total += time.perf_counter() - t0
        reps += 1
        flops = 3 * 2.0 * int((nm != SC.SENTINEL).sum()) * w.ci * w.ci
    sec = t_total / reps
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"whole workload ({len(w.coords)} input voxels: output sites, map and the three passes), "
                      f"{reps} repetition(s), float64 numpy/BLAS", "seconds_per_step": sec}


def plan_key_width(w) -> int:
    """Key width the plan of workload w uses (the build's rule: 32 bits when the grid volume fits)."""
    if w.key_bits:
        return w.key_bits
    B, X, Y, Z = w.shape
    return 32 if B * X * Y * Z <= 0xFFFFFFFF else 64


def grid_sample_cpu_baseline(w, pts, dout, budget_s: float) -> dict:
    """The grid-sampling oracle (float64 numpy) on a bounded sample of the points, whole voxel set."""
    from oracle import grid_sample as G
    k = min(len(pts), 200000)
    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < budget_s / 2 and reps < 3):
        t0 = time.perf_counter()
        G.sample_fwd(w.coords, w.feats, w.shape, pts[:k])
        G.sample_bwd(w.coords, w.shape, pts[:k], dout[:k])
        t_total += time.perf_counter() - t0
        reps += 1
    sec = t_total / reps
    return {"value": k / sec, "unit": "points/s", "cores": 1, "kind": "oracle",
            "sample": f"first {k} of {len(pts)} points against all {w.n} voxels, fwd + bwd, "
                      f"{reps} repetition(s), float64 numpy"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(the design for sharding is described in DESIGN.md). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return
    if args.serialize:
        serialize_bench(args)
        return
    if args.grid_sample:
        grid_sample_bench(args)
        return
    if args.sparse_conv:
        sparse_conv_bench(args)
        return

    import numpy as np
    import torch
    import sparse_submanifold_convolution_amd as ssc
    from sparse_submanifold_convolution_amd import workloads as WL

    dev = torch.device("cuda:0")
    ssc.lib()
    w = WL.make_workload(args.config)
    print(f"[bench] workload {args.config}: {w.desc}, n={w.n}", file=sys.stderr, flush=True)
    coords = torch.from_numpy(w.coords).to(dev)
    X, W, b, dY = (t.to(dev) for t in (w.feats, w.weight, w.bias, w.dout))
    n, ci, co = w.n, w.ci, w.co

    # buffers allocated once; a step only enqueues kernels
    B_, Xd, Yd, Zd = w.shape
    pbytes = ssc.plan_bytes(n, w.shape, w.key_bits)
    plan = ssc.Plan(torch.empty((n, 27), dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int32, device=dev),
                    torch.empty(pbytes, dtype=torch.uint8, device=dev), n, tuple(w.shape), w.key_bits)
    ws = ssc.workspace(plan, ci, co, X.dtype)
    out = torch.empty((n, co), dtype=X.dtype, device=dev)
    dX = torch.empty((n, ci), dtype=X.dtype, device=dev)
    dW = torch.empty((27, ci, co), dtype=X.dtype, device=dev)
    db = torch.empty((co,), dtype=X.dtype, device=dev)
    L = ssc.lib()
    stream = torch.cuda.current_stream(dev)
    P_ = ssc.binding._ptr

    def build():
        # the current stream: the capturing stream while a graph is recorded
        r = L.ssc_build_neighbor_map(P_(coords), n, B_, Xd, Yd, Zd, w.key_bits, P_(plan.nmap), P_(plan.perm),
                                     P_(plan.buf), pbytes, ssc.binding._stream(dev))
        if r:
            raise ssc.SSCError("ssc_build_neighbor_map", r)

    def fwd():
        ssc.subm_conv3d_fwd(plan, X, W, b, out=out, ws=ws)

    def dgrad():
        ssc.subm_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(dX, None, None))

    def wgrad():
        ssc.subm_conv3d_bwd(plan, X, W, dY, ws=ws, outs=(None, dW, db))

    parts = [("plan", build), ("fwd", fwd), ("dgrad", dgrad), ("wgrad", wgrad)]
    build()
    st = ssc.plan_status(plan)
    if st:
        raise ssc.SSCError("plan", st)
    counts = ssc.plan_pair_counts(plan)
    P = sum(counts)
    flops_pass = 2.0 * P * ci * co
    orders, union_rows, mask_bits = ssc.plan_row_orders(plan)

    def step():
        for _, f in parts:
            f()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-call times of eagerly launched steps: HIP events on the stream the kernels run on
    # (torch's current stream, which the binding hands to every call), at least 20 repetitions
    reps = max(1, args.phase_reps)
    ev = {k: [] for k, _ in parts}
    for _ in range(reps):
        for name, f in parts:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    per = {k: [a.elapsed_time(c) for a, c in v] for k, v in ev.items()}
    med = {k: float(np.median(v)) for k, v in per.items()}
    mins = {k: float(np.min(v)) for k, v in per.items()}

    # the timed region: exactly K whole steps (plan build + fwd + dgrad + wgrad), synchronised on both sides
    if args.no_graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        mode = "eager launches"
    else:
        # the whole step captured once and replayed
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        mode = "one captured HIP graph per step"

    value = 3 * flops_pass / (ms_step * 1e-3) / 1e12
    conv_ms = med["fwd"] + med["dgrad"] + med["wgrad"]
    esize = X.element_size()
    # dominant kernel: the masked implicit GEMM, timed on the input-gradient call, which enqueues
    # nothing but its launches; one call = one pass of valid work
    kernel = "igemm"
    alg_bytes = 4.0 * P + esize * n * (ci + co) + esize * 27 * ci * co
    ai = flops_pass / alg_bytes
    peak_f = PEAK_TFLOPS[w.dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    t_k = med["dgrad"] * 1e-3
    wl_name = f"cfg{args.config}"
    traffic = measured_traffic(kernel, wl_name)
    if ai >= ridge:
        ach = flops_pass / t_k / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak_f, "unit": "TFLOP/s", "frac": ach / peak_f,
                "traffic": traffic}
    else:
        ach = alg_bytes / t_k / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": traffic}
    roof.update({"kernel": f"{kernel} (masked implicit GEMM, the input-gradient call's launches)",
                 "call_ms_median": med["dgrad"], "call_ms_min": mins["dgrad"],
                 "flops_per_call": flops_pass, "alg_bytes_per_call": alg_bytes,
                 "arith_intensity": ai, "ridge": ridge})
    ctr = measured_counters(kernel, wl_name)

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"config {args.config}: {w.desc}", "voxels": n, "valid_pairs": P, "ci": ci, "co": co,
                   "key_bits": w.key_bits or 32, "step": "neighbour-cache build + fwd + dgrad + wgrad + dbias",
                   "launch": mode, "parallelism": "single GPU", "gemm_row_orders": orders},
        "voxels_per_s": n / (ms_step * 1e-3),
        # the three convolution passes on a built plan, and the plan build on its own (medians)
        "conv_only": {"ms": conv_ms, "tflops": 3 * flops_pass / (conv_ms * 1e-3) / 1e12,
                      "voxels_per_s": n / (conv_ms * 1e-3), "frac_of_peak": 3 * flops_pass / (conv_ms * 1e-3)
                      / 1e12 / peak_f},
        "plan_build_ms": {"median": med["plan"], "min": mins["plan"]},
        "phase_ms": {"median": med, "min": mins, "repetitions": reps,
                     "timing": "HIP events around each call of eagerly launched steps"},
        "executed_over_valid": None if ctr is None else ctr.get("executed_over_valid"),
        # rows multiplied by a single (mask, z-order) order's 32-row waves per valid pair, as the build counted
        # them (only counted where the build considers a second order)
        "single_order_rows_over_valid": (union_rows / mask_bits) if mask_bits else None,
        "mfma_busy": None if ctr is None else ctr.get("mfma_busy"),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget_s)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
