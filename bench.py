"""Benchmark: mixed-precision Tile-CSC CG on one MI355X.

Workload: 3D 7-point Laplacian on a 128^3 grid (n = 2,097,152,
nnz = 14,581,760), 16x16 tiles, a seeded static per-tile map with 50 % FP64,
30 % FP32 and 20 % BF16 tiles, b = A x* with x* ~ U[-1, 1], x0 = 0, stopping
at ||r_k||/||r_0|| <= 1e-8. One step is one complete cg_solve (every
iteration: SpMV with fused p.q, the x/r update with fused reductions, the
direction update, the device stop flag), with b already resident on the GPU.

Prints one JSON line: CG iterations/s over the timed solves, time to
solution, the Tile-CSC SpMV bandwidth against the 8 TB/s HBM roofline, the
all-FP64-map time to solution for comparison, and the CPU oracle's rate on a
bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
COPY_BYTES = 256 << 20
METRIC = "Tile-CSC SpMV GB/s (% HBM peak); CG iterations/sec; time-to-solution"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spmv_tilecsc_cfg2_traffic.json")
KERNEL_SOURCES = ["mixed_precision_sparse_amd/csrc/mpcg_kernels.hpp",
                  "mixed_precision_sparse_amd/csrc/mpcg_runtime.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def spmv_algorithmic_bytes(L, prec_map) -> int:
    """Bytes one Tile-CSC SpMV must move: values in their stored width, one byte each
    for the local row and column, 9 B per tile (column block i32, nnz offset i32,
    map u8), the row-block pointers, x read once and y written once."""
    nnz_t = np.diff(L.tile_nnz_ptr)
    width = np.array([8, 4, 2], dtype=np.int64)[prec_map]
    nrb = -(-L.n // L.R)
    return int((nnz_t * width).sum() + 2 * L.nnz + 9 * L.T + 4 * (nrb + 1) + 16 * L.n)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--spmv-reps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile-shapes", default="",
                    help="comma-separated workloads (e.g. 2,3,4): instead of the CG bench, time cg_spmv "
                         "(FP64 map) at the workload's tile shape and at the tuned row-block heights "
                         "(paper Sec. 3.3.3) for C = 64 and the workload's C; prints one JSON line")
    ap.add_argument("--workloads", default="",
                    help="comma-separated workloads (e.g. 1,2,3,4,5): instead of the CG bench, report per "
                         "workload the warm time to solution under the all-FP64 map and under the "
                         "workload's own map, CG iterations/s, true residuals and SpMV GB/s with their "
                         "roofline fractions; prints one JSON line")
    ap.add_argument("--col-slices", default="",
                    help="with --workloads or --spmv-probe: comma-separated column-slice counts (e.g. 8,16) whose handles "
                         "are timed beside the unsliced ones")
    ap.add_argument("--small-systems", action="store_true",
                    help="instead of the CG bench, time CG (FP64 map, tol 1e-10) on 2D 5-point and 3D "
                         "7-point Laplacians of a few hundred to a few thousand rows, on one workgroup "
                         "(single_block=1) and with three launches per iteration (single_block=-1); "
                         "prints one JSON line")
    ap.add_argument("--spmv-probe", default="",
                    help="counter run on comma-separated workloads (e.g. 4,5): a 256 MiB copy (the scale "
                         "reference), then per workload 5 cg_spmv launches under the all-FP64 map on the "
                         "unsliced handle and on one per --col-slices count; no timing")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="counter run: a 256 MiB copy (the scale reference), then 5 cg_spmv "
                         "launches per map (all FP64, the bench's mixed map, all BF16); no timing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_precision_sparse_amd as mpcg
    from gen import make_workload, static_map, tile_scores

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.tile_shapes:
        tile_shapes(torch, dev, mpcg, [int(c) for c in args.tile_shapes.split(",")], args.spmv_reps)
        return
    if args.small_systems:
        small_systems(torch, dev, mpcg)
        return
    if args.spmv_probe:
        spmv_probe(torch, dev, mpcg, [int(c) for c in args.spmv_probe.split(",")],
                   [int(c) for c in args.col_slices.split(",") if c])
        return
    if args.workloads:
        all_workloads(torch, dev, mpcg, [int(c) for c in args.workloads.split(",")], args.spmv_reps,
                      [int(c) for c in args.col_slices.split(",") if c])
        return
    t0 = time.time()
    w = make_workload(2, "full")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    pmap = static_map(tile_scores(L.T, 2), w.map_spec["frac_bf16"], w.map_spec["frac_fp32"])
    S = mpcg.Solver(L, pmap)
    setup_s = time.time() - t0
    print(f"# setup {setup_s:.1f}s: n={A.n} nnz={A.nnz} T={L.T} map counts "
          f"{np.bincount(pmap, minlength=3).tolist()}", file=sys.stderr, flush=True)

    b = torch.from_numpy(w.b).to(dev)
    x = torch.zeros_like(b)

    if args.pmc_probe:
        pmc_probe(torch, dev, S, L, A, pmap, b, w, mpcg)
        return

    def run_solves(solver, steps):
        its = 0
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            status, K, hist = solver.cg_solve(b, x, w.tol, w.maxit)
            its += K
        torch.cuda.synchronize()
        return time.perf_counter() - t, its, status, K, hist

    run_solves(S, args.warmup)
    el, its, status, K, hist = run_solves(S, args.steps)
    tts_ms = 1e3 * el / args.steps
    iters_per_s = its / el
    xs = x.cpu().numpy()
    true_res = float(np.linalg.norm(w.b - A.to_scipy() @ xs) / np.linalg.norm(w.b))
    print(f"# mixed map: {status} K={K} TTS {tts_ms:.3f} ms, {iters_per_s:.1f} it/s, "
          f"true residual {true_res:.3e}", file=sys.stderr, flush=True)

    # Tile-CSC SpMV on its own: average launch time from HIP events on the launch stream.
    y = torch.empty_like(b)
    xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
    for _ in range(10):
        S.cg_spmv(xin, y)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.spmv_reps):
        S.cg_spmv(xin, y)
    e1.record()
    torch.cuda.synchronize()
    spmv_ms = e0.elapsed_time(e1) / args.spmv_reps
    bytes_spmv = spmv_algorithmic_bytes(L, pmap)
    spmv_gbs = bytes_spmv / (spmv_ms * 1e-3) / 1e9
    bytes_spmv64 = spmv_algorithmic_bytes(L, np.zeros(L.T, np.uint8))
    bytes_vec = 56 * A.n
    iter_gbs = (bytes_spmv + bytes_vec) * its / el / 1e9

    # Measured bandwidth ceiling: a device-to-device copy of 256 MiB.
    c_src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    c_dst = torch.empty_like(c_src)
    for _ in range(3):
        c_dst.copy_(c_src)
    e0.record()
    for _ in range(20):
        c_dst.copy_(c_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    del c_src, c_dst

    # The all-FP64 map on the same substrate.
    S64 = mpcg.Solver(L, np.zeros(L.T, np.uint8))
    run_solves(S64, max(1, args.warmup))
    el64, its64, status64, K64, _ = run_solves(S64, args.steps)
    tts64_ms = 1e3 * el64 / args.steps
    e0.record()
    for _ in range(args.spmv_reps):
        S64.cg_spmv(xin, y)
    e1.record()
    torch.cuda.synchronize()
    spmv64_ms = e0.elapsed_time(e1) / args.spmv_reps
    print(f"# fp64 map: {status64} K={K64} TTS {tts64_ms:.3f} ms; spmv mixed {spmv_ms * 1e3:.1f} us, "
          f"fp64 {spmv64_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # The per-segment max|p| rule (paper Sec. 4.7) at its paper setting,
    # lo = tol/10, hi = tol, on the same substrate: evaluated every iteration,
    # then reused over K* iterations, K* chosen offline (Sec. 3.4) from a
    # recorded per-iteration run.
    Spm = mpcg.Solver(L)
    Spm.cg_set_schedule_pmag(w.tol / 10, w.tol, 1)
    run_solves(Spm, max(1, args.warmup))
    elpm, itspm, statuspm, Kpm, _ = run_solves(Spm, args.steps)
    ttspm_ms = 1e3 * elpm / args.steps
    ks, cnt = Spm.cg_get_map_trace(cap=w.maxit + 2)
    pm_frac = (cnt.sum(axis=0) / max(cnt.sum(), 1)).round(4).tolist()
    truepm = float(np.linalg.norm(w.b - A.to_scipy() @ x.cpu().numpy()) / np.linalg.norm(w.b))
    Spm.cg_record_column_codes(True)
    Spm.cg_solve(b, x, w.tol, w.maxit)
    kstar, ktable = mpcg.cg_select_reuse_interval(Spm.cg_get_column_codes(), 0.1)
    Spm.cg_record_column_codes(False)
    Spm.cg_set_schedule_pmag(w.tol / 10, w.tol, kstar)
    run_solves(Spm, max(1, args.warmup))
    elks, itsks, statusks, Kks, _ = run_solves(Spm, args.steps)
    ttsks_ms = 1e3 * elks / args.steps
    print(f"# max|p| rule: {statuspm} K={Kpm} TTS {ttspm_ms:.3f} ms; tile-iterations FP64/FP32/BF16 "
          f"{pm_frac}; K*={kstar}: {statusks} K={Kks} TTS {ttsks_ms:.3f} ms", file=sys.stderr, flush=True)
    Spm.close()

    # The paper's own SpMV numerics on the bench's map: the vector entry rounded
    # with its tile (Eq. 9/10); with the per-column scale and the sentinel
    # padding of Sec. 3.3.2 / Fig. 4(b) on top.
    p1 = {}
    for name, flags in (("round_vector", mpcg.CG_P1_ROUND_VECTOR),
                        ("round_scale_pad", mpcg.CG_P1_ROUND_VECTOR | mpcg.CG_P1_COLUMN_SCALE
                         | mpcg.CG_P1_PAD_COLUMNS)):
        Sp = mpcg.Solver(L, pmap, p1=flags)
        for _ in range(10):
            Sp.cg_spmv(xin, y)
        e0.record()
        for _ in range(args.spmv_reps):
            Sp.cg_spmv(xin, y)
        e1.record()
        torch.cuda.synchronize()
        sp_ms = e0.elapsed_time(e1) / args.spmv_reps
        run_solves(Sp, max(1, args.warmup))
        elp, itsp, statusp, Kp, _ = run_solves(Sp, args.steps)
        truep = float(np.linalg.norm(w.b - A.to_scipy() @ x.cpu().numpy()) / np.linalg.norm(w.b))
        extra = 2 * A.n if flags & mpcg.CG_P1_COLUMN_SCALE else 0  # the scale exponents
        p1[name] = {"flags": flags, "spmv_us": round(sp_ms * 1e3, 2),
                    "spmv_gbs": round((bytes_spmv + extra) / (sp_ms * 1e-3) / 1e9, 1),
                    "stored_nonzeros": Sp.nnz, "status": statusp, "iterations": Kp,
                    "time_to_solution_ms": round(1e3 * elp / args.steps, 4), "true_residual": truep}
        print(f"# P1 {name}: spmv {sp_ms * 1e3:.1f} us; {statusp} K={Kp} TTS {1e3 * elp / args.steps:.3f} ms, "
              f"true residual {truep:.3e}", file=sys.stderr, flush=True)
        Sp.close()

    # Counter results (rocprofv3 runs of --pmc-probe), reported only while they
    # describe the kernels as built from the current sources.
    traffic, l2 = None, None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")
            c = tr.get("l2", {})
            if c:
                l2 = {"spmv_hit_rate_mixed_map": c["mixed"]["hit_rate"],
                      "spmv_hit_rate_fp64_map": c["fp64"]["hit_rate"],
                      "x_gather_hit_rate_estimate": c.get("x_gather_estimate", {}).get("hit_rate"),
                      "source": os.path.relpath(TRAFFIC_FILE, ROOT)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, pmap, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(iters_per_s, 2),
        "unit": "CG iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tts_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded generator; no dataset)",
        "config": {
            "workload": "3D 7-point Laplacian 128^3, 16x16 Tile-CSC, static 50/30/20 FP64/FP32/BF16 "
                        "tile map, CG to rel. residual 1e-8 from x0 = 0",
            "n": A.n, "nnz": A.nnz, "tiles": L.T,
            "map_tiles_fp64_fp32_bf16": np.bincount(pmap, minlength=3).tolist(),
        },
        "iterations": K,
        "status": status,
        "time_to_solution_ms": round(tts_ms, 4),
        "true_residual": true_res,
        "tile_csc_spmv_gbs": round(spmv_gbs, 1),
        "tile_csc_spmv_frac_hbm": round(spmv_gbs / HBM_PEAK_GBS, 4),
        "tile_csc_spmv_us": round(spmv_ms * 1e3, 2),
        "cg_iteration_gbs": round(iter_gbs, 1),
        "cg_iteration_frac_hbm": round(iter_gbs / HBM_PEAK_GBS, 4),
        "fp64_map": {"iterations": K64, "time_to_solution_ms": round(tts64_ms, 4),
                     "spmv_us": round(spmv64_ms * 1e3, 2),
                     "spmv_gbs": round(bytes_spmv64 / (spmv64_ms * 1e-3) / 1e9, 1)},
        "mixed_over_fp64_tts_speedup": round(tts64_ms / tts_ms, 4),
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "pmag_rule": {"lo": w.tol / 10, "hi": w.tol, "status": statuspm, "iterations": Kpm,
                      "time_to_solution_ms": round(ttspm_ms, 4),
                      "iterations_per_s": round(itspm / elpm, 2),
                      "true_residual": truepm,
                      "tile_iterations_fp64_fp32_bf16": pm_frac,
                      "reuse_interval_kstar": kstar,
                      "kstar_delayed_upward_fractions": ktable,
                      "reused": {"status": statusks, "iterations": Kks,
                                 "time_to_solution_ms": round(ttsks_ms, 4)}},
        "p1_numerics": p1,
        "roofline": {
            "bound": "hbm",
            "kernel": "spmv_tilecsc_kernel (cg_spmv)",
            "achieved": round(spmv_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(spmv_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_spmv,
        },
        "l2": l2,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def configure_map(S, w, L, mpcg_mod):
    """Apply a workload's own precision map or schedule to a handle; returns the static map or None."""
    from gen import static_map, tile_scores

    kind = w.map_spec["kind"]
    scores = tile_scores(L.T, 2)
    if kind == "static":
        m = static_map(scores, w.map_spec["frac_bf16"], w.map_spec["frac_fp32"])
        S.cg_set_precision_map(m)
        return m
    if kind == "magnitude":
        S.cg_map_from_magnitude(w.map_spec["t_bf16"], w.map_spec["t_fp32"])
        return S.cg_get_active_map()
    if kind == "ratchet":
        S.cg_set_schedule_residual(w.map_spec["thresholds"], w.map_spec["prec"])
    elif kind == "tile_rule":
        S.cg_set_schedule_tile_rule(w.map_spec["period"], scores, w.map_spec["hi"], w.map_spec["lo"])
    return None


def all_workloads(torch, dev, mpcg, cfgs, reps, slices=()):
    """Warm time to solution, iterations/s and SpMV bandwidth per workload, both maps.

    Every solve starts from x0 = 0 on the device with b resident; one untimed
    solve, then the median of three timed ones. SpMV bytes are the algorithmic
    count of the map the SpMV runs with (the FP64 map, and the workload's own
    map where it is a fixed per-tile map); an iteration's bytes add 56n (64n
    with Jacobi) for the vector step. Every count in ``slices`` adds the same
    runs on a handle with that many column slices.
    """
    from gen import make_workload

    out = {"metric": "cg_time_to_solution_by_workload", "workloads": []}
    for cfg in cfgs:
        t0 = time.time()
        w = make_workload(cfg, "full")
        A = w.A
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        print(f"# cfg{cfg}: generated and tiled in {time.time() - t0:.0f}s, n={A.n} nnz={A.nnz} T={L.T}",
              file=sys.stderr, flush=True)
        b = torch.from_numpy(w.b).to(dev)
        x = torch.zeros_like(b)
        xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
        y = torch.empty_like(xin)
        vec_bytes = (64 if w.jacobi else 56) * A.n
        rec = {"workload": w.description, "n": A.n, "nnz": A.nnz, "tiles": L.T, "tol": w.tol, "maxit": w.maxit}
        own = w.map_spec["kind"]
        runs = [("fp64", None, 0)] + ([("own", own, 0)] if own != "fp64" else [])
        for ns in slices:  # column-sliced handles (the tile rule needs canonical order)
            runs += [(f"fp64_slices{ns}", None, ns)] + \
                ([(f"own_slices{ns}", own, ns)] if own not in ("fp64", "tile_rule") else [])
        static_own = None  # the magnitude rule's map, set as a fixed map on sliced handles
        for label, kind, ns in runs:
            S = mpcg.Solver(L, np.zeros(L.T, np.uint8), jacobi=w.jacobi, col_slices=ns)
            if kind == "magnitude" and ns > 0:
                S.cg_set_precision_map(static_own)
                m = static_own
            else:
                m = np.zeros(L.T, np.uint8) if kind is None else configure_map(S, w, L, mpcg)
                if kind == "magnitude":
                    static_own = m
            r = {"map": "all FP64" if kind is None else kind, "col_slices": ns}
            if m is not None:
                for _ in range(5):
                    S.cg_spmv(xin, y)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    S.cg_spmv(xin, y)
                e1.record()
                torch.cuda.synchronize()
                sp_ms = e0.elapsed_time(e1) / reps
                nb = spmv_algorithmic_bytes(L, m)
                r.update(spmv_us=round(sp_ms * 1e3, 2), spmv_gbs=round(nb / (sp_ms * 1e-3) / 1e9, 1),
                         spmv_frac_hbm=round(nb / (sp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
            S.cg_solve(b, x, w.tol, w.maxit)
            times = []
            for _ in range(3):
                torch.cuda.synchronize()
                t1 = time.perf_counter()
                status, K, hist = S.cg_solve(b, x, w.tol, w.maxit)
                torch.cuda.synchronize()
                times.append(time.perf_counter() - t1)
            tts = sorted(times)[1]
            true_res = float(np.linalg.norm(w.b - A.to_scipy() @ x.cpu().numpy()) / np.linalg.norm(w.b))
            r.update(status=status, iterations=K, time_to_solution_ms=round(tts * 1e3, 3),
                     iterations_per_s=round(K / tts, 1), recurrence_residual=float(hist[-1]),
                     true_residual=true_res)
            if m is not None:
                it_gbs = (spmv_algorithmic_bytes(L, m) + vec_bytes) * K / tts / 1e9
                r.update(iteration_gbs=round(it_gbs, 1), iteration_frac_hbm=round(it_gbs / HBM_PEAK_GBS, 4))
            rec[label] = r
            print(f"# cfg{cfg} {label}: {status} K={K} TTS {tts * 1e3:.2f} ms ({K / tts:.0f} it/s), "
                  f"true residual {true_res:.2e}" + (f", SpMV {r['spmv_us']} us = {r['spmv_frac_hbm']:.2f} of "
                                                     f"8 TB/s" if 'spmv_us' in r else ""),
                  file=sys.stderr, flush=True)
            S.close()
        if "own" in rec:
            rec["own_over_fp64_tts_speedup"] = round(rec["fp64"]["time_to_solution_ms"] /
                                                     rec["own"]["time_to_solution_ms"], 4)
        L.close()
        out["workloads"].append(rec)
    print(json.dumps(out), flush=True)


def tile_shapes(torch, dev, mpcg, cfgs, reps):
    """cg_spmv under the all-FP64 map at the workload's tile shape and at the tuned heights.

    The tuned height comes from cg_tune_row_height (paper Sec. 3.3.3) with its
    defaults (R <= 256, at least 1024 row blocks). Maps are per tile and differ
    between tilings, so every shape is timed with the FP64 map.
    """
    from gen import make_workload

    out = {"metric": "tile_csc_spmv_by_tile_shape", "map": "all FP64", "workloads": []}
    for cfg in cfgs:
        t0 = time.time()
        w = make_workload(cfg, "full")
        A = w.A
        print(f"# cfg{cfg}: generated in {time.time() - t0:.0f}s, n={A.n} nnz={A.nnz}", file=sys.stderr,
              flush=True)
        shapes = [(w.R, w.C, "workload")]
        for C in (64, w.C):
            R, rows = mpcg.cg_tune_row_height(A.n, A.indptr, A.indices, C)
            if (R, C) not in [(s[0], s[1]) for s in shapes]:
                shapes.append((R, C, f"tuned for C={C}"))
        res = []
        for R, C, label in shapes:
            L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, R, C)
            S = mpcg.Solver(L, np.zeros(L.T, np.uint8))
            xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
            y = torch.empty_like(xin)
            for _ in range(10):
                S.cg_spmv(xin, y)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                S.cg_spmv(xin, y)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            nbytes = spmv_algorithmic_bytes(L, np.zeros(L.T, np.uint8))
            gbs = nbytes / (ms * 1e-3) / 1e9
            counts = np.diff(L.tile_row_ptr)
            rec = {"R": R, "C": C, "shape": label, "tiles": L.T, "spmv_us": round(ms * 1e3, 2),
                   "algorithmic_bytes": nbytes, "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                   "row_block_tile_cv": round(float(counts.std() / max(counts.mean(), 1e-300)), 4)}
            res.append(rec)
            print(f"# cfg{cfg} {label}: {R}x{C} T={L.T} spmv {ms * 1e3:.1f} us, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
            S.close()
            L.close()
        out["workloads"].append({"workload": w.description, "n": A.n, "nnz": A.nnz, "shapes": res})
    print(json.dumps(out), flush=True)


def pmc_probe(torch, dev, S, L, A, pmap, b, w, mpcg):
    """Launch sequence for the HBM counter runs: the copy of known size first, then the
    SpMV under each map, then five CG iterations on the mixed map launched one by one
    (no graph), so that the update and direction kernels are counted too. Counters are
    read per dispatch by rocprofv3."""
    src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
    y = torch.empty_like(xin)
    for name, m in (("fp64", np.zeros(L.T, np.uint8)), ("mixed", pmap), ("bf16", np.full(L.T, 2, np.uint8))):
        S.cg_set_precision_map(m)
        for _ in range(5):
            S.cg_spmv(xin, y)
        torch.cuda.synchronize()
        print(f"# pmc probe: 5 cg_spmv launches, {name} map, algorithmic bytes "
              f"{spmv_algorithmic_bytes(L, m)}", file=sys.stderr, flush=True)
    Sc = mpcg.Solver(L, pmap, use_graph=0)
    x = torch.zeros_like(b)
    Sc.cg_solve(b, x, 0.0, 5)
    torch.cuda.synchronize()
    Sc.close()
    print(f"# pmc probe: 5 CG iterations, mixed map, vector bytes per iteration: update {24 * A.n}, "
          f"direction {40 * A.n}", file=sys.stderr, flush=True)


def small_systems(torch, dev, mpcg):
    """Time per CG iteration of the single-workgroup and the multi-launch solve.

    Laplacians (16x16 tiles, FP64 map, b = A x*, x* ~ U[-1, 1] seed 0, x0 = 0,
    tol 1e-10): one untimed solve, then the best of three timed ones per path.
    """
    from gen.matrices import laplace2d_5pt, laplace3d_7pt

    out = {"metric": "cg_us_per_iteration_small_systems", "cases": []}
    cases = [("2D 5-point", m, laplace2d_5pt) for m in (8, 16, 32, 48, 64, 96, 128, 192)] + \
        [("3D 7-point", m, laplace3d_7pt) for m in (6, 8, 12, 16, 21, 28, 36)]
    for name, m, gen_fn in cases:
        A = gen_fn(m)
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, 16, 16)
        b = torch.from_numpy(A.to_scipy() @ np.random.default_rng(0).uniform(-1, 1, A.n)).to(dev)
        rec = {"matrix": f"{name} Laplacian {m}^{2 if name.startswith('2D') else 3}", "n": A.n, "nnz": A.nnz}
        for label, sb in (("single_workgroup", 1), ("multi_launch", -1)):
            S = mpcg.Solver(L, single_block=sb)
            x = torch.zeros_like(b)
            S.cg_solve(b, x, 1e-10, 20000)
            best = float("inf")
            for _ in range(3):
                torch.cuda.synchronize()
                t = time.perf_counter()
                st, K, _ = S.cg_solve(b, x, 1e-10, 20000)
                torch.cuda.synchronize()
                best = min(best, time.perf_counter() - t)
            rec[label] = {"status": st, "iterations": K, "time_to_solution_ms": round(best * 1e3, 3),
                          "us_per_iteration": round(best / max(K, 1) * 1e6, 2)}
            S.close()
        L.close()
        rec["speedup"] = round(rec["multi_launch"]["time_to_solution_ms"] /
                               rec["single_workgroup"]["time_to_solution_ms"], 3)
        print(f"# {rec['matrix']}: n={A.n} nnz={A.nnz} one workgroup "
              f"{rec['single_workgroup']['us_per_iteration']} us/it, three launches "
              f"{rec['multi_launch']['us_per_iteration']} us/it", file=sys.stderr, flush=True)
        out["cases"].append(rec)
    print(json.dumps(out), flush=True)


def spmv_probe(torch, dev, mpcg, cfgs, slices):
    """Launch sequence for counter runs of the SpMV on any workload: the copy of known
    size, then per workload and column-slice count (0 = unsliced) five cg_spmv launches
    under the all-FP64 map. With slices the combine kernel follows every SpMV."""
    from gen import make_workload

    src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    for cfg in cfgs:
        w = make_workload(cfg, "full")
        A = w.A
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        m = np.zeros(L.T, np.uint8)
        xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
        y = torch.empty_like(xin)
        for ns in [0] + list(slices):
            S = mpcg.Solver(L, m, col_slices=ns)
            for _ in range(5):
                S.cg_spmv(xin, y)
            torch.cuda.synchronize()
            S.close()
            print(f"# spmv probe: cfg{cfg}, {ns} column slices, 5 cg_spmv launches, all-FP64 map, "
                  f"algorithmic bytes {spmv_algorithmic_bytes(L, m)}", file=sys.stderr, flush=True)
        L.close()


def cpu_baseline(w, pmap, budget_s):
    """The CPU oracle on a bounded sample: its CG iterations on the full workload for
    about ``budget_s`` seconds on one thread. The per-iteration rate is the difference of
    two runs of different lengths, so the oracle's set-up (layout build, value streams,
    first residual) is excluded, as it is from the GPU time to solution."""
    from threadpoolctl import threadpool_limits

    from oracle import cg as ocg, tilecsc as otc

    A = w.A

    def timed(iters):
        t = time.time()
        r = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, ocg.StaticSchedule(pmap), 0.0, iters)
        return time.time() - t, r.K

    with threadpool_limits(limits=1):
        Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        t_a, k_a = timed(2)
        t_b, k_b = timed(12)
        per_iter = max((t_b - t_a) / max(k_b - k_a, 1), 1e-6)
        iters = max(20, int(budget_s / per_iter))
        t_c, k_c = timed(iters)
    rate = (k_c - k_a) / (t_c - t_a)
    return {"value": round(rate, 3), "unit": "CG iterations/s", "cores": 1, "kind": "oracle",
            "sample": f"{k_c - k_a} oracle CG iterations (runs of {k_c} and {k_a} differenced) on the "
                      f"full 128^3 workload with the same map, {t_c - t_a:.1f} s on one thread; "
                      f"layout build and value streams excluded"}


if __name__ == "__main__":
    main()
