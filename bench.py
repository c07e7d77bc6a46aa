"""Benchmark: mixed-precision Tile-CSC CG on one MI355X.

Workload (the largest of the five, and the only one whose SpMV working set,
1.8 GB, is far larger than the 256 MB Infinity Cache): the Q1 finite-element
stiffness of -div(diag(1, 1e-3) grad u) on a 4096^2 grid (a 2D 9-point
anisotropic stencil, n = 16,777,216, nnz = 150,945,796), 32x32 tiles,
b = A x* with x* ~ U[-1, 1], x0 = 0, CG to ||r_k||/||r_0|| <= 1e-9 or 5000
iterations. Its own precision map: every 10 iterations each tile is
re-selected from a seeded score s_t and the current residual rho_k
(v_t = s_t rho_k; BF16 if v_t > 1e-3, FP32 if v_t > 1e-6, else FP64).

One step is one complete cg_solve (every iteration: the window map step,
the SpMV with fused p.q, the x/r update with fused reductions, the direction
update, the device stop flag) with b already resident on the GPU. The
all-FP64 map is timed on the same substrate beside it.

Prints one JSON line: CG iterations/s over the timed solves, time to
solution, the true residuals (FP64, recomputed by the library after each
solve, untimed), the Tile-CSC SpMV bandwidth against the 8 TB/s HBM roofline
and against the read and copy bandwidth measured in the same run, the
iteration's bandwidth, and the CPU oracle's rate on a bounded sample.
"""

import argparse
import csv
import glob
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
STREAM_BYTES = 2 << 30  # bandwidth references: far larger than the 256 MB Infinity Cache
METRIC = "Tile-CSC SpMV GB/s (% HBM peak); CG iterations/sec; time-to-solution"
HEADLINE_CFG = 5
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spmv_tilecsc_cfg5_traffic.json")
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


def tile_rule_bytes_per_iteration(L, scores, hist, period, hi, lo):
    """Average algorithmic SpMV bytes per iteration of a solve under the windowed tile rule.

    The rule is a pure function of the scores and of rho at each window start
    (v_t = s_t rho_k: BF16 if v_t > hi, FP32 if v_t > lo, else FP64), so each
    window's map follows from the residual history; with the tiles sorted by
    score, a window's nonzeros per precision are two prefix sums. Returns
    (mean bytes, mean nonzero fractions FP64/FP32/BF16)."""
    nnz_t = np.diff(L.tile_nnz_ptr).astype(np.int64)
    order = np.argsort(scores, kind="stable")
    s_sorted = scores[order]
    cum = np.concatenate([[0], np.cumsum(nnz_t[order])])
    fixed = 2 * L.nnz + 9 * L.T + 4 * (-(-L.n // L.R) + 1) + 16 * L.n
    K = len(hist) - 1
    tot_bytes, fr = 0.0, np.zeros(3)
    v = np.empty_like(s_sorted)
    for k0 in range(0, K, period):
        rho = hist[k0]
        its = min(period, K - k0)
        # v_t = s_t rho is non-decreasing along the sorted scores, so the tiles with
        # v_t > hi (BF16) and v_t > lo (BF16 or FP32) are suffixes of that order
        np.multiply(s_sorted, rho, out=v)
        i_hi = int(np.searchsorted(v, hi, side="right"))
        i_lo = int(np.searchsorted(v, lo, side="right"))
        n16 = cum[-1] - cum[i_hi]
        n32 = cum[i_hi] - cum[i_lo]
        n64 = cum[i_lo]
        tot_bytes += its * (8 * n64 + 4 * n32 + 2 * n16 + fixed)
        fr += its * np.array([n64, n32, n16]) / L.nnz
    return tot_bytes / max(K, 1), (fr / max(K, 1)).round(4).tolist()


def time_events(torch, fn, reps, warm=5):
    """Average milliseconds of fn() over reps launches, HIP events on the current stream."""
    for _ in range(warm):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def median_launch_ms(torch, fn, reps=20, warm=5):
    """Median over reps launches of fn(), each between its own pair of HIP events on the
    current stream, after warm untimed launches."""
    for _ in range(warm):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def bandwidth_references(torch, dev, mpcg, write_share=None):
    """Read-only and copy bandwidth of the library's stream kernels on 2 GiB buffers (best grid);
    with write_share (bytes written per byte read), also a 2 GiB read stream that writes that
    share alongside (None otherwise). Bytes per second count reads and writes."""
    src = torch.empty(STREAM_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    dst = torch.empty_like(src)
    sink = torch.empty(65536, dtype=torch.float64, device=dev)
    wdst = None
    if write_share is not None:
        wdst = dst[: int(STREAM_BYTES * write_share) // 16 * 2]
    best_r, best_c, best_m = 0.0, 0.0, None
    for blocks in (4096, 8192, 16384, 32768):
        ms = time_events(torch, lambda: mpcg.cg_stream_read(src, sink, blocks), 10, 3)
        best_r = max(best_r, STREAM_BYTES / (ms * 1e-3) / 1e9)
        ms = time_events(torch, lambda: mpcg.cg_stream_copy(src, dst, blocks), 10, 3)
        best_c = max(best_c, 2 * STREAM_BYTES / (ms * 1e-3) / 1e9)
        if wdst is not None:
            ms = time_events(torch, lambda: mpcg.cg_stream_mix(src, wdst, sink, blocks), 10, 3)
            best_m = max(best_m or 0.0, (STREAM_BYTES + wdst.numel() * 8) / (ms * 1e-3) / 1e9)
    del src, dst, sink, wdst
    torch.cuda.empty_cache()
    return round(best_r, 1), round(best_c, 1), (round(best_m, 1) if best_m is not None else None)


def load_counters():
    """Traffic and L2 figures of the counter runs (profiles/), only while they describe the
    kernels as built from the current sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    tr = json.load(open(TRAFFIC_FILE))
    if tr.get("kernel_source_hash") != kernel_source_hash():
        return None, None
    l2 = None
    if tr.get("l2"):
        l2 = dict(tr["l2"], source=os.path.relpath(TRAFFIC_FILE, ROOT))
    return tr.get("bytes_per_launch"), l2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--spmv-reps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=13.0,
                    help="approximate CPU time of the oracle's timed iterations")
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
    ap.add_argument("--pmag", default="",
                    help="comma-separated workloads (e.g. 2,5): instead of the CG bench, time CG under the "
                         "max|p| rule (paper Sec. 4.7) evaluated every iteration, select the reuse interval "
                         "K* from a recorded run (Sec. 3.4) and time the rule reused over K* iterations, "
                         "at the paper's setting (lo = tol/10, hi = tol) and at lo = 1e-4, hi = 1e-2, beside "
                         "the all-FP64 map; prints one JSON line")
    ap.add_argument("--stage-x", action="store_true",
                    help="with --workloads: also time each workload on a handle with cg_options.stage_x = 1 (x "
                         "segments staged in LDS per batch); with --spmv-probe: one more group of five launches "
                         "per workload on such a handle")
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
                    help="counter run on the headline workload: the 256 MiB copy of cg_stream_copy (the "
                         "scale reference), then 5 cg_spmv launches per map (all FP64, 50/30/20 mixed, "
                         "all BF16); no timing")
    ap.add_argument("--map-switch-probe", action="store_true",
                    help="copy-trace run on the headline workload: after the handle is built, three map "
                         "switches (cg_set_precision_map), each followed by one cg_spmv; prints the bytes a "
                         "switch should move (the map) beside the matrix's value and index bytes")
    ap.add_argument("--spmv-only", action="store_true",
                    help="kernel-trace run on the headline workload: --spmv-reps timed cg_spmv launches under "
                         "the all-FP64 map and nothing else on the GPU; prints one JSON line")
    ap.add_argument("--traffic-from", nargs="+", default=None, metavar="DIR",
                    help="no GPU: read rocprofv3 counter CSVs of --pmc-probe runs (directories holding "
                         "FETCH_SIZE, WRITE_SIZE and optionally TCC_HIT_sum/TCC_MISS_sum), scale them by the "
                         "copy reference, and write " + os.path.relpath(TRAFFIC_FILE, ROOT))
    ap.add_argument("--traffic-groups", default="",
                    help="with --traffic-from: comma-separated names of the groups of 5 SpMV dispatches, in "
                         "order (default: the three maps of --pmc-probe)")
    ap.add_argument("--traffic-out", default=None,
                    help="with --traffic-from: JSON file to write (default: the file the benchmark reads)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.traffic_from:
        if args.traffic_groups:
            traffic_from(args.traffic_from, args.traffic_groups.split(","), args.traffic_out)
        else:
            traffic_from(args.traffic_from, out_path=args.traffic_out)
        return

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
    if args.pmag:
        pmag_bench(torch, dev, mpcg, [int(c) for c in args.pmag.split(",")])
        return
    if args.spmv_probe:
        spmv_probe(torch, dev, mpcg, [int(c) for c in args.spmv_probe.split(",")],
                   [int(c) for c in args.col_slices.split(",") if c], args.stage_x)
        return
    if args.workloads:
        all_workloads(torch, dev, mpcg, [int(c) for c in args.workloads.split(",")], args.spmv_reps, args.stage_x,
                      [int(c) for c in args.col_slices.split(",") if c])
        return

    t0 = time.time()
    w = make_workload(HEADLINE_CFG, "full")
    A = w.A
    L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    scores = tile_scores(L.T, 2)
    ms = w.map_spec
    zeros = np.zeros(L.T, np.uint8)
    S = mpcg.Solver(L, zeros)
    setup_s = time.time() - t0
    print(f"# setup {setup_s:.1f}s: n={A.n} nnz={A.nnz} T={L.T}", file=sys.stderr, flush=True)
    xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
    y = torch.empty_like(xin)

    if args.pmc_probe:
        pmc_probe(torch, dev, S, L, A, xin, y, scores, mpcg)
        return
    if args.map_switch_probe:
        map_switch_probe(torch, S, L, xin, y, scores)
        return
    if args.spmv_only:
        spmv_ms = time_events(torch, lambda: S.cg_spmv(xin, y), args.spmv_reps, 10)
        nb = spmv_algorithmic_bytes(L, zeros)
        print(json.dumps({"metric": "tile_csc_spmv_fp64_map", "workload": w.description, "launches": args.spmv_reps,
                          "spmv_us": round(spmv_ms * 1e3, 2), "algorithmic_bytes": nb,
                          "gbs": round(nb / (spmv_ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    # The SpMV alone under the all-FP64 map (the roofline kernel), a 50/30/20 mixed
    # map, all BF16, and the tile rule's first-window map (rho = 1).
    spmv = {}
    m_static = static_map(scores, 0.2, 0.3)
    S.cg_set_schedule_tile_rule(ms["period"], scores, ms["hi"], ms["lo"])
    S.cg_eval_tile_rule(1.0)
    m_first = S.cg_get_active_map()
    for name, m in (("fp64", zeros), ("mixed_50_30_20", m_static), ("bf16", np.full(L.T, 2, np.uint8)),
                    ("tile_rule_first_window", m_first)):
        S.cg_set_precision_map(m)
        t_ms = time_events(torch, lambda: S.cg_spmv(xin, y), args.spmv_reps, 10)
        med_ms = median_launch_ms(torch, lambda: S.cg_spmv(xin, y))
        nb = spmv_algorithmic_bytes(L, m)
        spmv[name] = {"us": round(t_ms * 1e3, 2), "us_median_of_20": round(med_ms * 1e3, 2), "algorithmic_bytes": nb,
                      "gbs": round(nb / (t_ms * 1e-3) / 1e9, 1),
                      "frac_hbm": round(nb / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "map_nnz_fp64_fp32_bf16": [int(v) for v in
                                                 np.bincount(m, weights=np.diff(L.tile_nnz_ptr), minlength=3)]}
        print(f"# spmv {name}: {t_ms * 1e3:.1f} us, {spmv[name]['gbs']} GB/s", file=sys.stderr, flush=True)

    b = torch.from_numpy(w.b).to(dev)
    x = torch.zeros_like(b)

    def run_solves(solver, steps):
        its, ks = 0, []
        status, K, hist = None, 0, None
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            status, K, hist = solver.cg_solve(b, x, w.tol, w.maxit)
            its += K
            ks.append(K)
        torch.cuda.synchronize()
        return time.perf_counter() - t, its, status, K, hist

    # The workload's own map: the windowed tile rule.
    S.cg_set_schedule_tile_rule(ms["period"], scores, ms["hi"], ms["lo"])
    run_solves(S, args.warmup)
    el, its, status, K, hist = run_solves(S, args.steps)
    tts_ms = 1e3 * el / args.steps
    iters_per_s = its / el
    true_res = S.cg_true_residual(b, x)
    ks, cnt = S.cg_get_map_trace(cap=w.maxit // ms["period"] + 2)
    it_bytes, nnz_frac = tile_rule_bytes_per_iteration(L, scores, hist, ms["period"], ms["hi"], ms["lo"])
    vec_bytes = 56 * A.n
    iter_gbs = (it_bytes + vec_bytes) * its / el / 1e9
    print(f"# tile rule: {status} K={K} TTS {tts_ms:.1f} ms, {iters_per_s:.1f} it/s, true residual {true_res:.3e}, "
          f"SpMV nnz fractions FP64/FP32/BF16 {nnz_frac}", file=sys.stderr, flush=True)

    # The all-FP64 map on the same substrate (fewer steps: the same solve length).
    S64 = mpcg.Solver(L, zeros)
    st64 = max(1, min(args.steps, 3))
    run_solves(S64, 1)
    el64, its64, status64, K64, hist64 = run_solves(S64, st64)
    tts64_ms = 1e3 * el64 / st64
    true64 = S64.cg_true_residual(b, x)
    bytes64 = spmv_algorithmic_bytes(L, zeros)
    iter64_gbs = (bytes64 + vec_bytes) * its64 / el64 / 1e9
    print(f"# fp64 map: {status64} K={K64} TTS {tts64_ms:.1f} ms, true residual {true64:.3e}",
          file=sys.stderr, flush=True)
    S64.close()
    S.close()

    # The FP64-map SpMV writes y (8n bytes) and reads the rest of its algorithmic bytes.
    sp64 = spmv["fp64"]
    share = 8 * A.n / (sp64["algorithmic_bytes"] - 8 * A.n)
    read_gbs, copy_gbs, mix_gbs = bandwidth_references(torch, dev, mpcg, share)
    traffic, l2 = load_counters()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, L.T, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(iters_per_s, 2),
        "unit": "CG iterations/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tts_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded generator; no dataset)",
        "config": {
            "workload": "Q1 FEM stiffness of -div(diag(1, 1e-3) grad u) on a 4096^2 grid (2D 9-point anisotropic "
                        "stencil), 32x32 Tile-CSC, per-tile precision re-selected every 10 iterations from seeded "
                        "scores and rho_k, CG to rel. residual 1e-9 or 5000 iterations from x0 = 0",
            "n": A.n, "nnz": A.nnz, "tiles": L.T, "tol": w.tol, "maxit": w.maxit,
        },
        "status": status,
        "iterations": K,
        "time_to_solution_ms": round(tts_ms, 3),
        "recurrence_residual": float(hist[-1]),
        "true_residual": true_res,
        "spmv_nnz_fraction_fp64_fp32_bf16": nnz_frac,
        "cg_iteration_algorithmic_bytes": int(it_bytes + vec_bytes),
        "cg_iteration_gbs": round(iter_gbs, 1),
        "cg_iteration_frac_hbm": round(iter_gbs / HBM_PEAK_GBS, 4),
        "fp64_map": {"status": status64, "iterations": K64, "time_to_solution_ms": round(tts64_ms, 3),
                     "iterations_per_s": round(its64 / el64, 2), "recurrence_residual": float(hist64[-1]),
                     "true_residual": true64, "cg_iteration_gbs": round(iter64_gbs, 1),
                     "cg_iteration_frac_hbm": round(iter64_gbs / HBM_PEAK_GBS, 4)},
        "own_map_over_fp64_tts_speedup": round(tts64_ms / tts_ms, 4),
        "own_map_vs_fp64_true_residual": [true_res, true64],
        "tile_csc_spmv": spmv,
        "read_ceiling_gbs": read_gbs,
        "copy_ceiling_gbs": copy_gbs,
        "spmv_mix_ceiling_gbs": mix_gbs,
        "spmv_mix_write_share": round(share, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "spmv_tilecsc_kernel (cg_spmv, all-FP64 map)",
            "achieved": sp64["gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": sp64["frac_hbm"],
            "traffic": traffic,
            "algorithmic_bytes_per_launch": sp64["algorithmic_bytes"],
            "launch_us": sp64["us"],
            "frac_of_read_ceiling": round(sp64["gbs"] / read_gbs, 4),
            "frac_of_mix_ceiling": round(sp64["gbs"] / mix_gbs, 4),
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


def all_workloads(torch, dev, mpcg, cfgs, reps, stage_x=False, slices=()):
    """Warm time to solution, iterations/s and SpMV bandwidth per workload, both maps.

    Every solve starts from x0 = 0 on the device with b resident; one untimed
    solve, then the median of three timed ones. SpMV bytes are the algorithmic
    count of the map the SpMV runs with (the FP64 map, and the workload's own
    map where it is a fixed per-tile map); an iteration's bytes add 56n (64n
    with Jacobi) for the vector step. Every count in ``slices`` adds the same
    runs on a handle with that many column slices.
    """
    from gen import make_workload, tile_scores

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
        # default handles (automatic column slices), then one per forced slice count
        runs = [("fp64", None, 0)] + ([("own", own, 0)] if own != "fp64" else [])
        for ns in slices:
            runs += [(f"fp64_slices{ns}", None, ns)] + ([(f"own_slices{ns}", own, ns)] if own != "fp64" else [])
        if stage_x:  # x segments staged in LDS per batch (cg_options.stage_x)
            runs += [("fp64_stage_x", None, 0)]
        for label, kind, ns in runs:
            S = mpcg.Solver(L, np.zeros(L.T, np.uint8), jacobi=w.jacobi, col_slices=ns,
                            stage_x=1 if label.endswith("stage_x") else 0)
            m = np.zeros(L.T, np.uint8) if kind is None else configure_map(S, w, L, mpcg)
            r = {"map": "all FP64" if kind is None else kind, "col_slices_option": ns,
                 "col_slices": S.cg_get_options()["col_slices"], "stage_x": S.cg_get_options()["stage_x"]}
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
            true_res = S.cg_true_residual(b, x)
            r.update(status=status, iterations=K, time_to_solution_ms=round(tts * 1e3, 3),
                     iterations_per_s=round(K / tts, 1), recurrence_residual=float(hist[-1]),
                     true_residual=true_res)
            sp_bytes = None
            if m is not None:
                sp_bytes = spmv_algorithmic_bytes(L, m)
            elif kind == "tile_rule":
                sp_bytes, fr = tile_rule_bytes_per_iteration(L, tile_scores(L.T, 2), hist, w.map_spec["period"],
                                                             w.map_spec["hi"], w.map_spec["lo"])
                r.update(spmv_nnz_fraction_fp64_fp32_bf16=fr)
            if sp_bytes is not None:
                it_gbs = (sp_bytes + vec_bytes) * K / tts / 1e9
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
    defaults (every candidate 32 .. 16384, at least 1024 row blocks). Maps are
    per tile and differ between tilings, so every shape is timed with the FP64
    map. A height above 256 runs on the device as slabs of R' rows (R' the
    largest divisor of R not above 256) whose pieces are the tiles of the
    R' x C layout: its algorithmic bytes count those pieces.
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
            Rs, Ld = R, L
            if R > 256:
                Rs = max(d for d in range(1, 257) if R % d == 0)
                Ld = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, Rs, C)
            nbytes = spmv_algorithmic_bytes(Ld, np.zeros(Ld.T, np.uint8))
            pieces = Ld.T
            if Ld is not L:
                Ld.close()
            gbs = nbytes / (ms * 1e-3) / 1e9
            counts = np.diff(L.tile_row_ptr)
            rec = {"R": R, "C": C, "shape": label, "tiles": L.T, "device_rows": Rs, "device_tiles": pieces,
                   "spmv_us": round(ms * 1e3, 2),
                   "algorithmic_bytes": nbytes, "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                   "row_block_tile_cv": round(float(counts.std() / max(counts.mean(), 1e-300)), 4)}
            res.append(rec)
            print(f"# cfg{cfg} {label}: {R}x{C} T={L.T} spmv {ms * 1e3:.1f} us, {gbs:.0f} GB/s", file=sys.stderr,
                  flush=True)
            S.close()
            L.close()
        out["workloads"].append({"workload": w.description, "n": A.n, "nnz": A.nnz, "shapes": res})
    print(json.dumps(out), flush=True)


def pmc_probe(torch, dev, S, L, A, xin, y, scores, mpcg):
    """Launch sequence for the HBM counter runs on the headline workload: the library's
    stream copy of 256 MiB first (the scale reference: 256 MiB read, 256 MiB written), then
    5 cg_spmv launches per map (all FP64, 50/30/20 mixed, all BF16). Counters are read per
    dispatch by rocprofv3; --traffic-from turns them into bytes per launch."""
    from gen import static_map

    src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    mpcg.cg_stream_copy(src, dst, 8192)
    torch.cuda.synchronize()
    del src, dst
    for name, m in (("fp64", np.zeros(L.T, np.uint8)), ("mixed_50_30_20", static_map(scores, 0.2, 0.3)),
                    ("bf16", np.full(L.T, 2, np.uint8))):
        S.cg_set_precision_map(m)
        for _ in range(5):
            S.cg_spmv(xin, y)
        torch.cuda.synchronize()
        print(f"# pmc probe: 5 cg_spmv launches, {name} map, algorithmic bytes "
              f"{spmv_algorithmic_bytes(L, m)}", file=sys.stderr, flush=True)


def map_switch_probe(torch, S, L, xin, y, scores):
    """Launch sequence for a memory-copy trace: one cg_spmv, then three map switches on the live
    handle, each followed by one cg_spmv. A switch must move the map (one byte per tile) and
    nothing of the matrix: the packed copy of the selected values is rebuilt on the device from
    the resident planes. The copies after the first product's dispatch are the switches'."""
    from gen import static_map

    S.cg_spmv(xin, y)  # everything before this product is set-up; the switches come after it
    torch.cuda.synchronize()
    print(f"# map switch probe: T = {L.T} tiles (map bytes), nnz = {L.nnz}: values "
          f"{14 * L.nnz} bytes in three planes, indices {L.nnz * (2 if max(L.R, L.C) > 16 else 1)} bytes",
          file=sys.stderr, flush=True)
    for name, m in (("mixed_50_30_20", static_map(scores, 0.2, 0.3)), ("bf16", np.full(L.T, 2, np.uint8)),
                    ("fp64", np.zeros(L.T, np.uint8))):
        S.cg_set_precision_map(m)
        S.cg_spmv(xin, y)
        torch.cuda.synchronize()
        print(f"# map switch probe: switched to {name}, one cg_spmv", file=sys.stderr, flush=True)


def _counter_rows(d):
    """(kernel name, counter name, value, dispatch id) of every counter row under directory d."""
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), int(r["Dispatch_Id"])))
    return rows


def traffic_from(dirs, names=("fp64", "mixed_50_30_20", "bf16"), out_path=None):
    """Bytes per SpMV launch from rocprofv3 --pmc runs of --pmc-probe (or --spmv-probe).

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they read for the
    stream copy of 256 MiB that opens the probe (its bytes are known: 256 MiB each way).
    The SpMV dispatches come in groups of five, one group per name in `names` (for
    --pmc-probe: FP64, mixed, BF16 maps, in that order). With TCC_HIT_sum/TCC_MISS_sum,
    the L2 hit rate of each group is reported too. Writes a JSON file (by default the one
    the benchmark reads, bytes_per_launch from the first group), stamped with the kernel
    source hash."""
    names = list(names)
    per = {}  # counter -> list of (dispatch, kernel, value)
    for d in dirs:
        for kname, cname, val, disp in _counter_rows(d):
            per.setdefault(cname, []).append((disp, kname, val))
    out = {"kernel_source_hash": kernel_source_hash(), "counters_from": [os.path.basename(d.rstrip("/")) for d in dirs]}

    def groups(cname):
        rows = sorted(per.get(cname, []))
        copy = [v for _, k, v in rows if "stream_copy_kernel" in k]
        spmv = [v for _, k, v in rows if "spmv_tilecsc_kernel" in k]
        return copy, [spmv[i:i + 5] for i in range(0, len(spmv), 5)]

    ref = float(COPY_BYTES) / 1024.0  # KiB moved each way by the reference copy
    res = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        copy, g = groups(cname)
        if not copy or len(g) < len(names):
            raise SystemExit(f"{cname}: expected the stream copy and {len(names)} groups of 5 SpMV dispatches")
        scale = ref / copy[0]
        res[cname] = {"reference_kib": copy[0], "scale": round(scale, 4),
                      "per_map_bytes": [float(np.mean(x)) * scale * 1024.0 for x in g[:len(names)]]}
    out["scale"] = {c: res[c]["scale"] for c in res}
    out["bytes_per_launch_by_map"] = {n: {"read": res["FETCH_SIZE"]["per_map_bytes"][i],
                                          "written": res["WRITE_SIZE"]["per_map_bytes"][i],
                                          "total": res["FETCH_SIZE"]["per_map_bytes"][i]
                                          + res["WRITE_SIZE"]["per_map_bytes"][i]} for i, n in enumerate(names)}
    out["bytes_per_launch"] = round(out["bytes_per_launch_by_map"][names[0]]["total"])
    if "TCC_HIT_sum" in per and "TCC_MISS_sum" in per:
        _, gh = groups("TCC_HIT_sum")
        _, gm = groups("TCC_MISS_sum")
        out["l2"] = {f"spmv_hit_rate_{n}_map": round(float(np.sum(gh[i]) / (np.sum(gh[i]) + np.sum(gm[i]))), 4)
                     for i, n in enumerate(names)}
    with open(out_path or TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


def pmag_bench(torch, dev, mpcg, cfgs):
    """Time to solution under the max|p| rule (Sec. 4.7), per iteration and reused over K*.

    Per workload: one untimed solve, then the median of three timed ones, for the all-FP64
    map and for the rule at two settings; the per-iteration run is recorded once more to
    select K* (cg_select_reuse_interval, 10 % of upward transitions delayed at most), and the
    rule is then timed with period K*. Precision fractions are tile-iterations summed over
    the map trace; true residuals from cg_true_residual.
    """
    from gen import make_workload

    out = {"metric": "cg_time_to_solution_pmag_rule", "workloads": []}
    for cfg in cfgs:
        w = make_workload(cfg, "full")
        A = w.A
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        b = torch.from_numpy(w.b).to(dev)
        x = torch.zeros_like(b)

        def timed(S):
            S.cg_solve(b, x, w.tol, w.maxit)
            best = []
            for _ in range(3):
                torch.cuda.synchronize()
                t = time.perf_counter()
                st, K, _ = S.cg_solve(b, x, w.tol, w.maxit)
                torch.cuda.synchronize()
                best.append(time.perf_counter() - t)
            return {"status": st, "iterations": K, "time_to_solution_ms": round(float(np.median(best)) * 1e3, 3),
                    "true_residual": S.cg_true_residual(b, x)}

        rec = {"workload": w.description, "n": A.n, "nnz": A.nnz, "tol": w.tol, "maxit": w.maxit}
        S = mpcg.Solver(L, np.zeros(L.T, np.uint8), jacobi=w.jacobi)
        rec["fp64"] = timed(S)
        for name, lo, hi in (("paper_setting", w.tol / 10, w.tol), ("lo_1e-4_hi_1e-2", 1e-4, 1e-2)):
            S.cg_set_schedule_pmag(lo, hi, 1)
            r = {"lo": lo, "hi": hi, "per_iteration": timed(S)}
            ks, cnt = S.cg_get_map_trace(cap=w.maxit + 2)
            r["per_iteration"]["tile_iterations_fp64_fp32_bf16"] = \
                (cnt.sum(axis=0) / max(cnt.sum(), 1)).round(4).tolist()
            S.cg_record_column_codes(True)
            S.cg_solve(b, x, w.tol, w.maxit)
            kstar, table = mpcg.cg_select_reuse_interval(S.cg_get_column_codes(), 0.1)
            S.cg_record_column_codes(False)
            r["kstar"] = kstar
            r["delayed_upward_fraction_by_interval"] = table
            S.cg_set_schedule_pmag(lo, hi, kstar)
            r["reused"] = timed(S)
            rec[name] = r
            print(f"# cfg{cfg} max|p| {name}: per iteration {r['per_iteration']['time_to_solution_ms']} ms "
                  f"(K={r['per_iteration']['iterations']}, fractions {r['per_iteration']['tile_iterations_fp64_fp32_bf16']}), "
                  f"K*={kstar}: {r['reused']['time_to_solution_ms']} ms; FP64 map {rec['fp64']['time_to_solution_ms']} ms",
                  file=sys.stderr, flush=True)
        S.close()
        L.close()
        out["workloads"].append(rec)
    print(json.dumps(out), flush=True)


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


def spmv_probe(torch, dev, mpcg, cfgs, slices, stage_x=False):
    """Launch sequence for counter runs of the SpMV on any workload: the library's stream
    copy of 256 MiB (the scale reference of --traffic-from), then per workload and
    column-slice count (1 = unsliced, then each of `slices`) five cg_spmv launches under
    the all-FP64 map, one group of five per handle; with stage_x, one more handle per
    workload that stages x segments in LDS. With slices the combine kernel follows every
    SpMV."""
    from gen import make_workload

    src = torch.empty(COPY_BYTES // 8, dtype=torch.float64, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    mpcg.cg_stream_copy(src, dst, 8192)
    torch.cuda.synchronize()
    del src, dst
    for cfg in cfgs:
        w = make_workload(cfg, "full")
        A = w.A
        L = mpcg.cg_tilecsc_from_csr(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        m = np.zeros(L.T, np.uint8)
        xin = torch.from_numpy(np.random.default_rng(7).uniform(-1, 1, A.n)).to(dev)
        y = torch.empty_like(xin)
        for ns in [1] + list(slices) + ([-1] if stage_x else []):
            S = mpcg.Solver(L, m, col_slices=max(ns, 1), stage_x=1 if ns < 0 else 0)
            for _ in range(5):
                S.cg_spmv(xin, y)
            torch.cuda.synchronize()
            S.close()
            what = "x staged in LDS" if ns < 0 else f"{ns} column slices"
            print(f"# spmv probe: cfg{cfg}, {what}, 5 cg_spmv launches, all-FP64 map, "
                  f"algorithmic bytes {spmv_algorithmic_bytes(L, m)}", file=sys.stderr, flush=True)
        L.close()


def cpu_baseline(w, T, budget_s):
    """The CPU oracle on a bounded sample of the headline workload: its CG iterations
    under the same windowed tile rule, on one thread. The per-iteration rate is the
    difference of two runs of different lengths, so the oracle's set-up (perturbed
    operator, first residual) is excluded, as the GPU's handle set-up is; the oracle's
    layout build is excluded too."""
    from threadpoolctl import threadpool_limits

    from gen import tile_scores
    from oracle import cg as ocg, tilecsc as otc

    A = w.A
    ms = w.map_spec

    def timed(iters):
        sched = ocg.TileRuleSchedule(tile_scores(Lo.T, 2), ms["period"], ms["hi"], ms["lo"])
        t = time.time()
        r = ocg.solve(Lo, A.indptr, A.indices, A.data, w.b, sched, 0.0, iters, keep_maps=False)
        return time.time() - t, r.K

    with threadpool_limits(limits=1):
        Lo = otc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
        assert Lo.T == T
        t_a, k_a = timed(2)
        t_e, k_e = timed(7)  # estimates the time per iteration on this host
        per_it = max((t_e - t_a) / max(k_e - k_a, 1), 1e-3)
        t_b, k_b = timed(2 + max(5, int(budget_s / per_it)))
    rate = (k_b - k_a) / (t_b - t_a)
    return {"value": round(rate, 3), "unit": "CG iterations/s", "cores": 1, "kind": "oracle",
            "host_logical_cpus": os.cpu_count(),
            "sample": f"{k_b - k_a} oracle CG iterations (runs of {k_b} and {k_a} differenced, {t_b - t_a:.1f} s) "
                      f"on the full 4096^2 workload under the same windowed tile rule, one thread of a host with "
                      f"{os.cpu_count()} logical CPUs; layout build and set-up excluded"}


if __name__ == "__main__":
    main()
