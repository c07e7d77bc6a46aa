"""Write the oracle's full-size CG results for the GPU parity tests.

Runs only ``gen`` and ``oracle`` (never the HIP library) and stores, per
workload and per map (the all-FP64 map and the workload's own map), the
iteration count, status, recurrence history and the FP64-recomputed true
residual, plus the map trace and, where the layout is cheap to hash, SHA-256
digests of the canonical Tile-CSC arrays.

Usage: python tests/golden/make_golden.py CFG [CFG ...]
       python tests/golden/make_golden.py --only LABEL CFG   (one map: fp64 or mixed,
                                                               written to a part file)
       python tests/golden/make_golden.py --merge CFG        (part files -> the result)
Each run is single-threaded and takes from about a minute (cfg2) to more
than an hour (cfg5, two 5000-iteration solves); the two maps of one
workload can run as two processes with --only, then --merge.
"""

import hashlib
import json
import os
import sys
import time

for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(v, "1")

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from gen import make_workload, static_map, tile_scores  # noqa: E402
from oracle import cg, tilecsc as tc  # noqa: E402


def sha(a, dtype):
    return hashlib.sha256(np.ascontiguousarray(a, dtype=dtype).tobytes()).hexdigest()


def layout_digest(L):
    return dict(tile_row_ptr=sha(L.tile_row_ptr, np.int64), tile_col_idx=sha(L.tile_col_idx, np.int32),
                tile_nnz_ptr=sha(L.tile_nnz_ptr, np.int64), row_idx=sha(L.row_idx, np.uint8),
                col_local=sha(L.col_local, np.uint8))


def run(cfg, scale="full", only=None):
    t0 = time.time()
    w = make_workload(cfg, scale)
    A = w.A
    L = tc.build(A.n, A.indptr, A.indices, A.data, w.R, w.C)
    print(f"cfg{cfg}: n={A.n} nnz={A.nnz} T={L.T} built in {time.time() - t0:.1f}s", flush=True)
    out = dict(workload=w.name, description=w.description, input_hash=w.input_hash(), n=A.n,
               nnz=A.nnz, T=L.T, R=w.R, C=w.C, tol=w.tol, maxit=w.maxit, jacobi=w.jacobi,
               map_spec={k: (list(v) if isinstance(v, tuple) else v) for k, v in w.map_spec.items()},
               layout=layout_digest(L), runs={})
    scores = tile_scores(L.T, 2)
    static = static_map(scores, w.map_spec.get("frac_bf16", 0.2), w.map_spec.get("frac_fp32", 0.3)) \
        if w.map_spec["kind"] == "static" else None
    specs = [("fp64", dict(kind="fp64"))]
    if w.map_spec["kind"] != "fp64":
        specs.append(("mixed", w.map_spec))
    if only is not None:
        specs = [s for s in specs if s[0] == only]
    for label, spec in specs:
        t1 = time.time()
        sched = cg.schedule_for(spec, L, scores=scores, static=static)
        res = cg.solve(L, A.indptr, A.indices, A.data, w.b, sched, w.tol, w.maxit,
                       jacobi=w.jacobi, keep_maps=False)
        el = time.time() - t1
        wins = []
        for (k, counts, _m) in res.windows:
            wins.append(dict(k=int(k), counts=[int(c) for c in counts]))
        if spec["kind"] in ("static", "magnitude"):
            m = sched.map
            wins[0]["sha"] = sha(m, np.uint8)
        out["runs"][label] = dict(K=res.K, status=res.status, hist=[float(h) for h in res.hist],
                                  true_residual=res.true_residual, seconds=el, windows=wins)
        print(f"  {label}: K={res.K} {res.status} rho={res.hist[-1]:.3e} "
              f"true={res.true_residual:.3e} ({el:.1f}s)", flush=True)
    path = os.path.join(HERE, f"cg_cfg{cfg}_{scale}.json" if only is None else f"cg_cfg{cfg}_{scale}.{only}.part")
    with open(path, "w") as f:
        json.dump(out, f)
    print(f"wrote {path}", flush=True)


def merge(cfg, scale="full"):
    """Combine the per-map part files of one workload into its result file."""
    parts = [os.path.join(HERE, f"cg_cfg{cfg}_{scale}.{label}.part") for label in ("fp64", "mixed")]
    docs = [json.load(open(p)) for p in parts if os.path.exists(p)]
    if not docs:
        raise SystemExit("no part files")
    out = docs[0]
    for d in docs[1:]:
        if d["input_hash"] != out["input_hash"] or d["layout"] != out["layout"]:
            raise SystemExit("part files disagree on the inputs")
        out["runs"].update(d["runs"])
    path = os.path.join(HERE, f"cg_cfg{cfg}_{scale}.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print(f"wrote {path} with runs {sorted(out['runs'])}", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:]
    if args and args[0] == "--only":
        run(int(args[2]), only=args[1])
    elif args and args[0] == "--merge":
        merge(int(args[1]))
    else:
        for a in args:
            run(int(a))
