"""Run one decode step with the timeline build of the library and print its
parity against the oracle and the per-wavefront records, as one JSON line.
Started as a child process by test_gpu_timeline.py (a process loads one
build of the library)."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import paged_kv_decode_step_amd as pkv  # noqa: E402

pkv.load_library(pkv.TIMELINE_LIB_PATH)

import gpu_problem as gp  # noqa: E402
import problem  # noqa: E402
import workloads  # noqa: E402


def main():
    lens = np.random.default_rng(41).integers(1, 3000, size=40)
    wl = workloads.custom_workload(lens, n_q_heads=32, n_kv_heads=8, head_dim=128,
                                   block_size=16, kv_dtype="bf16", io_dtype="bf16",
                                   rope_theta=5.0e5, seed=41)
    arrs = problem.build(wl)
    ref = problem.oracle_step(wl, arrs)
    run = gp.Run(wl, arrs).step()
    err = float(gp.row_rel_err(run.out_f64(), ref["out"]).max())
    rec = run.pool.read_timeline()
    n_waves = int(run.pool.info()["n_waves"])
    run.close()
    print(json.dumps({"err": err, "tol": gp.tolerance("bf16"), "n_waves": n_waves,
                      "tiles_expected": int(((lens + 15) // 16).sum()) * 8,
                      "records": rec.astype(np.int64).tolist()}), flush=True)


if __name__ == "__main__":
    main()
