"""Run decode steps with the timeline build of the library and print, for
each, its parity against the oracle, the per-wavefront records and the
tiles per wavefront of the host replay of the partition, as one JSON line.
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
import oracle  # noqa: E402
import problem  # noqa: E402
import workloads  # noqa: E402


def expected_tiles(pool, wl):
    """Tiles per wavefront of the host replay of the partition, with the
    pool's own parameters (decode_step's weight threshold is 256 units)."""
    inf = pool.info()
    c = wl.cfg
    pieces, _ = pkv.plan_host(wl.context_lens, c.n_kv_heads, wl.block_tables.shape[1] * c.block_size,
                              inf["n_waves"], max(inf["min_units"], inf["piece_cost"] + 1),
                              inf["piece_cost"], inf["n_first"], 100, inf["young_weight_pct"],
                              256, weight_odd=inf["odd_weight_pct"], window=inf["window"])
    tiles = np.zeros(inf["n_waves"], dtype=np.int64)
    np.add.at(tiles, pieces[:, 0], pieces[:, 4] - pieces[:, 3])
    return tiles


def case(lens, hq, hkv, window, seed):
    wl = workloads.custom_workload(lens, n_q_heads=hq, n_kv_heads=hkv, head_dim=128,
                                   block_size=16, kv_dtype="bf16", io_dtype="bf16",
                                   rope_theta=5.0e5, seed=seed)
    arrs = problem.build(wl)
    ref = oracle.decode_step(
        k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype="bf16", io_dtype="bf16",
        q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"], positions=wl.positions,
        block_tables=wl.block_tables, context_lens=wl.context_lens, block_size=16,
        rope_theta=5.0e5, window=window)
    run = gp.Run(wl, arrs)
    run.pool.set_window(window)
    run.step()
    err = float(gp.row_rel_err(run.out_f64(), ref["out"]).max())
    rec = run.pool.read_timeline()
    n_waves = int(run.pool.info()["n_waves"])
    exp = expected_tiles(run.pool, wl)
    run.close()
    lens = np.asarray(lens)
    first = np.where((window > 0) & (lens > window), (lens - window) // 16, 0)
    return {"err": err, "tol": gp.tolerance("bf16"), "n_waves": n_waves,
            "tiles_expected": int((np.maximum((lens + 15) // 16, 1) - first).sum()) * hkv,
            "tiles_per_wave_expected": exp.tolist(),
            "records": rec.astype(np.int64).tolist()}


def main():
    rng = np.random.default_rng(41)
    cases = [
        # 40 requests: every wavefront active
        case(rng.integers(1, 3000, size=40), 32, 8, 0, 41),
        # 3 requests: a small step, spread over the first workgroups
        case([138, 1012, 84], 16, 4, 0, 42),
        # 64 requests with a 256-token window
        case(np.random.default_rng(43).integers(64, 2048, size=64), 32, 8, 256, 43),
    ]
    print(json.dumps(cases), flush=True)


if __name__ == "__main__":
    main()
