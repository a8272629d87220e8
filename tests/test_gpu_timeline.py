"""The timeline build (libpkv_timeline.so): the same kernels with
per-wavefront phase stamps.  Its steps match the oracle like the normal
build's, every wavefront's record is whole and ordered, and the tiles each
wavefront recorded are those the host replay of the partition gives it (a
full step, a small one spread over the first workgroups, a windowed one);
the normal build refuses to read a timeline."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import paged_kv_decode_step_amd as pkv

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_normal_build_has_no_timeline():
    import gpu_problem as gp
    import problem
    import workloads
    wl = workloads.custom_workload([5, 40], n_q_heads=8, n_kv_heads=2, head_dim=128,
                                   block_size=16, kv_dtype="bf16", io_dtype="bf16", seed=3)
    run = gp.Run(wl, problem.build(wl)).step()
    try:
        with pytest.raises(pkv.PkvError, match="UNSUPPORTED"):
            run.pool.read_timeline()
    finally:
        run.close()


@pytest.mark.skipif(not os.path.exists(pkv.TIMELINE_LIB_PATH),
                    reason="timeline build not present (python -m paged_kv_decode_step_amd.build --timeline)")
def test_timeline_build_matches_oracle_and_records_every_wavefront():
    res = subprocess.run([sys.executable, os.path.join(HERE, "timeline_child.py")],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    cases = json.loads(res.stdout.strip().splitlines()[-1])
    assert len(cases) == 3
    for d in cases:
        assert d["err"] <= d["tol"], d["err"]
        rec = np.array(d["records"], dtype=np.int64)
        assert rec.shape == (d["n_waves"], 8)
        stamps, tiles = rec[:, :6], rec[:, 6]
        assert (stamps[:, 0] > 0).all()                  # every wavefront recorded its entry
        assert (np.diff(stamps, axis=1) >= 0).all()      # phases in order
        assert tiles.sum() == d["tiles_expected"]        # every tile belongs to one wavefront
        # the device's partition is the host replay's, wavefront by wavefront
        assert np.array_equal(tiles, np.array(d["tiles_per_wave_expected"]))
        assert ((rec[:, 7] >> 32) & 0xF).max() < 8       # XCC ids
        span = (stamps[:, 5].max() - stamps[:, 0].min()) / 100.0
        assert 0.0 < span < 10_000.0                     # microseconds, one small step
    # the small step uses more wavefronts than min_units alone would give it
    small = np.array(cases[1]["records"])[:, 6]
    assert (small > 0).sum() > 24


@pytest.mark.skipif(not os.path.exists(pkv.TIMELINE_LIB_PATH),
                    reason="timeline build not present (python -m paged_kv_decode_step_amd.build --timeline)")
def test_bench_timeline_mode_summarises_a_step():
    """``bench.py --timeline`` on the small ragged workload: one JSON line
    whose phases are ordered and whose wavefronts with tiles hold them all."""
    root = os.path.dirname(HERE)
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--timeline", "--config", "1",
                          "--steps", "2", "--warmup", "2"],
                         capture_output=True, text=True, timeout=300, cwd=root)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    d = json.loads(res.stdout.strip().splitlines()[-1])
    assert d["workload"].startswith("tiny_ragged") and len(d["steps"]) == 2
    for s in d["steps"]:
        assert s["active"] >= 1 and s["span_us"] > 0
        assert all(v >= 0 for v in s["phase_us_p50"].values())
        e = s["end_us"]
        assert e["p10"] <= e["p50"] <= e["p90"] <= e["max"] == s["span_us"]
