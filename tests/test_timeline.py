"""The per-wavefront timeline summary bench.py prints (``--timeline``),
on hand-made records whose phases, ends and per-XCD figures are known."""
import numpy as np

import bench


def record(start, phases, tiles, xcc, cu=0):
    """One wavefront: entry at `start` ticks (100 MHz), then the five phase
    lengths in ticks; HW_ID with the compute unit in bits 11:8."""
    stamps = [start]
    for d in phases:
        stamps.append(stamps[-1] + d)
    return stamps + [tiles, (xcc << 32) | (cu << 8)]


def test_summary_of_known_records():
    base = 5_000_000_000
    rec = np.array([
        record(base + 0, [100, 200, 300, 2000, 50], 10, 0),      # ends at 2650 ticks = 26.5 us
        record(base + 100, [100, 200, 300, 2200, 50], 11, 1),    # ends at 2950 = 29.5 us
        record(base + 200, [120, 180, 280, 1800, 70], 9, 0),     # ends at 2650 = 26.5 us
        record(base + 50, [0, 0, 0, 0, 0], 0, 1),                # no tiles
    ], dtype=np.uint64)
    s = bench.timeline_summary(rec)
    assert s["waves"] == 4 and s["active"] == 3
    assert s["span_us"] == 29.5
    assert s["start_us"]["max"] == 2.0
    assert s["phase_us_p50"] == {"request_table": 1.0, "tile_range": 2.0, "ring_fill": 3.0,
                                 "tile_loop": 20.0, "writes_and_exit": 0.5}
    assert s["end_us"]["p50"] == 26.5 and s["end_us"]["max"] == 29.5
    # busy: (26.5 + 28.5 + 24.5) / (3 * 29.5)
    assert abs(s["busy_fraction"] - round(79.5 / 88.5, 4)) < 1e-12
    assert s["per_xcd"][0]["waves"] == 2 and s["per_xcd"][1]["waves"] == 1
    assert s["per_xcd"][1]["end_max"] == 29.5
    assert s["per_xcd"][0]["start_p50"] == 1.0                  # entries at 0 and 2 us
    assert abs(s["per_xcd"][1]["tiles_per_us_p50"] - round(11 / 22.0, 3)) < 1e-12
    assert s["tiles_p50"] == 10.0
