"""GPU: seeded random decode steps across the supported space against the
oracle.

Each case draws a cache type (bf16, fp8, f32), head dim (64, 128), block size
(16, 32, 64), KV heads (1-8) and group size (1-16), a batch of 1-80 requests
(either side of the 64-request boundary of the prologue) whose lengths mix
single tokens, short and long contexts (up to 1500 tokens, so that the oracle
finishes each case in seconds), an attention window or none, one or
several new tokens, and a tuning of the partition (the default, few or many
wavefronts per compute unit, no start cost).  Every output row is checked
within the cache type's tolerance and the whole pool bit for bit (the
appended slots included); no range flag may be raised.
"""
import numpy as np
import pytest
import torch

import gpu_problem as gp
import oracle
import paged_kv_decode_step_amd as pkv
import problem
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 100


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    kv = ["bf16", "fp8", "f32"][rng.integers(3)]
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 8, 16]))
    if hkv * g > 64:            # keeps the oracle's side of a case within seconds
        g = 64 // hkv
    tq = 1
    if kv != "f32" and rng.random() < 0.3:
        tq = int(rng.choice([t for t in (2, 3, 4, 8) if g * t <= 16] or [1]))
    window = int(rng.choice([0, 0, 1, 16, 17, 100, 700])) if tq == 1 else 0
    batch = int(rng.choice([1, 2, 3, 7, 20, 63, 64, 65, 80]))
    kind = rng.random(batch)
    lens = np.where(kind < 0.15, rng.integers(1, 4, batch),
                    np.where(kind < 0.75, rng.integers(1, 600, batch), rng.integers(600, 1500, batch)))
    lens = np.maximum(lens, tq)
    tuning = [{}, {"waves_per_cu": 4}, {"waves_per_cu": 12, "min_units": 3},
              {"min_units": 1, "piece_cost": 0}][rng.integers(4)]
    return dict(kv=kv, d=d, bs=bs, hkv=hkv, hq=hkv * g, tq=tq, window=window,
                lens=[int(x) for x in lens], tuning=tuning, seed=seed)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_step_matches_the_oracle(seed):
    c = draw(seed)
    print(f"case {seed}: " + ", ".join(f"{k}={v}" for k, v in c.items() if k != "lens")
          + f", batch={len(c['lens'])}", flush=True)
    kv, tq = c["kv"], c["tq"]
    io = "f32" if kv == "f32" else "bf16"
    wl = workloads.custom_workload(c["lens"], n_q_heads=c["hq"], n_kv_heads=c["hkv"],
                                   head_dim=c["d"], block_size=c["bs"], kv_dtype=kv,
                                   io_dtype=io, rope_theta=1.0e4, seed=500 + seed)
    arrs = problem.build(wl, poison=tq == 1)
    if tq == 1:
        ref = oracle.decode_step(
            k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=kv, io_dtype=io,
            q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"], positions=wl.positions,
            block_tables=wl.block_tables, context_lens=wl.context_lens,
            block_size=c["bs"], rope_theta=1.0e4, k_scale=arrs["k_scale"],
            v_scale=arrs["v_scale"], window=c["window"])
        run = gp.Run(wl, arrs, **c["tuning"])
        try:
            run.pool.set_window(c["window"])
            run.step()
            got = run.out_f64()
            kp, vp = run.pools()
            flags = run.pool.device_errors()
        finally:
            run.close()
    else:
        rng = np.random.default_rng(700 + seed)
        b, hq, hkv, d = len(c["lens"]), c["hq"], c["hkv"], c["d"]
        bits = lambda shape: oracle.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))
        q, kn, vn = bits((b, tq, hq, d)), bits((b, tq, hkv, d)), bits((b, tq, hkv, d))
        pos = np.array(c["lens"], np.int32) - tq + 3
        ref = oracle.decode_step_multi(
            k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=kv, io_dtype="bf16", q=q,
            k_new=kn, v_new=vn, positions=pos, block_tables=wl.block_tables,
            context_lens=wl.context_lens, block_size=c["bs"], rope_theta=1.0e4,
            k_scale=arrs["k_scale"], v_scale=arrs["v_scale"])
        run = gp.Run(wl, arrs, max_position=int(pos.max()) + tq + 1, **c["tuning"])
        try:
            out = torch.full((b, tq, hq, d), float("nan"), dtype=torch.bfloat16, device=gp.DEV)
            pkv.decode_step_multi(run.pool, gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"),
                                  gp.io_to_torch(vn, "bf16"), torch.from_numpy(pos).to(gp.DEV),
                                  run.tables, run.lens, out)
            torch.cuda.synchronize()
            got = gp.io_from_torch(out)
            kp, vp = run.pools()
            flags = run.pool.device_errors()
        finally:
            run.close()
    assert flags == 0
    assert np.all(np.isfinite(got))
    err = gp.row_rel_err(got, ref["out"])
    assert err.max() <= gp.tolerance(kv), float(err.max())
    assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"]))
    assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"]))
