"""GPU: sliding-window attention (kv_pool_set_window) against the oracle's
window, with every slot below each request's window, and every unused slot,
poisoned with NaN: a window tile read or weighted by mistake shows up.  The
pool after the step must equal the oracle's bit for bit (the append is not
windowed)."""
import numpy as np
import pytest

import gpu_problem as gp
import oracle
import paged_kv_decode_step_amd as pkv
import problem
import workloads
from problem import NAN_CODE

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 31, 33, 48, 67, 300, 1000, 2000]


def windowed_case(kv, d, bs, window, seed):
    wl = workloads.custom_workload(LENS, n_q_heads=4 * 2, n_kv_heads=2, head_dim=d,
                                   block_size=bs, kv_dtype=kv,
                                   io_dtype="f32" if kv == "f32" else "bf16",
                                   rope_theta=1.0e4, seed=seed)
    arrs = problem.build(wl, poison=True)
    nan = NAN_CODE[kv]
    for b, L in enumerate(wl.context_lens):
        L = int(L)
        for t in range(max(0, L - window)):
            blk = int(wl.block_tables[b, t // bs])
            arrs["k_pool"][blk, :, t % bs] = nan
            arrs["v_pool"][blk, :, t % bs] = nan
    c = wl.cfg
    ref = oracle.decode_step(
        k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=kv, io_dtype=c.io_dtype,
        q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"], positions=wl.positions,
        block_tables=wl.block_tables, context_lens=wl.context_lens, block_size=bs,
        rope_theta=c.rope_theta, k_scale=arrs["k_scale"], v_scale=arrs["v_scale"],
        window=window)
    return wl, arrs, ref


@pytest.mark.parametrize("kv,d,bs", [("bf16", 128, 16), ("fp8", 128, 32), ("f32", 64, 16),
                                     ("bf16", 64, 64)])
@pytest.mark.parametrize("window", [1, 7, 16, 17, 33, 100, 1000])
def test_window_matches_the_oracle(kv, d, bs, window):
    wl, arrs, ref = windowed_case(kv, d, bs, window, seed=60 + window)
    for tuning in ({}, {"waves_per_cu": 16, "min_units": 1, "piece_cost": 0}):
        run = gp.Run(wl, arrs, **tuning)
        try:
            run.pool.set_window(window)
            run.step()
            out = run.out_f64()
            assert np.all(np.isfinite(out))
            err = gp.row_rel_err(out, ref["out"])
            assert err.max() <= gp.tolerance(kv), (tuning, err.max())
            kp, vp = run.pools()
            assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"]))
            assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"]))
            assert run.pool.device_errors() == 0
        finally:
            run.close()


def test_negative_window_is_refused():
    wl, arrs, _ = windowed_case("bf16", 128, 16, 7, seed=99)
    run = gp.Run(wl, arrs)
    try:
        with pytest.raises(pkv.PkvError) as e:
            run.pool.set_window(-1)
        assert e.value.status == -1
        assert run.pool.info()["window"] == 0
    finally:
        run.close()
