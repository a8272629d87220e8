"""GPU: steps with several new tokens per request (decode_step_multi) against
the oracle's causal multi-token step: outputs row by row within the
tolerance, the whole pool bit for bit (all new tokens appended), with and
without forced many-way splits; plus the unsupported combinations."""
import numpy as np
import pytest
import torch

import gpu_problem as gp
import oracle
import paged_kv_decode_step_amd as pkv
import problem
import workloads

pytestmark = pytest.mark.gpu


def case(kv, d, bs, hq, hkv, tq, seed):
    # every context holds at least the T new tokens
    lens = [tq, tq + 1] + [L for L in (15, 16, 17, 33, 100, 1000, 2000) if L > tq + 1]
    wl = workloads.custom_workload(lens, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block_size=bs,
                                   kv_dtype=kv, io_dtype="bf16", rope_theta=1.0e4, seed=seed)
    arrs = problem.build(wl, poison=True)
    rng = np.random.default_rng(seed)
    b = len(lens)
    io = lambda shape: oracle.bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))
    q, kn, vn = io((b, tq, hq, d)), io((b, tq, hkv, d)), io((b, tq, hkv, d))
    pos = np.array(lens, np.int32) - tq + 5
    ref = oracle.decode_step_multi(
        k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=kv, io_dtype="bf16", q=q,
        k_new=kn, v_new=vn, positions=pos, block_tables=wl.block_tables,
        context_lens=wl.context_lens, block_size=bs, rope_theta=1.0e4,
        k_scale=arrs["k_scale"], v_scale=arrs["v_scale"])
    return wl, arrs, (q, kn, vn, pos), ref


@pytest.mark.parametrize("kv,d,bs,hq,hkv,tq", [
    ("bf16", 128, 16, 8, 2, 2), ("bf16", 128, 16, 8, 2, 3), ("bf16", 128, 16, 8, 2, 4),
    ("fp8", 128, 32, 32, 8, 4), ("bf16", 64, 64, 4, 4, 16), ("bf16", 128, 16, 16, 2, 2),
    ("fp8", 64, 16, 4, 2, 5)])
def test_multi_token_step_matches_the_oracle(kv, d, bs, hq, hkv, tq):
    wl, arrs, (q, kn, vn, pos), ref = case(kv, d, bs, hq, hkv, tq, seed=80 + tq)
    for tuning in ({}, {"waves_per_cu": 16, "min_units": 1, "piece_cost": 0}):
        run = gp.Run(wl, arrs, max_position=int(pos.max()) + tq + 1, **tuning)
        try:
            out = torch.full((len(pos), tq, hq, d), float("nan"), dtype=torch.bfloat16, device=gp.DEV)
            pkv.decode_step_multi(run.pool, gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"),
                                  gp.io_to_torch(vn, "bf16"), torch.from_numpy(pos).to(gp.DEV),
                                  run.tables, run.lens, out)
            torch.cuda.synchronize()
            got = gp.io_from_torch(out)
            assert np.all(np.isfinite(got))
            err = gp.row_rel_err(got, ref["out"])
            assert err.max() <= gp.tolerance(kv), (tuning, float(err.max()))
            kp, vp = run.pools()
            assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"]))
            assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"]))
            assert run.pool.device_errors() == 0
        finally:
            run.close()


def test_one_new_token_is_decode_step():
    wl, arrs, (q, kn, vn, pos), ref = case("bf16", 128, 16, 8, 2, 1, seed=90)
    run = gp.Run(wl, arrs, max_position=int(pos.max()) + 2)
    try:
        out = torch.empty((len(pos), 1, 8, 128), dtype=torch.bfloat16, device=gp.DEV)
        pkv.decode_step_multi(run.pool, gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"),
                              gp.io_to_torch(vn, "bf16"), torch.from_numpy(pos).to(gp.DEV),
                              run.tables, run.lens, out)
        torch.cuda.synchronize()
        assert gp.row_rel_err(gp.io_from_torch(out), ref["out"]).max() <= gp.tolerance("bf16")
    finally:
        run.close()


def test_unsupported_multi_token_combinations_are_refused():
    wl, arrs, (q, kn, vn, pos), _ = case("bf16", 128, 16, 32, 2, 2, seed=91)   # G 16 x 2 > 16
    run = gp.Run(wl, arrs, max_position=4096)
    try:
        out = torch.empty((len(pos), 2, 32, 128), dtype=torch.bfloat16, device=gp.DEV)
        args = (gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"), gp.io_to_torch(vn, "bf16"),
                torch.from_numpy(pos).to(gp.DEV), run.tables, run.lens, out)
        with pytest.raises(pkv.PkvError) as e:
            pkv.decode_step_multi(run.pool, *args)
        assert e.value.status == -2
    finally:
        run.close()
    wl, arrs, (q, kn, vn, pos), _ = case("bf16", 128, 16, 8, 2, 2, seed=92)
    run = gp.Run(wl, arrs, max_position=4096)
    try:
        run.pool.set_window(64)
        out = torch.empty((len(pos), 2, 8, 128), dtype=torch.bfloat16, device=gp.DEV)
        with pytest.raises(pkv.PkvError) as e:
            pkv.decode_step_multi(run.pool, gp.io_to_torch(q, "bf16"), gp.io_to_torch(kn, "bf16"),
                                  gp.io_to_torch(vn, "bf16"), torch.from_numpy(pos).to(gp.DEV),
                                  run.tables, run.lens, out)
        assert e.value.status == -2
    finally:
        run.close()
