"""GPU: the PKV_DEBUG=1 validation of device-resident arguments.  Every
rejected case is caught on the host before anything is launched: lengths
out of range, a block that receives new tokens of two requests, and (with
several new tokens) a block receiving new tokens that another request
reads.  A valid step still matches the oracle."""
import os

import numpy as np
import pytest
import torch

import gpu_problem as gp
import paged_kv_decode_step_amd as pkv
import problem
import workloads

pytestmark = pytest.mark.gpu

DEVICE_DATA = -6


@pytest.fixture
def debug_env():
    old = os.environ.get("PKV_DEBUG")
    os.environ["PKV_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["PKV_DEBUG"]
    else:
        os.environ["PKV_DEBUG"] = old


def small():
    wl = workloads.custom_workload([40, 17, 5], n_q_heads=8, n_kv_heads=2, head_dim=128,
                                   block_size=16, kv_dtype="bf16", io_dtype="bf16", seed=70)
    return wl, problem.build(wl)


def test_debug_accepts_a_valid_step(debug_env):
    wl, arrs = small()
    ref = problem.oracle_step(wl, arrs)
    run = gp.Run(wl, arrs).step()
    try:
        assert gp.row_rel_err(run.out_f64(), ref["out"]).max() <= gp.tolerance("bf16")
    finally:
        run.close()


def test_debug_rejects_bad_device_data(debug_env):
    wl, arrs = small()
    run = gp.Run(wl, arrs)
    try:
        def call(lens=None, tables=None):
            pkv.decode_step(run.pool, run.q, run.k_new, run.v_new, run.positions,
                            run.tables if tables is None else tables,
                            run.lens if lens is None else lens, run.out)

        bad = run.lens.clone()
        bad[1] = 0
        with pytest.raises(pkv.PkvError) as e:
            call(lens=bad)
        assert e.value.status == DEVICE_DATA
        bad = run.lens.clone()
        bad[2] = int(run.tables.shape[1]) * 16 + 1
        with pytest.raises(pkv.PkvError) as e:
            call(lens=bad)
        assert e.value.status == DEVICE_DATA
        # request 2's last block handed to request 1 as well: two appends into one block
        t = run.tables.clone()
        t[1, 1] = t[2, 0]
        with pytest.raises(pkv.PkvError) as e:
            call(tables=t)
        assert e.value.status == DEVICE_DATA
        # request 0 reads (block 0 of) request 2's appended block
        t = run.tables.clone()
        t[0, 0] = t[2, 0]
        with pytest.raises(pkv.PkvError) as e:
            call(tables=t)
        assert e.value.status == DEVICE_DATA
    finally:
        run.close()


def test_debug_checks_every_block_receiving_new_tokens(debug_env):
    wl, arrs = small()                 # lens 40, 17, 5 with block 16
    run = gp.Run(wl, arrs)
    try:
        tq, b = 3, 3
        q = torch.zeros(b, tq, 8, 128, dtype=torch.bfloat16, device=gp.DEV)
        kn = torch.zeros(b, tq, 2, 128, dtype=torch.bfloat16, device=gp.DEV)
        vn = torch.zeros_like(kn)
        out = torch.empty_like(q)
        pos = (run.lens - tq).contiguous()
        # request 1 (17 tokens) gets new tokens at slots 14, 15 (block 0) and 16 (block 1);
        # request 0 reading request 1's block 0 is refused
        t = run.tables.clone()
        t[0, 1] = t[1, 0]
        with pytest.raises(pkv.PkvError) as e:
            pkv.decode_step_multi(run.pool, q, kn, vn, pos, t, run.lens, out)
        assert e.value.status == DEVICE_DATA
        # a context shorter than its new tokens
        short = run.lens.clone()
        short[2] = tq - 1
        with pytest.raises(pkv.PkvError) as e:
            pkv.decode_step_multi(run.pool, q, kn, vn, pos, run.tables, short, out)
        assert e.value.status == DEVICE_DATA
        torch.cuda.synchronize()
        assert run.pool.device_errors() == 0
    finally:
        run.close()
