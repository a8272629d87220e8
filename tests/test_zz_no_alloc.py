"""GPU: decode_step_noalloc, the entry point whose split-K workspace is the
library's fixed per-device array, against decode_step (the pool's own
workspace) and the oracle, through the C ABI.  Two calls in a row share the
array, the second with a smaller batch: each must give decode_step's
outputs and pools bit for bit (same kernels, same partition) and the
oracle's within the tolerance."""
import numpy as np
import pytest
import torch

import paged_kv_decode_step_amd as pkv
import workloads

import gpu_problem as gp
import problem

pytestmark = pytest.mark.gpu


def both_ways(wl):
    arrs = problem.build(wl)
    ref = problem.oracle_step(wl, arrs)
    a = gp.Run(wl, arrs)
    b = gp.Run(wl, arrs)
    try:
        pkv.decode_step_noalloc(a.pool, a.q, a.k_new, a.v_new, a.positions, a.tables, a.lens,
                                a.out)
        b.step()
        torch.cuda.synchronize()
        assert a.pool.device_errors() == 0
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16)), \
            "outputs differ from decode_step"
        ka, va = a.pools()
        kb, vb = b.pools()
        assert np.array_equal(gp.bits(ka), gp.bits(kb)) and np.array_equal(gp.bits(va), gp.bits(vb))
        assert np.array_equal(gp.bits(ka), gp.bits(ref["k_pool"]))
        assert np.array_equal(gp.bits(va), gp.bits(ref["v_pool"]))
        err = gp.row_rel_err(a.out_f64(), ref["out"]).max()
        assert err <= gp.tolerance(wl.cfg.kv_dtype), err
        return a.pool.info()["n_waves"]
    finally:
        a.close()
        b.close()


def test_noalloc_matches_decode_step_twice_second_smaller():
    # the Llama-3-8B-shaped batch: 64 requests, long sequences split over
    # many wavefronts, so the partial states and headers fill the array
    n_waves = both_ways(workloads.make_workload(2))
    print(f"first call: {n_waves} wavefronts", flush=True)
    # then a smaller ragged batch on the same array (stale contents of the
    # first call must not leak into it)
    small = workloads.custom_workload([1, 40, 700, 1500, 3, 2049], n_q_heads=32, n_kv_heads=8,
                                      head_dim=128, block_size=16, kv_dtype="bf16",
                                      io_dtype="bf16", rope_theta=5.0e5, seed=77)
    both_ways(small)


def test_noalloc_refuses_more_wavefronts_than_the_array_holds():
    pool = pkv.KVPool(64, 16, 8, 128, "bf16")
    try:
        pool.set_rope(1.0e4, 64)
        cus = pool.info()["n_waves"] // 8
        if 16 * cus <= 2048:
            pytest.skip("this GPU has too few compute units to exceed 2048 wavefronts")
        pool.set_tuning(16)
        z = torch.zeros(1, 8, 128, dtype=torch.bfloat16, device=gp.DEV)
        i = torch.zeros(1, dtype=torch.int32, device=gp.DEV)
        with pytest.raises(pkv.PkvError) as e:
            pkv.decode_step_noalloc(pool, z, z, z, i, i.view(1, 1), i + 1, z.clone())
        assert e.value.status == -2
    finally:
        pool.close()
