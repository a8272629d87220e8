"""Parity of the HIP decode step with the CPU oracle, through the C ABI.

Every test here runs the library on the GPU and compares with the oracle on
the same seeded inputs: outputs within the row-wise tolerance of
``gpu_problem.tolerance``, the appended cache slots and every other pool byte
bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_step_amd as pkv
import workloads
from paged_kv_decode_step_amd import pool_io

import gpu_problem as gp
import problem

pytestmark = pytest.mark.gpu


def run_and_check(wl, arrs=None, *, tol=None, **run_kw):
    """Run one step on the GPU and check it fully against the oracle."""
    arrs = arrs if arrs is not None else problem.build(wl)
    ref = problem.oracle_step(wl, arrs)
    run = gp.Run(wl, arrs, **run_kw).step()
    out = run.out_f64()
    kp, vp = run.pools()
    run.close()
    kv = wl.cfg.kv_dtype
    assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"])), "K pool differs from oracle"
    assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"])), "V pool differs from oracle"
    assert np.all(np.isfinite(out))
    err = gp.row_rel_err(out, ref["out"])
    t = gp.tolerance(kv) if tol is None else tol
    assert err.max() <= t, f"max row error {err.max():.3e} > {t}"
    return out, ref, err


def small(lengths, kv="bf16", hq=32, hkv=8, d=128, bs=16, seed=3, **kw):
    io = "f32" if kv == "f32" else "bf16"
    return workloads.custom_workload(lengths, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                     block_size=bs, kv_dtype=kv, io_dtype=io,
                                     rope_theta=5.0e5, seed=seed, **kw)


# ---------------------------------------------------------------- configs
@pytest.mark.parametrize("k", [1, 2])
def test_config_full(k):
    wl = workloads.make_workload(k)
    run_and_check(wl)


@pytest.mark.parametrize("k,batch", [(3, 24), (4, 6), (5, 48)])
def test_config_leading_requests(k, batch):
    wl = workloads.make_workload(k, batch=batch)
    run_and_check(wl)


# ---------------------------------------------------------------- edge cases
def edge_lengths(kv, bs):
    t = pkv.tile_tokens()
    ls = {1, 2, 3, 4, 5, bs - 1, bs, bs + 1, 2 * bs, t - 1, t, t + 1,
          2 * t + 7, 3 * t, 4 * t + 3, 300}
    return sorted(x for x in ls if x >= 1)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64])
def test_edge_lengths(kv, d, bs):
    wl = small(edge_lengths(kv, bs), kv=kv, d=d, bs=bs, hq=16, hkv=4)
    run_and_check(wl)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_group_sizes(g):
    wl = small([1, 40, 129, 700], hq=2 * g, hkv=2)
    run_and_check(wl)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_nan_poison_in_unused_slots_blocks_and_table_tails(kv):
    wl = small([3, 17, 64, 100, 250], kv=kv, hq=16, hkv=4, max_blocks=20)
    arrs = problem.build(wl, poison=True)
    run_and_check(wl, arrs)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_many_splits_and_no_split_agree(kv):
    wl = small([2000, 50, 3333, 1, 900], kv=kv, hq=32, hkv=8)
    arrs = problem.build(wl)
    out_a, ref, _ = run_and_check(wl, arrs, waves_per_cu=16, min_units=1, piece_cost=0)
    out_b, _, _ = run_and_check(wl, arrs, waves_per_cu=4, min_units=100000)
    out_c, _, _ = run_and_check(wl, arrs, waves_per_cu=8, min_units=2, piece_cost=9)
    # later workgroups weighted down to almost nothing, and evenly weighted
    out_d, _, _ = run_and_check(wl, arrs, waves_per_cu=8, min_units=1, piece_cost=0,
                                young_weight=1)
    out_e, _, _ = run_and_check(wl, arrs, waves_per_cu=12, min_units=1, piece_cost=2,
                                young_weight=100, odd_weight=100)
    # odd workgroups weighted down to almost nothing, on top of the age weights
    out_f, _, _ = run_and_check(wl, arrs, waves_per_cu=8, min_units=1, piece_cost=3,
                                young_weight=40, odd_weight=1)
    for other in (out_b, out_c, out_d, out_e, out_f):
        assert gp.row_rel_err(out_a, other).max() <= gp.tolerance(kv)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_single_long_request_spread_over_many_wavefronts(kv):
    """One 32768-token request with one KV head: its one sequence is cut into
    over a hundred pieces, whose merge the first piece's merge wavefront
    shares by columns with the three after it."""
    run_and_check(small([32768], kv=kv, hq=8, hkv=1))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("min_units", [16, 3])
def test_long_and_short_sequences_with_many_pieces(kv, min_units):
    """Long sequences (tens to hundreds of pieces each, shared merges) next to
    short ones, at two piece sizes."""
    run_and_check(small([20000, 10, 8000, 3, 3000, 1], kv=kv, hq=16, hkv=2),
                  waves_per_cu=8, min_units=min_units)


@pytest.mark.parametrize("batch", [63, 64, 65])
def test_batches_around_the_per_wavefront_request_table(batch):
    """Up to 64 requests every wavefront builds the request table and finds
    its requests by ballot; from 65 on the workgroup builds it in LDS: both
    sides of the boundary, ragged lengths, against the oracle."""
    lens = np.random.default_rng(batch).integers(1, 700, size=batch)
    run_and_check(small(lens.tolist(), kv="bf16", hq=16, hkv=4))


def test_block_permutation_is_bit_exact_on_gpu():
    wl = small([77, 300, 5, 1200], kv="bf16")
    arrs = problem.build(wl)
    base = gp.Run(wl, arrs).step()
    out0 = base.out.clone()
    base.close()
    perm = np.random.default_rng(1).permutation(wl.num_blocks)
    a2 = dict(arrs)
    a2["k_pool"] = np.empty_like(arrs["k_pool"])
    a2["v_pool"] = np.empty_like(arrs["v_pool"])
    a2["k_pool"][perm] = arrs["k_pool"]
    a2["v_pool"][perm] = arrs["v_pool"]
    tb = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
    wl2 = workloads.Workload(wl.cfg, wl.context_lens, wl.positions, tb, wl.num_blocks, wl.seeds)
    run2 = gp.Run(wl2, a2).step()
    assert torch.equal(run2.out.view(torch.int16), out0.view(torch.int16))
    run2.close()


def test_shared_read_only_prefix_blocks():
    # requests 1 and 2 read request 0's first three blocks (a shared prefix)
    wl = small([64, 80, 100], kv="bf16", bs=16)
    tb = wl.block_tables.copy()
    tb[1, :3] = tb[0, :3]
    tb[2, :3] = tb[0, :3]
    wl2 = workloads.Workload(wl.cfg, wl.context_lens, wl.positions, tb, wl.num_blocks, wl.seeds)
    run_and_check(wl2)


def test_positions_independent_of_lengths():
    wl = small([10, 40, 90], positions=[500, 3, 77])
    run_and_check(wl, max_position=600)


def test_repeated_step_is_idempotent():
    wl = small([33, 600, 1])
    arrs = problem.build(wl)
    run = gp.Run(wl, arrs).step()
    o1 = run.out.clone()
    k1, v1 = run.pools()
    run.step()
    k2, v2 = run.pools()
    assert torch.equal(run.out.view(torch.int16), o1.view(torch.int16))
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    run.close()


def test_batch_zero_is_a_noop():
    pool = pkv.KVPool(4, 16, 2, 64, "bf16")
    pool.set_rope(1e4, 8)
    z = torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    zk = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    zi = torch.empty(0, dtype=torch.int32, device="cuda")
    zt = torch.empty(0, 1, dtype=torch.int32, device="cuda")
    pkv.decode_step(pool, z, zk, zk, zi, zt, zi, z)
    torch.cuda.synchronize()
    pool.close()


def test_tensors_off_the_pool_device_are_refused():
    pool = pkv.KVPool(4, 16, 2, 64, "bf16")
    pool.set_rope(1e4, 8)
    assert pool.device == torch.cuda.current_device()
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    one = torch.ones(1, dtype=torch.int32, device="cuda")
    tab = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_step(pool, q.cpu(), kn, kn, one - 1, tab, one, torch.empty_like(q))
    assert e.value.status == -1
    with pytest.raises(pkv.PkvError) as e:
        pool.copy_blocks(torch.tensor([[0, 1]], dtype=torch.int32))
    assert e.value.status == -1
    out = torch.empty_like(q)
    pkv.decode_step(pool, q, kn, kn, one - 1, tab, one, out)   # the same step on the device runs
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert pool.device_errors() == 0
    pool.close()


def test_largest_batch():
    """4096 requests (the most one step takes, every slot of the per-request
    prefix array in use) with short ragged contexts of 1..70 tokens."""
    rng = np.random.default_rng(41)
    lens = [int(x) for x in rng.integers(1, 71, 4096)]
    wl = small(lens, hq=4, hkv=2, d=64, seed=41)
    run_and_check(wl)


def test_missing_rope_table_is_a_state_error():
    pool = pkv.KVPool(4, 16, 2, 64, "bf16")
    q = torch.zeros(1, 4, 64, dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros(1, 2, 64, dtype=torch.bfloat16, device="cuda")
    one = torch.ones(1, dtype=torch.int32, device="cuda")
    tb = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_step(pool, q, kn, kn, one, tb, one, q)
    assert e.value.status == -5
    pool.close()


def test_default_piece_cost_follows_ring_depth():
    pool = pkv.KVPool(4, 16, 2, 128, "bf16")
    try:
        inf = pool.info()
        assert inf["ring_tiles"] >= 2
        assert inf["piece_cost"] == inf["ring_tiles"] + 2
        pool.set_tuning(0, 16, 5)
        assert pool.info()["piece_cost"] == 5
        pool.set_tuning(0, 16, -1)
        assert pool.info()["piece_cost"] == inf["ring_tiles"] + 2
        with pytest.raises(pkv.PkvError):
            pool.set_tuning(0, 16, -2)
    finally:
        pool.close()
