"""Parity at the full sizes of the large ragged workloads, in the launch
configuration the benchmark times (default tuning, every wavefront the GPU
holds, pools drawn on the device).

A whole step of these workloads is gigabytes of cache, more than the oracle
can take on the host in seconds, so each step is checked three ways:

* sampled requests (the longest and shortest, the first and last, the
  median and seeded picks) are compared whole with the oracle run on that
  request alone: every output row within the tolerance, every byte of the
  request's blocks (the appended slot included) bit-exact;
* the appended slot of every request is bit-exact: the append depends only
  on the request's new K/V row, its position and the slot, so the oracle
  computes it from a one-block stand-in with the same slot and position;
* every output row is finite.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_step_amd as pkv
import workloads
from paged_kv_decode_step_amd import pool_io

import gpu_problem as gp

pytestmark = pytest.mark.gpu


def sampled_requests(wl, n_random=5, seed=11):
    lens = wl.context_lens
    order = np.argsort(lens, kind="stable")
    picks = {0, wl.batch - 1, int(order[0]), int(order[-1]), int(order[-2]),
             int(order[len(order) // 2])}
    rng = np.random.default_rng(seed)
    picks.update(int(x) for x in rng.choice(wl.batch, size=n_random, replace=False))
    return sorted(picks)


def blocks_of(wl, b):
    c = wl.cfg
    n = (int(wl.context_lens[b]) + c.block_size - 1) // c.block_size
    return wl.block_tables[b, :n].astype(np.int64)


def gather(pool, ids, kv):
    t = torch.from_numpy(ids).to(gp.DEV)
    k, v = pool_io.gather_blocks_logical(pool, t)
    return gp.codes_from_torch(k, kv), gp.codes_from_torch(v, kv)


def appended_slots_expected(wl, io, scales):
    """The oracle's appended K/V codes of every request, from a stand-in
    with one block per request, the request's slot in it and its position."""
    c = wl.cfg
    B, bs = wl.batch, c.block_size
    lens = wl.context_lens.astype(np.int64)
    stand_lens = ((lens - 1) % bs + 1).astype(np.int32)
    shape = (B, c.n_kv_heads, bs, c.head_dim)
    dt = problem_storage(c.kv_dtype)
    ref = oracle.decode_step(
        k_pool=np.zeros(shape, dt), v_pool=np.zeros(shape, dt), kv_dtype=c.kv_dtype,
        io_dtype=c.io_dtype, q=io["q"], k_new=io["k_new"], v_new=io["v_new"],
        positions=wl.positions, block_tables=np.arange(B, dtype=np.int32)[:, None],
        context_lens=stand_lens, block_size=bs, rope_theta=c.rope_theta,
        k_scale=None if scales is None else scales[0],
        v_scale=None if scales is None else scales[1])
    return ref["k_app"], ref["v_app"]


def problem_storage(kv):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[kv]


@pytest.mark.parametrize("k", [3, 4, 5])
def test_full_size_sampled(k):
    wl = workloads.make_workload(k)
    c = wl.cfg
    print(f"full-size parity: workload {c.name}, {wl.batch} requests, "
          f"{wl.num_blocks} blocks", flush=True)
    chunks, scales = gp.device_pool_codes(wl)
    pool = pkv.KVPool(wl.num_blocks, c.block_size, c.n_kv_heads, c.head_dim, c.kv_dtype)
    try:
        pool.set_rope(c.rope_theta, wl.max_position)
        if scales is not None:
            pool.set_fp8_scales(*scales)
        for b0, kc, vc in chunks():
            pool_io.write_logical(pool, kc, vc, b0)
            del kc, vc
        io = gp.host_io_arrays(wl)
        q = gp.io_to_torch(io["q"], c.io_dtype)
        kn = gp.io_to_torch(io["k_new"], c.io_dtype)
        vn = gp.io_to_torch(io["v_new"], c.io_dtype)
        pos = torch.from_numpy(wl.positions.astype(np.int32)).to(gp.DEV)
        tab = torch.from_numpy(np.ascontiguousarray(wl.block_tables, np.int32)).to(gp.DEV)
        lens = torch.from_numpy(wl.context_lens.astype(np.int32)).to(gp.DEV)
        out = torch.full_like(q, float("nan"))

        picks = sampled_requests(wl)
        before = {b: gather(pool, blocks_of(wl, b), c.kv_dtype) for b in picks}
        torch.cuda.synchronize()

        pkv.decode_step(pool, q, kn, vn, pos, tab, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0

        got = gp.io_from_torch(out)
        assert np.all(np.isfinite(got)), "non-finite output rows"

        # every request's appended slot
        k_app, v_app = appended_slots_expected(wl, io, scales)
        L = wl.context_lens.astype(np.int64)
        last_blk = wl.block_tables[np.arange(wl.batch), (L - 1) // c.block_size].astype(np.int64)
        kl, vl = gather(pool, last_blk, c.kv_dtype)
        slot = (L - 1) % c.block_size
        rows = np.arange(wl.batch)
        assert np.array_equal(gp.bits(kl[rows, :, slot, :]), gp.bits(k_app)), "appended K differs"
        assert np.array_equal(gp.bits(vl[rows, :, slot, :]), gp.bits(v_app)), "appended V differs"

        # sampled requests, whole
        tol = gp.tolerance(c.kv_dtype)
        for b in picks:
            kb, vb = before[b]
            mwl, arrs = gp.mini_problem(wl, b, kb, vb, io, scales)
            ref = oracle.decode_step(
                k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=c.kv_dtype,
                io_dtype=c.io_dtype, q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"],
                positions=mwl.positions, block_tables=mwl.block_tables,
                context_lens=mwl.context_lens, block_size=c.block_size,
                rope_theta=c.rope_theta, k_scale=arrs["k_scale"], v_scale=arrs["v_scale"])
            err = gp.row_rel_err(got[b], ref["out"][0]).max()
            print(f"  request {b}: length {int(wl.context_lens[b])}, max row error {err:.2e}",
                  flush=True)
            assert err <= tol, f"request {b}: max row error {err:.3e} > {tol}"
            ka, va = gather(pool, blocks_of(wl, b), c.kv_dtype)
            assert np.array_equal(gp.bits(ka), gp.bits(ref["k_pool"])), f"request {b}: K blocks"
            assert np.array_equal(gp.bits(va), gp.bits(ref["v_pool"])), f"request {b}: V blocks"
            del kb, vb, ka, va, ref, arrs
    finally:
        pool.close()
        torch.cuda.empty_cache()


def load_device_pool(wl):
    c = wl.cfg
    chunks, scales = gp.device_pool_codes(wl)
    pool = pkv.KVPool(wl.num_blocks, c.block_size, c.n_kv_heads, c.head_dim, c.kv_dtype)
    pool.set_rope(c.rope_theta, wl.max_position)
    if scales is not None:
        pool.set_fp8_scales(*scales)
    for b0, kc, vc in chunks():
        pool_io.write_logical(pool, kc, vc, b0)
        del kc, vc
    return pool, scales


def test_full_size_window():
    """The mixed B=512 workload with a 4096-token window (as the benchmark
    runs it): sampled requests whole against the oracle's window, all
    appended slots bit-exact, every row finite."""
    wl = workloads.make_workload(5)
    c = wl.cfg
    window = 4096
    print(f"full-size window parity: workload {c.name}, window {window}", flush=True)
    pool, scales = load_device_pool(wl)
    try:
        pool.set_window(window)
        io = gp.host_io_arrays(wl)
        q = gp.io_to_torch(io["q"], c.io_dtype)
        kn = gp.io_to_torch(io["k_new"], c.io_dtype)
        vn = gp.io_to_torch(io["v_new"], c.io_dtype)
        pos = torch.from_numpy(wl.positions.astype(np.int32)).to(gp.DEV)
        tab = torch.from_numpy(np.ascontiguousarray(wl.block_tables, np.int32)).to(gp.DEV)
        lens = torch.from_numpy(wl.context_lens.astype(np.int32)).to(gp.DEV)
        out = torch.full_like(q, float("nan"))
        picks = sampled_requests(wl)
        before = {b: gather(pool, blocks_of(wl, b), c.kv_dtype) for b in picks}
        pkv.decode_step(pool, q, kn, vn, pos, tab, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0
        got = gp.io_from_torch(out)
        assert np.all(np.isfinite(got)), "non-finite output rows"
        k_app, v_app = appended_slots_expected(wl, io, scales)
        L = wl.context_lens.astype(np.int64)
        last_blk = wl.block_tables[np.arange(wl.batch), (L - 1) // c.block_size].astype(np.int64)
        kl, vl = gather(pool, last_blk, c.kv_dtype)
        slot = (L - 1) % c.block_size
        rows = np.arange(wl.batch)
        assert np.array_equal(gp.bits(kl[rows, :, slot, :]), gp.bits(k_app)), "appended K differs"
        assert np.array_equal(gp.bits(vl[rows, :, slot, :]), gp.bits(v_app)), "appended V differs"
        tol = gp.tolerance(c.kv_dtype)
        for b in picks:
            kb, vb = before[b]
            mwl, arrs = gp.mini_problem(wl, b, kb, vb, io, scales)
            ref = oracle.decode_step(
                k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=c.kv_dtype,
                io_dtype=c.io_dtype, q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"],
                positions=mwl.positions, block_tables=mwl.block_tables,
                context_lens=mwl.context_lens, block_size=c.block_size,
                rope_theta=c.rope_theta, k_scale=arrs["k_scale"], v_scale=arrs["v_scale"],
                window=window)
            err = gp.row_rel_err(got[b], ref["out"][0]).max()
            print(f"  request {b}: length {int(wl.context_lens[b])}, max row error {err:.2e}",
                  flush=True)
            assert err <= tol, f"request {b}: max row error {err:.3e} > {tol}"
            del kb, vb, ref, arrs
    finally:
        pool.close()


def test_full_size_multi_token():
    """The Llama-3-8B-shaped B=64 workload with 4 new tokens per request (as
    the benchmark runs it): sampled requests whole against the oracle's
    multi-token step (outputs within the tolerance, the request's blocks
    bit-exact), every row finite."""
    wl = workloads.make_workload(2)
    c = wl.cfg
    T = 4
    print(f"full-size multi-token parity: workload {c.name}, {T} new tokens", flush=True)
    pool, scales = load_device_pool(wl)
    try:
        rng = np.random.default_rng(2024)
        enc = oracle.bf16_bits_from_f32
        io = {"q": enc(rng.standard_normal((wl.batch, T, c.n_q_heads, c.head_dim)).astype(np.float32)),
              "k_new": enc(rng.standard_normal((wl.batch, T, c.n_kv_heads, c.head_dim)).astype(np.float32)),
              "v_new": enc(rng.standard_normal((wl.batch, T, c.n_kv_heads, c.head_dim)).astype(np.float32))}
        q, kn, vn = (gp.io_to_torch(io[w], "bf16") for w in ("q", "k_new", "v_new"))
        first = (wl.context_lens - T).astype(np.int32)
        pos = torch.from_numpy(first).to(gp.DEV)
        tab = torch.from_numpy(np.ascontiguousarray(wl.block_tables, np.int32)).to(gp.DEV)
        lens = torch.from_numpy(wl.context_lens.astype(np.int32)).to(gp.DEV)
        out = torch.full_like(q, float("nan"))
        picks = sampled_requests(wl)
        before = {b: gather(pool, blocks_of(wl, b), c.kv_dtype) for b in picks}
        pkv.decode_step_multi(pool, q, kn, vn, pos, tab, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0
        got = gp.io_from_torch(out)
        assert np.all(np.isfinite(got)), "non-finite output rows"
        tol = gp.tolerance(c.kv_dtype)
        for b in picks:
            kb, vb = before[b]
            n = kb.shape[0]
            ref = oracle.decode_step_multi(
                k_pool=kb, v_pool=vb, kv_dtype=c.kv_dtype, io_dtype="bf16",
                q=io["q"][b:b + 1], k_new=io["k_new"][b:b + 1], v_new=io["v_new"][b:b + 1],
                positions=first[b:b + 1], block_tables=np.arange(n, dtype=np.int32)[None, :],
                context_lens=wl.context_lens[b:b + 1], block_size=c.block_size,
                rope_theta=c.rope_theta)
            err = gp.row_rel_err(got[b], ref["out"][0]).max()
            print(f"  request {b}: length {int(wl.context_lens[b])}, max row error {err:.2e}",
                  flush=True)
            assert err <= tol, f"request {b}: max row error {err:.3e} > {tol}"
            ka, va = gather(pool, blocks_of(wl, b), c.kv_dtype)
            assert np.array_equal(gp.bits(ka), gp.bits(ref["k_pool"])), f"request {b}: K blocks"
            assert np.array_equal(gp.bits(va), gp.bits(ref["v_pool"])), f"request {b}: V blocks"
    finally:
        pool.close()
