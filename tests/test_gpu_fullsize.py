"""Parity at the full sizes of the large ragged workloads, in the launch
configuration the benchmark times (default tuning, every wavefront the GPU
holds, pools drawn on the device).

Each full step is checked whole:

* the whole pool after the step, chunk by chunk on the device, equals the
  pool before it (redrawn from the same seeded generator) with the oracle's
  appended rows written in: the appended slots are bit-exact and nothing
  else is written.  The append depends only on the request's new K/V row,
  its position and its slot, so the oracle computes it from a one-block
  stand-in per request with the same slot and position;
* every request's output is compared with the oracle run on that request
  alone (its blocks read back after the step, which the first check has
  shown to be the pre-step blocks plus the append): every output row within
  the tolerance.  The largest row error of each workload is printed.

The workloads are the pages' ragged in-flight batches ("TensorRT-LLM Guide:
High-Throughput GPU Inference Engine", section "1. In-Flight Batching:
Continuous Iteration Scheduling").
"""
import time

import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_step_amd as pkv
import workloads
from paged_kv_decode_step_amd import pool_io

import gpu_problem as gp

pytestmark = pytest.mark.gpu


def blocks_of(wl, b):
    c = wl.cfg
    n = (int(wl.context_lens[b]) + c.block_size - 1) // c.block_size
    return wl.block_tables[b, :n].astype(np.int64)


def gather(pool, ids, kv):
    t = torch.from_numpy(ids).to(gp.DEV)
    k, v = pool_io.gather_blocks_logical(pool, t)
    return gp.codes_from_torch(k, kv), gp.codes_from_torch(v, kv)


def problem_storage(kv):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[kv]


def appended_rows(wl, io, scales):
    """The oracle's appended K/V codes of every request ([B, Hkv, D] each),
    from a stand-in with one block per request, the request's slot in it and
    its position."""
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
    return pool, chunks, scales


def check_whole_pool(wl, pool, chunks, k_app, v_app):
    """Every pool byte after the step: the pre-step codes (redrawn) with the
    appended rows of every request at (its last block, slot L - 1)."""
    c = wl.cfg
    L = wl.context_lens.astype(np.int64)
    blk = wl.block_tables[np.arange(wl.batch), (L - 1) // c.block_size].astype(np.int64)
    slot = (L - 1) % c.block_size
    ka = gp.codes_to_torch(k_app, c.kv_dtype)
    va = gp.codes_to_torch(v_app, c.kv_dtype)
    checked = 0
    for b0, kc, vc in chunks():
        n = kc.shape[0]
        sel = np.nonzero((blk >= b0) & (blk < b0 + n))[0]
        if len(sel):
            bi = torch.from_numpy(blk[sel] - b0).to(gp.DEV)
            si = torch.from_numpy(slot[sel]).to(gp.DEV)
            st = torch.from_numpy(sel).to(gp.DEV)
            kc[bi, :, si, :] = ka[st]
            vc[bi, :, si, :] = va[st]
        kg, vg = pool_io.read_logical(pool, b0, n)
        assert torch.equal(kg, kc), f"K blocks {b0}..{b0 + n - 1} differ"
        assert torch.equal(vg, vc), f"V blocks {b0}..{b0 + n - 1} differ"
        checked += len(sel)
        del kc, vc, kg, vg
    assert checked == wl.batch


def oracle_every_request(wl, pool, got, io, scales, window=0):
    """Row errors of every request against the oracle on that request alone."""
    c = wl.cfg
    errs = np.empty(wl.batch)
    t0 = time.perf_counter()
    for b in range(wl.batch):
        kb, vb = gather(pool, blocks_of(wl, b), c.kv_dtype)
        mwl, arrs = gp.mini_problem(wl, b, kb, vb, io, scales)
        ref = oracle.decode_step(
            k_pool=arrs["k_pool"], v_pool=arrs["v_pool"], kv_dtype=c.kv_dtype,
            io_dtype=c.io_dtype, q=arrs["q"], k_new=arrs["k_new"], v_new=arrs["v_new"],
            positions=mwl.positions, block_tables=mwl.block_tables,
            context_lens=mwl.context_lens, block_size=c.block_size,
            rope_theta=c.rope_theta, k_scale=arrs["k_scale"], v_scale=arrs["v_scale"],
            window=window)
        errs[b] = gp.row_rel_err(got[b], ref["out"][0]).max()
        del kb, vb, arrs, ref
    worst = int(np.argmax(errs))
    print(f"  {wl.batch} requests vs the oracle in {time.perf_counter() - t0:.1f} s: "
          f"max row error {errs.max():.3e} (request {worst}, length "
          f"{int(wl.context_lens[worst])}), median {np.median(errs):.3e}", flush=True)
    return errs


def run_full(k, window=0, tp=1):
    wl = workloads.shard_workload(k, tp) if tp > 1 else workloads.make_workload(k)
    c = wl.cfg
    print(f"full-size parity: workload {c.name}, {wl.batch} requests, {wl.num_blocks} blocks"
          + (f", window {window}" if window else ""), flush=True)
    pool, chunks, scales = load_device_pool(wl)
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
        pkv.decode_step(pool, q, kn, vn, pos, tab, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0
        got = gp.io_from_torch(out)
        assert np.all(np.isfinite(got)), "non-finite output rows"
        k_app, v_app = appended_rows(wl, io, scales)
        check_whole_pool(wl, pool, chunks, k_app, v_app)
        errs = oracle_every_request(wl, pool, got, io, scales, window)
        tol = gp.tolerance(c.kv_dtype)
        bad = np.nonzero(errs > tol)[0]
        assert len(bad) == 0, f"requests {bad[:10].tolist()} above {tol}: {errs[bad[:10]]}"
    finally:
        pool.close()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [3, 4, 5])
def test_full_size_every_request(k):
    run_full(k)


@pytest.mark.parametrize("k", [3, 5])
def test_full_size_tensor_parallel_shard(k):
    """One GPU's share of the 70B-shaped and the mixed B=512 workloads when
    their heads are split over 8 GPUs (8 query heads, 1 KV head, the same
    requests), as ``bench.py --tp 8`` runs it."""
    run_full(k, tp=8)


def test_full_size_window():
    """The mixed B=512 workload with a 4096-token window (as the benchmark
    runs it)."""
    run_full(5, window=4096)


def test_full_size_multi_token():
    """The Llama-3-8B-shaped B=64 workload with 4 new tokens per request (as
    the benchmark runs it): the whole step against the oracle's multi-token
    step on the whole batch, every output row within the tolerance and the
    whole pool bit-exact."""
    wl = workloads.make_workload(2)
    c = wl.cfg
    T = 4
    print(f"full-size multi-token parity: workload {c.name}, {T} new tokens", flush=True)
    pool, chunks, scales = load_device_pool(wl)
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
        kpre, vpre = pool_io.read_logical(pool)
        kpre, vpre = gp.codes_from_torch(kpre, c.kv_dtype), gp.codes_from_torch(vpre, c.kv_dtype)
        pkv.decode_step_multi(pool, q, kn, vn, pos, tab, lens, out)
        torch.cuda.synchronize()
        assert pool.device_errors() == 0
        got = gp.io_from_torch(out)
        t0 = time.perf_counter()
        ref = oracle.decode_step_multi(
            k_pool=kpre, v_pool=vpre, kv_dtype=c.kv_dtype, io_dtype="bf16", q=io["q"],
            k_new=io["k_new"], v_new=io["v_new"], positions=first,
            block_tables=wl.block_tables, context_lens=wl.context_lens,
            block_size=c.block_size, rope_theta=c.rope_theta)
        err = gp.row_rel_err(got, ref["out"])
        print(f"  {wl.batch} x {T} queries vs the oracle in {time.perf_counter() - t0:.1f} s: "
              f"max row error {err.max():.3e}", flush=True)
        assert err.max() <= gp.tolerance(c.kv_dtype)
        kp, vp = pool_io.read_logical(pool)
        assert np.array_equal(gp.bits(gp.codes_from_torch(kp, c.kv_dtype)), gp.bits(ref["k_pool"]))
        assert np.array_equal(gp.bits(gp.codes_from_torch(vp, c.kv_dtype)), gp.bits(ref["v_pool"]))
    finally:
        pool.close()
