"""GPU: the pool's own calls and the kernel's handling of unusual cache data.

* an out-of-range block id for a request's new slot raises device flag 0 and
  writes nothing (every other request's output and the whole pool as the
  oracle computes them without that request);
* ``kv_pool_layout`` and ``kv_pool_rope_table`` describe the pool the
  kernels read (strides against the header's layout, the table bit-equal to
  the host-built one), and the RoPE table keeps its address when a new
  table fits; a graph captured before the table grows still replays;
* FP8 caches: the NaN codes read as NaN, and every finite E4M3 code is
  widened exactly (a zero query averages the values, which the kernel then
  sums exactly in fp32)."""
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


def small(lengths, kv="bf16", hq=8, hkv=2, d=128, bs=16, seed=21):
    io = "f32" if kv == "f32" else "bf16"
    return workloads.custom_workload(lengths, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                     block_size=bs, kv_dtype=kv, io_dtype=io,
                                     rope_theta=5.0e5, seed=seed)


def sub_batch(wl, arrs, keep):
    """The same step with only the requests `keep` (same pool, same blocks)."""
    wl2 = workloads.Workload(wl.cfg, wl.context_lens[keep], wl.positions[keep],
                             wl.block_tables[keep], wl.num_blocks, wl.seeds)
    a2 = dict(arrs)
    for w in ("q", "k_new", "v_new"):
        a2[w] = arrs[w][keep]
    return wl2, a2


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_bad_block_id_for_the_new_slot_writes_nothing(kv):
    wl = small([40, 33, 17, 5], kv=kv)
    bs = wl.cfg.block_size
    tables = wl.block_tables.copy()
    # block 0 belongs to request 0, so a write redirected to block 0 would
    # corrupt a live request
    b0 = int(tables[0, 0])
    where = np.argwhere(tables == 0)
    if len(where):
        tables[tuple(where[0])] = b0
    tables[0, 0] = 0
    wl = workloads.Workload(wl.cfg, wl.context_lens, wl.positions, tables, wl.num_blocks,
                            wl.seeds)
    arrs = problem.build(wl)
    bad = 1
    L = int(wl.context_lens[bad])
    bad_tables = tables.copy()
    bad_tables[bad, (L - 1) // bs] = wl.num_blocks          # one past the pool
    keep = np.array([b for b in range(wl.batch) if b != bad])
    wl_ok, arrs_ok = sub_batch(wl, arrs, keep)
    ref = problem.oracle_step(wl_ok, arrs_ok)
    run = gp.Run(wl, arrs, tables=bad_tables).step()
    try:
        assert run.pool.device_errors() & 1
        out = run.out_f64()
        kp, vp = run.pools()
        assert np.array_equal(gp.bits(kp), gp.bits(ref["k_pool"])), "K pool written"
        assert np.array_equal(gp.bits(vp), gp.bits(ref["v_pool"])), "V pool written"
        err = gp.row_rel_err(out[keep], ref["out"])
        assert err.max() <= gp.tolerance(kv)
    finally:
        run.close()


def test_layout_describes_the_pool():
    wl = small([40, 17], bs=32)
    c = wl.cfg
    pool = pkv.KVPool(wl.num_blocks, c.block_size, c.n_kv_heads, c.head_dim, c.kv_dtype)
    try:
        lay, info = pool.layout(), pool.info()
        t = 16 * c.head_dim * 2
        assert lay["tile_bytes"] == t == info["tile_bytes"]
        assert lay["byte_strides"] == (c.n_kv_heads * 2 * t, 2 * t, t)
        assert lay["k_base"] == info["k_base"] and lay["v_base"] == info["v_base"]
        assert lay["byte_strides"][0] * wl.num_blocks == info["k_bytes"]
        # one element written through the logical view lands where the
        # strides and the header's in-tile formula put it
        k = torch.zeros(wl.num_blocks, c.n_kv_heads, c.block_size, c.head_dim,
                        dtype=torch.int16, device=gp.DEV)
        n, h, slot, d = 3, 1, 21, 77
        k[n, h, slot, d] = 0x1234
        pool_io.write_logical(pool, k, torch.zeros_like(k))
        raw = pool.k_storage().view(-1).view(torch.int16)
        st = lay["byte_strides"]
        x = 8                                     # bf16 dims per 16-byte row
        t16 = slot % 16
        byte = (n * st[0] + h * st[1] + (slot // 16) * st[2]
                + ((d // x) * 16 + t16) * 16 + (d % x) * 2)
        assert int(raw[byte // 2]) == 0x1234
        assert int((raw != 0).sum()) == 1
    finally:
        pool.close()


def test_rope_table_call_and_its_address():
    pool = pkv.KVPool(8, 16, 2, 64, "bf16")
    try:
        with pytest.raises(pkv.PkvError) as e:
            pool.rope_table()
        assert e.value.status == -5
        pool.set_rope(1.0e4, 64)
        c, s = pool.rope_table()
        hc, hs = pkv.rope_table_host(1.0e4, 64, 64)
        assert np.array_equal(c.cpu().numpy(), hc) and np.array_equal(s.cpu().numpy(), hs)
        ptr = pool.info()["rope_cos"]
        pool.set_rope(5.0e5, 64)                  # same size: rewritten in place
        c, _ = pool.rope_table()
        assert pool.info()["rope_cos"] == ptr
        assert np.array_equal(c.cpu().numpy(), pkv.rope_table_host(5.0e5, 64, 64)[0])
        pool.set_rope(1.0e4, 16)                  # smaller: in place too
        assert pool.info()["rope_cos"] == ptr
        assert pool.rope_table()[0].shape == (16, 32)
        pool.set_rope(1.0e4, 4096)                # larger: a new buffer
        assert pool.info()["rope_cos"] != ptr
        c, s = pool.rope_table()
        hc, hs = pkv.rope_table_host(1.0e4, 64, 4096)
        assert np.array_equal(c.cpu().numpy(), hc) and np.array_equal(s.cpu().numpy(), hs)
    finally:
        pool.close()


def test_graph_captured_before_the_table_grows_still_replays():
    wl = small([300, 17, 64])
    arrs = problem.build(wl)
    run = gp.Run(wl, arrs)
    try:
        run.step()
        eager = run.out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pkv.decode_step(run.pool, run.q, run.k_new, run.v_new, run.positions, run.tables,
                            run.lens, run.out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pkv.decode_step(run.pool, run.q, run.k_new, run.v_new, run.positions, run.tables,
                            run.lens, run.out)
        old = run.pool.info()["rope_cos"]
        run.pool.set_rope(wl.cfg.rope_theta, 1 << 16)        # grows: the old table is kept
        assert run.pool.info()["rope_cos"] != old
        for _ in range(3):
            run.out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(run.out, eager)
        del g
    finally:
        run.close()


def test_fp8_nan_codes_read_as_nan():
    wl = small([70, 40, 33], kv="fp8", seed=5)
    arrs = problem.build(wl)
    bs = wl.cfg.block_size
    # request 0: a NaN key code in token 20 of KV head 1; request 1: a NaN
    # value code (negative) in token 7, head 0, dim 5; request 2 untouched
    blk, off = int(wl.block_tables[0, 20 // bs]), 20 % bs
    arrs["k_pool"][blk, 1, off, 9] = 0x7F
    blk, off = int(wl.block_tables[1, 7 // bs]), 7 % bs
    arrs["v_pool"][blk, 0, off, 5] = 0xFF
    ref = problem.oracle_step(wl, arrs)
    run = gp.Run(wl, arrs).step()
    try:
        out = run.out_f64()
        nan_ref = np.isnan(ref["out"])
        assert nan_ref[0].any() and nan_ref[1].any() and not nan_ref[2].any()
        assert np.array_equal(np.isnan(out), nan_ref)
        rows = ~nan_ref.any(axis=-1)
        assert gp.row_rel_err(out[rows], ref["out"][rows]).max() <= gp.tolerance("fp8")
        # request 1's other dims stay finite and correct
        o1, r1 = out[1][:, [d for d in range(128) if d != 5]], ref["out"][1][:, [d for d in range(128) if d != 5]]
        assert np.all(np.isfinite(o1))
        assert np.max(np.abs(o1 - r1)) <= gp.tolerance("fp8") * np.max(np.abs(r1))
        kp, vp = run.pools()
        assert np.array_equal(kp, ref["k_pool"]) and np.array_equal(vp, ref["v_pool"])
    finally:
        run.close()


def fp8_binade_codes(d, t):
    """E4M3 code of token t, dim d: dim d walks the eight mantissas of the
    binade (sign, exponent) = divmod(d % 32, 16), seven in the two binades
    whose last code is NaN."""
    k = d % 32
    n = 7 if k in (15, 31) else 8
    return 8 * k + t % n


def test_fp8_values_widen_exactly():
    """Every finite E4M3 code in the V cache (subnormals included), a zero
    query (all weights 1) and unit scales: the output is the mean of each
    dim's 256 values.  A dim's values share one binade, so their sum needs
    at most 12 significant bits: the kernel sums them exactly in fp32,
    divides by 256 exactly and rounds once to bf16, so its output equals the
    oracle's exact mean rounded to bf16, bit for bit."""
    L = 256
    wl = small([L], kv="fp8", hq=2, hkv=1, seed=9)
    arrs = problem.build(wl)
    bs = wl.cfg.block_size
    dims = np.arange(128)
    for t in range(L - 1):
        blk, off = int(wl.block_tables[0, t // bs]), t % bs
        arrs["v_pool"][blk, 0, off, :] = [fp8_binade_codes(d, t) for d in dims]
    arrs["k_scale"] = np.ones(1, np.float32)
    arrs["v_scale"] = np.ones(1, np.float32)
    arrs["q"] = np.zeros_like(arrs["q"])
    # the new token (slot 255) continues the pattern: its bf16 values are
    # E4M3 values, which encode with scale 1 to exactly those codes
    codes = np.array([fp8_binade_codes(d, L - 1) for d in dims])
    vals = np.array([oracle.fp8_code_value(c) for c in codes], np.float32)
    arrs["v_new"] = oracle.bf16_bits_from_f32(vals[None, None, :])
    ref = problem.oracle_step(wl, arrs)
    assert np.array_equal(ref["v_app"][0, 0], codes)
    assert np.all(ref["out"] == ref["out"].astype(np.float32))    # the mean is exact in fp32
    run = gp.Run(wl, arrs).step()
    try:
        got = run.out.view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.bf16_bits_from_f32(ref["out"].astype(np.float32))
        assert np.array_equal(got, want)
        kp, vp = run.pools()
        assert np.array_equal(vp, ref["v_pool"])
    finally:
        run.close()
