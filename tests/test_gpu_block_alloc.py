"""GPU: whole-block copies in the pool, and decode steps driven by the host
block allocator (sequences added, forked to share a prefix, released, a late
arrival) against the dense-history oracle.  Every step's output is compared
with the oracle row by row; at the end every live sequence's cache, gathered
through its final block list from the device pool, must equal its history
bit for bit."""
import numpy as np
import pytest
import torch

import gpu_problem as gp
import oracle
import paged_kv_decode_step_amd as pkv
from paged_kv_decode_step_amd import pool_io
from problem import NAN_CODE

pytestmark = pytest.mark.gpu


def kv_codes(rng, shape, kv, scale=None):
    x = rng.standard_normal(shape).astype(np.float32)
    if kv == "bf16":
        return oracle.bf16_bits_from_f32(x)
    if kv == "fp8":
        return oracle.fp8_encode(x * oracle.fp8_inverse_scale(scale)[None, :, None, None]
                                 if x.ndim == 4 else x * oracle.fp8_inverse_scale(scale)[:, None, None])
    return x


def io_vals(rng, shape, io):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if io == "f32" else oracle.bf16_bits_from_f32(x)


@pytest.mark.parametrize("kv,d,bs", [("bf16", 128, 16), ("fp8", 128, 32), ("f32", 64, 16)])
def test_copy_blocks_is_bit_exact(kv, d, bs):
    rng = np.random.default_rng(11)
    nb, hkv = 24, 2
    scale = np.array([0.01, 0.02], np.float32)
    k = kv_codes(rng, (nb, hkv, bs, d), kv, scale)
    v = kv_codes(rng, (nb, hkv, bs, d), kv, scale)
    pool = pkv.KVPool(nb, bs, hkv, d, kv)
    try:
        pool_io.write_logical(pool, gp.codes_to_torch(k, kv), gp.codes_to_torch(v, kv))
        pairs = [(3, 10), (5, 11), (0, 23), (7, 7)]
        pool.copy_blocks(torch.tensor(pairs, dtype=torch.int32, device=gp.DEV))
        torch.cuda.synchronize()
        ek, ev = k.copy(), v.copy()
        for s, t in pairs:
            ek[t], ev[t] = k[s], v[s]
        gk, gv = pool_io.read_logical(pool)
        assert np.array_equal(gp.bits(gp.codes_from_torch(gk, kv)), gp.bits(ek))
        assert np.array_equal(gp.bits(gp.codes_from_torch(gv, kv)), gp.bits(ev))
        assert pool.device_errors() == 0
        # an id outside the pool is skipped and flagged; the others still copy
        pool.copy_blocks(torch.tensor([(1, 30), (2, 12)], dtype=torch.int32, device=gp.DEV))
        torch.cuda.synchronize()
        assert pool.device_errors() & 1
        ek[12], ev[12] = k[2], v[2]
        gk, gv = pool_io.read_logical(pool)
        assert np.array_equal(gp.bits(gp.codes_from_torch(gk, kv)), gp.bits(ek))
        assert np.array_equal(gp.bits(gp.codes_from_torch(gv, kv)), gp.bits(ev))
    finally:
        pool.close()


@pytest.mark.parametrize("kv,io", [("bf16", "bf16"), ("fp8", "bf16")])
def test_decode_steps_with_the_block_allocator(kv, io):
    rng = np.random.default_rng(21)
    hkv, hq, d, bs, nb, maxb, theta = 2, 8, 128, 16, 64, 8, 1.0e4
    k_scale = np.array([0.012, 0.02], np.float32) if kv == "fp8" else None
    v_scale = np.array([0.015, 0.01], np.float32) if kv == "fp8" else None
    alloc = pkv.BlockAllocator(nb, bs, 8)
    hist = oracle.DenseHistories(kv, io, theta, k_scale, v_scale)
    pool = pkv.KVPool(nb, bs, hkv, d, kv)
    host_k = np.empty((nb, hkv, bs, d), dtype=kv_codes(rng, (1, 1, 1, 1), kv, k_scale).dtype)
    host_k[...] = NAN_CODE[kv]
    host_v = host_k.copy()

    def add_prompt(length):
        s = alloc.add(length)
        kc = kv_codes(rng, (hkv, length, d), kv, k_scale)
        vc = kv_codes(rng, (hkv, length, d), kv, v_scale)
        hist.add(s, kc, vc)
        _, blocks = alloc.info(s)
        for t in range(length):
            host_k[blocks[t // bs], :, t % bs] = kc[:, t]
            host_v[blocks[t // bs], :, t % bs] = vc[:, t]
        return s, blocks

    try:
        pool.set_rope(theta, 4096)
        if kv == "fp8":
            pool.set_fp8_scales(k_scale, v_scale)
        seqs = [add_prompt(n)[0] for n in (20, 33, 7, 16)]
        pool_io.write_logical(pool, gp.codes_to_torch(host_k, kv), gp.codes_to_torch(host_v, kv))
        for parent in (seqs[0], seqs[0], seqs[3]):   # two share a half-full block, one a full one
            c = alloc.fork(parent)
            hist.fork(parent, c)
            seqs.append(c)
        n_copies = 0
        for step in range(7):
            if step == 3:                            # one finishes, one arrives
                alloc.release(seqs[1])
                hist.release(seqs[1])
                seqs.remove(seqs[1])
                s, blocks = add_prompt(5)
                for blk in blocks:
                    pool_io.write_logical(pool, gp.codes_to_torch(host_k[blk:blk + 1], kv),
                                          gp.codes_to_torch(host_v[blk:blk + 1], kv),
                                          first_block=blk)
                seqs.append(s)
            batch = [int(x) for x in rng.permutation(seqs)]
            if step == 5:
                batch = batch[:-2]                   # not every sequence steps every iteration
            tables, lens, pos, copies = alloc.prepare_step(batch, maxb)
            n_copies += len(copies)
            if len(copies):
                pool.copy_blocks(torch.from_numpy(np.ascontiguousarray(copies)).to(gp.DEV))
            b = len(batch)
            q, kn, vn = io_vals(rng, (b, hq, d), io), io_vals(rng, (b, hkv, d), io), io_vals(rng, (b, hkv, d), io)
            out = torch.full((b, hq, d), float("nan"), dtype=torch.bfloat16, device=gp.DEV)
            pkv.decode_step(pool, gp.io_to_torch(q, io), gp.io_to_torch(kn, io), gp.io_to_torch(vn, io),
                            torch.from_numpy(pos).to(gp.DEV), torch.from_numpy(tables).to(gp.DEV),
                            torch.from_numpy(lens).to(gp.DEV), out)
            torch.cuda.synchronize()
            ref = hist.step(batch, q, kn, vn, pos)
            err = gp.row_rel_err(gp.io_from_torch(out), ref)
            assert err.max() <= gp.tolerance(kv), (step, err.max())
        assert n_copies >= 2                          # the two forks of the half-full block
        assert pool.device_errors() == 0
        gk, gv = pool_io.read_logical(pool)
        gk, gv = gp.codes_from_torch(gk, kv), gp.codes_from_torch(gv, kv)
        for s in seqs:
            length, blocks = alloc.info(s)
            got_k = np.stack([gk[blocks[t // bs], :, t % bs] for t in range(length)], axis=1)
            got_v = np.stack([gv[blocks[t // bs], :, t % bs] for t in range(length)], axis=1)
            assert np.array_equal(gp.bits(got_k), gp.bits(hist.k[s])), s
            assert np.array_equal(gp.bits(got_v), gp.bits(hist.v[s])), s
    finally:
        pool.close()
        alloc.close()
