"""Block allocator (host, no GPU): the library against the plain reference in
``oracle.block_alloc`` on seeded random operation sequences (block ids,
tables, copies and errors exactly equal), their shared invariants, a
token-level simulation of the pool under the copy-on-write pairs, and the
dense-history oracle pinned to ``oracle.decode_step``."""
import numpy as np
import pytest

import oracle
import paged_kv_decode_step_amd as pkv

INVALID, OOM = -1, -3


def lib_call(fn, *a):
    """Run a library call; returns (result, None) or (None, status)."""
    try:
        return fn(*a), None
    except pkv.PkvError as e:
        return None, e.status


def ref_call(fn, *a):
    try:
        return fn(*a), None
    except oracle.AllocError as e:
        return None, {"invalid": INVALID, "oom": OOM}[e.kind]


def assert_same_state(lib, ref, num_blocks):
    live = sorted(ref.seqs)
    fb, ls = lib.stats()
    assert (fb, ls) == (len(ref.free), len(live))
    for s in live:
        length, blocks = lib.info(s)
        assert length == ref.seqs[s][0] and blocks == ref.seqs[s][1]
    assert [lib.refcount(b) for b in range(num_blocks)] == ref.ref


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_reference_on_random_operations(seed):
    rng = np.random.default_rng(seed)
    nb, bs, ms = int(rng.integers(8, 40)), int(rng.choice([1, 2, 4, 16])), int(rng.integers(2, 9))
    maxb = int(rng.integers(2, 12))
    lib = pkv.BlockAllocator(nb, bs, ms)
    ref = oracle.BlockAllocator(nb, bs, ms)
    for _ in range(300):
        live = sorted(ref.seqs)
        op = rng.choice(["add", "fork", "release", "step", "step", "step"])
        if op == "add":
            n = int(rng.integers(0, 3 * bs + 2))
            a, ea = lib_call(lib.add, n)
            b, eb = ref_call(ref.add, n)
            assert (a, ea) == (b, eb)
        elif op == "fork":
            p = int(rng.choice(live)) if live and rng.random() < 0.9 else int(rng.integers(0, ms + 1))
            a, ea = lib_call(lib.fork, p)
            b, eb = ref_call(ref.fork, p)
            assert (a, ea) == (b, eb)
        elif op == "release":
            s = int(rng.choice(live)) if live and rng.random() < 0.9 else int(rng.integers(-1, ms + 1))
            a, ea = lib_call(lib.release, s)
            b, eb = ref_call(ref.release, s)
            assert ea == eb
        else:
            k = int(rng.integers(0, len(live) + 1))
            ids = list(rng.permutation(live)[:k])
            if ids and rng.random() < 0.05:
                ids.append(ids[0])                     # a repeated id
            mc = int(rng.integers(0, 4)) if rng.random() < 0.2 else len(ids)
            a, ea = lib_call(lib.prepare_step, ids, maxb, mc)
            b, eb = ref_call(ref.prepare_step, ids, maxb, mc)
            assert ea == eb
            if ea is None:
                t, l, p, c = a
                rt, rl, rp, rc = b
                assert t.tolist() == rt and l.tolist() == rl and p.tolist() == rp
                assert [tuple(x) for x in c.tolist()] == rc
        assert_same_state(lib, ref, nb)


@pytest.mark.parametrize("impl", ["library", "reference"])
@pytest.mark.parametrize("seed", range(6))
def test_copy_on_write_keeps_every_sequence_its_own_tokens(impl, seed):
    """Simulate the pool at token level: each slot holds a tag (sequence of
    origin, token index).  Prompts are written into a sequence's blocks, a
    step first applies the copy pairs and then writes each new token at its
    slot through the table.  Every live sequence must read back exactly its
    own history, a forked one the parent's prefix and then its own tokens;
    reference counts must equal the holders and blocks must be conserved."""
    rng = np.random.default_rng(100 + seed)
    nb, bs, ms, maxb = 48, int(rng.choice([2, 4, 16])), 8, 10
    if impl == "library":
        lib = pkv.BlockAllocator(nb, bs, ms)
        add, fork, release = lib.add, lib.fork, lib.release
        step = lambda ids: lib.prepare_step(ids, maxb, len(ids))
        info = lib.info
        refc = lambda: [lib.refcount(b) for b in range(nb)]
    else:
        ref = oracle.BlockAllocator(nb, bs, ms)
        add, fork, release = ref.add, ref.fork, ref.release
        step = lambda ids: tuple(np.asarray(x, dtype=np.int32).reshape(-1, *shape)
                                 for x, shape in zip(ref.prepare_step(ids, maxb, len(ids)),
                                                     [(maxb,), (), (), (2,)]))
        info = lambda s: (ref.seqs[s][0], list(ref.seqs[s][1]))
        refc = lambda: list(ref.ref)
    pool = np.full((nb, bs), -1, dtype=np.int64)       # tag per slot
    hist = {}
    tag = [0]

    def new_tag():
        tag[0] += 1
        return tag[0]

    for it in range(120):
        live = sorted(hist)
        r = rng.random()
        try:
            if r < 0.15 or not live:
                n = int(rng.integers(0, 2 * bs + 3))
                s = add(n)
                _, blocks = info(s)
                hist[s] = [new_tag() for _ in range(n)]
                for t, tg in enumerate(hist[s]):
                    pool[blocks[t // bs], t % bs] = tg
            elif r < 0.3:
                p = int(rng.choice(live))
                c = fork(p)
                hist[c] = list(hist[p])
            elif r < 0.4:
                s = int(rng.choice(live))
                release(s)
                del hist[s]
            else:
                ids = [int(x) for x in rng.permutation(live)[:int(rng.integers(1, len(live) + 1))]]
                tables, lens, pos, copies = step(ids)
                for src, dst in copies:
                    pool[dst] = pool[src]
                for i, s in enumerate(ids):
                    L = int(lens[i])
                    assert L == len(hist[s]) + 1 and int(pos[i]) == L - 1
                    blk = int(tables[i][(L - 1) // bs])
                    tg = new_tag()
                    pool[blk, (L - 1) % bs] = tg
                    hist[s].append(tg)
                    # the written block is held by this sequence alone
                    assert refc()[blk] == 1
        except (pkv.PkvError, oracle.AllocError) as e:
            status = getattr(e, "status", None)
            kind = getattr(e, "kind", None)
            assert status == OOM or kind == "oom" or status == INVALID or kind == "invalid"
            continue
        held = [0] * nb
        for s in hist:
            length, blocks = info(s)
            assert length == len(hist[s]) and len(blocks) == -(-length // bs)
            got = [int(pool[blocks[t // bs], t % bs]) for t in range(length)]
            assert got == hist[s]
            for b in blocks:
                held[b] += 1
        assert held == refc()


def test_errors_leave_the_allocator_unchanged():
    lib = pkv.BlockAllocator(6, 4, 4)
    a = lib.add(8)                   # blocks 0, 1 (full)
    b = lib.fork(a)
    c = lib.add(6)                   # blocks 2, 3 (3 half full)
    d = lib.fork(c)
    snap = lambda: (lib.stats(), [lib.info(s) for s in (a, b, c, d)],
                    [lib.refcount(x) for x in range(6)])
    before = snap()
    with pytest.raises(pkv.PkvError) as e:
        lib.add(0)                   # all 4 sequence ids are in use
    assert e.value.status == OOM and snap() == before
    with pytest.raises(pkv.PkvError) as e:
        lib.add(9)                   # no id, and 3 blocks with 2 free
    assert e.value.status == OOM and snap() == before
    # a, b start new blocks (2 fresh), c and d share block 3 (one copy): 3 > 2 free
    with pytest.raises(pkv.PkvError) as e:
        lib.prepare_step([a, b, c], 4)
    assert e.value.status == OOM and snap() == before
    with pytest.raises(pkv.PkvError) as e:
        lib.prepare_step([a, a], 4)
    assert e.value.status == INVALID and snap() == before
    with pytest.raises(pkv.PkvError) as e:
        lib.prepare_step([c, 7], 4)
    assert e.value.status == INVALID and snap() == before
    with pytest.raises(pkv.PkvError) as e:
        lib.prepare_step([a], 2)     # 9 tokens do not fit 2 blocks of 4
    assert e.value.status == INVALID and snap() == before
    with pytest.raises(pkv.PkvError) as e:
        lib.prepare_step([c], 4, max_copies=0)
    assert e.value.status == INVALID and snap() == before
    # both holders of block 3 append: one copy, the last in batch order keeps it
    t, l, p, cp = lib.prepare_step([d, c], 4)
    assert cp.tolist() == [[3, 4]] and t[0].tolist()[:2] == [2, 4] and t[1].tolist()[:2] == [2, 3]
    assert l.tolist() == [7, 7] and p.tolist() == [6, 6]


def test_release_frees_blocks_for_reuse_last_block_first():
    lib = pkv.BlockAllocator(8, 2, 4)
    s = lib.add(5)                   # blocks 0, 1, 2
    assert lib.info(s) == (5, [0, 1, 2])
    lib.release(s)
    assert lib.stats() == (8, 0)
    t = lib.add(6)                   # the released sequence's blocks come back first
    assert lib.info(t) == (6, [0, 1, 2])


@pytest.mark.parametrize("kv,io", [("bf16", "bf16"), ("f32", "f32"), ("fp8", "bf16")])
def test_dense_histories_equal_decode_step_on_a_paged_layout(kv, io):
    """The dense-history step is the paged oracle's step on any block
    layout of the same histories (gather of the codes, then the same
    arithmetic): outputs and appended codes are exactly equal."""
    rng = np.random.default_rng(7)
    hkv, hq, d, bs = 2, 4, 8, 4
    lens = [1, 5, 9, 4]
    k_scale = v_scale = None
    if kv == "fp8":
        k_scale = np.array([0.01, 0.02], np.float32)
        v_scale = np.array([0.015, 0.005], np.float32)
    hist = oracle.DenseHistories(kv, io, 1.0e4, k_scale, v_scale)

    def codes(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        if kv == "bf16":
            return oracle.bf16_bits_from_f32(x)
        if kv == "fp8":
            return oracle.fp8_encode(x * 0.5 / 0.02)
        return x

    def io_arr(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return x if io == "f32" else oracle.bf16_bits_from_f32(x)

    for s, L in enumerate(lens):
        hist.add(s, codes((hkv, L - 1, d)), codes((hkv, L - 1, d)))
    nblk = sum(-(-L // bs) for L in lens) + 3
    perm = rng.permutation(nblk)
    kp = codes((nblk, hkv, bs, d))
    vp = codes((nblk, hkv, bs, d))
    maxb = max(-(-L // bs) for L in lens)
    tables = np.full((len(lens), maxb), -1, np.int32)
    at = 0
    for s, L in enumerate(lens):
        for j in range(-(-L // bs)):
            tables[s, j] = perm[at]
            at += 1
        for t in range(L - 1):
            kp[tables[s, t // bs], :, t % bs] = hist.k[s][:, t]
            vp[tables[s, t // bs], :, t % bs] = hist.v[s][:, t]
    q, kn, vn = io_arr((len(lens), hq, d)), io_arr((len(lens), hkv, d)), io_arr((len(lens), hkv, d))
    pos = np.array(lens, np.int32) - 1
    paged = oracle.decode_step(k_pool=kp, v_pool=vp, kv_dtype=kv, io_dtype=io, q=q, k_new=kn,
                               v_new=vn, positions=pos, block_tables=tables,
                               context_lens=np.array(lens, np.int32), block_size=bs,
                               rope_theta=1.0e4, k_scale=k_scale, v_scale=v_scale)
    dense = hist.step(list(range(len(lens))), q, kn, vn, pos)
    np.testing.assert_array_equal(dense, paged["out"])
    for s in range(len(lens)):
        np.testing.assert_array_equal(hist.k[s][:, -1], paged["k_app"][s])
        np.testing.assert_array_equal(hist.v[s][:, -1], paged["v_app"][s])


def test_prepare_step_into_reused_buffers():
    """``out=`` fills caller-owned arrays with exactly what fresh arrays get,
    step after step (stale contents from a longer earlier batch included)."""
    bs, maxb = 4, 6
    a = pkv.BlockAllocator(64, bs, 8)
    b = pkv.BlockAllocator(64, bs, 8)
    for n in (3, 8, 0, 5):
        assert a.add(n) == b.add(n)
    bufs = (np.full((4, maxb), 77, np.int32), np.full(4, 77, np.int32),
            np.full(4, 77, np.int32), np.full((4, 2), 77, np.int32))
    for ids in ([0, 1, 2, 3], [3, 1], [2], [0, 1, 2, 3]):
        got = a.prepare_step(ids, maxb, out=bufs)
        want = b.prepare_step(ids, maxb)
        for g, w in zip(got, want):
            assert g.shape == w.shape and np.array_equal(g, w)
        assert np.shares_memory(got[0], bufs[0])
    with pytest.raises(pkv.PkvError):
        a.prepare_step([0, 1], maxb + 1, out=bufs)                 # row width differs
    with pytest.raises(pkv.PkvError):
        a.prepare_step([0, 1], maxb, out=(bufs[0].astype(np.int64),) + bufs[1:])
    with pytest.raises(pkv.PkvError):
        a.prepare_step([0, 1, 2, 3], maxb, max_copies=8, out=bufs)  # copies too small
    assert [a.info(s) for s in range(4)] == [b.info(s) for s in range(4)]
