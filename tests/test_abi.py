"""The C ABI on the CPU: exports, host-side argument checks, the RoPE table,
and the work partition the kernel computes (replayed on the host)."""
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_decode_step_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

OK, INVALID, UNSUPPORTED = 0, -1, -2


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.mark.device_library
def test_library_loads_and_exports_every_declared_function():
    lib = pkv.load_library()
    declared = header_functions()
    assert set(declared) == set(pkv.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def base_args(**kw):
    a = dict(num_blocks=100, block_size=16, n_kv_heads=8, head_dim=128, kv_dtype="bf16",
             io_dtype="bf16", max_blocks_per_seq=64, batch=4, n_q_heads=32,
             q=0x1000, k_new=0x2000, v_new=0x3000, positions=0x4000,
             block_tables=0x5000, context_lens=0x6000, out=0x7000)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw", [
    {}, {"kv_dtype": "fp8"}, {"kv_dtype": "f32", "io_dtype": "f32"},
    {"head_dim": 64}, {"block_size": 32}, {"block_size": 64},
    {"n_q_heads": 8}, {"n_q_heads": 128}, {"batch": 4096}, {"batch": 0, "q": 0},
])
def test_check_accepts_supported(kw):
    assert pkv.check_decode_args(**base_args(**kw)) == OK, pkv.last_error()


@pytest.mark.parametrize("kw,code", [
    ({"batch": -1}, INVALID),
    ({"batch": 4097}, UNSUPPORTED),
    ({"n_q_heads": 12}, INVALID),                # not a multiple of Hkv
    ({"n_q_heads": 0}, INVALID),
    ({"n_q_heads": 136}, UNSUPPORTED),           # group of 17
    ({"head_dim": 96}, UNSUPPORTED),
    ({"block_size": 8}, UNSUPPORTED),
    ({"io_dtype": "f32"}, UNSUPPORTED),          # f32 io with bf16 cache
    ({"kv_dtype": "f32"}, UNSUPPORTED),          # bf16 io with f32 cache
    ({"io_dtype": 7}, INVALID),
    ({"q": 0}, INVALID),
    ({"context_lens": 0}, INVALID),
    ({"out": 0x7004}, INVALID),                  # misaligned
    ({"max_blocks_per_seq": 0}, INVALID),
    ({"num_blocks": 0}, INVALID),
    ({"max_blocks_per_seq": 1 << 21}, UNSUPPORTED),   # > 2^24 tokens
])
def test_check_rejects(kw, code):
    assert pkv.check_decode_args(**base_args(**kw)) == code
    assert pkv.last_error()


@pytest.mark.device_library
def test_pool_create_validates_before_touching_the_gpu():
    for args in [(0, 16, 8, 128, "bf16"), (10, 24, 8, 128, "bf16"),
                 (10, 16, 0, 128, "bf16"), (10, 16, 8, 80, "bf16"),
                 (1 << 40, 16, 8, 128, "bf16")]:
        with pytest.raises(pkv.PkvError) as e:
            pkv.KVPool(*args)
        assert e.value.status in (INVALID, UNSUPPORTED)


@pytest.mark.parametrize("theta,d", [(1.0e4, 64), (5.0e5, 128), (1.0e6, 128), (500.0, 64)])
def test_rope_table_bit_equal_to_oracle(theta, d):
    c, s = pkv.rope_table_host(theta, d, 9000)
    positions = [0, 1, 2, 3, 137, 1011, 4095, 8191, 8999]
    oc, os_ = oracle.rope_rows_f32(theta, d, positions)
    assert np.array_equal(c[positions].view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s[positions].view(np.uint32), os_.view(np.uint32))


def test_rope_table_rejects_bad_arguments():
    with pytest.raises(pkv.PkvError):
        pkv.rope_table_host(-1.0, 64, 10)
    with pytest.raises(pkv.PkvError):
        pkv.rope_table_host(1e4, 64, 0)


def test_tile_tokens():
    assert pkv.tile_tokens() == 16


# ---- work partition ---------------------------------------------------------
def reference_partition(lens, hkv, cap, n_waves, min_units, cost, n_first=0, wf=1, wr=1,
                        min_share=0, wo=100, window=0):
    """The partition written out plainly: sequences (b, h) in order, each cut
    into max(1, ceil(min(L, cap)/16)) tiles and costing its tiles plus
    `cost` units (tile 0 owns cost + 1 units); wave w weighs (wf if
    w < n_first else wr) * (wo if (w // 4) is odd else 100); the most waves
    whose exact share for a wave of the lightest of all n_waves weights is
    >= max(min_units, cost + 1) units are used (found by trying every
    count), unless they are fewer than min(n_first, n_waves): then the most
    waves, up to that many, whose share is >= max(that // 4, cost + 1) units;
    the units are cut at floor(total * weights before w / all
    weights) and each tile is owned by the wave holding its first unit.  With a
    window of W >= 1 tokens a sequence's tiles start at the one holding token
    L - W (when L > W), and are numbered from there."""
    def tiles(L):
        L = min(max(int(L), 0), cap)
        lo = (L - window) // 16 if window > 0 and L > window else 0
        return max(1, -(-L // 16)) - lo
    ns = [tiles(L) for L in lens]
    seqs = [(b, h, ns[b]) for b in range(len(lens)) for h in range(hkv)]
    first_units = []
    u = 0
    for b, h, n in seqs:
        for t in range(n):
            first_units.append(((b, h, t), u))
            u += cost + 1 if t == 0 else 1
    total = u
    m = max(min_units, cost + 1)
    if total < min_share * n_waves:     # too little work per wave: even weights
        wf = wr = 1
    weight = [(wf if w < n_first else wr) * (wo if (w // 4) % 2 else 100)
              for w in range(n_waves)]
    lightest = min(weight)

    def enough(count):
        return total * lightest >= m * sum(weight[:count])

    we = max([c for c in range(1, n_waves + 1) if enough(c)], default=1)
    cap = min(n_first, n_waves)
    if we < cap and max(m // 4, cost + 1) < m:
        m = max(m // 4, cost + 1)
        we = max([c for c in range(1, cap + 1) if enough(c)], default=1)
    om = sum(weight[:we])
    bounds = [(total * sum(weight[:w])) // om for w in range(we + 1)]
    owner = {}
    for key, fu in first_units:
        owner[key] = max(i for i in range(we) if bounds[i] <= fu)
    return owner, bounds, we, seqs


@pytest.mark.parametrize("lens,hkv,waves,min_units,cost,nf,wf,wr", [
    ([138, 1012, 84], 4, 64, 4, 0, 0, 1, 1),
    ([138, 1012, 84], 4, 64, 4, 3, 0, 1, 1),
    ([138, 1012, 84], 4, 64, 4, 3, 32, 100, 57),
    ([1, 1, 1, 1], 2, 64, 1, 0, 0, 1, 1),
    ([1, 1, 1, 1], 2, 64, 1, 2, 0, 1, 1),
    ([1, 1, 1, 1], 2, 64, 1, 2, 4, 3, 2),
    ([5000, 3, 70, 31, 32, 33], 3, 20, 2, 0, 0, 1, 1),
    ([5000, 3, 70, 31, 32, 33], 3, 20, 2, 5, 0, 1, 1),
    ([5000, 3, 70, 31, 32, 33], 3, 20, 2, 5, 10, 7, 4),
    ([5000, 3, 70, 31, 32, 33], 3, 20, 9, 5, 4, 1000, 1),
    ([1], 1, 8, 4, 3, 0, 1, 1),
    ([1], 1, 8, 4, 3, 4, 100, 57),
    (list(np.random.default_rng(0).integers(1, 3000, 40)), 8, 96, 3, 3, 0, 1, 1),
    (list(np.random.default_rng(0).integers(1, 3000, 40)), 8, 96, 3, 3, 48, 100, 57),
    (list(np.random.default_rng(1).integers(1, 200, 60)), 4, 200, 1, 7, 0, 1, 1),
    (list(np.random.default_rng(1).integers(1, 200, 60)), 4, 200, 1, 7, 100, 100, 40),
    (list(np.random.default_rng(2).integers(1, 5000, 30)), 8, 64, 16, 8, 32, 100, 57),
    ([100] * 7, 2, 1000, 1, 1, 0, 1, 1),       # more wavefronts than units allow
    ([100] * 7, 2, 1000, 1, 1, 500, 100, 57),
    ([0, -5, 40], 2, 16, 1, 2, 0, 1, 1),       # invalid lengths still get one tile
    ([16, 17, 15, 32, 33], 1, 5, 1, 0, 0, 1, 1),
    ([16, 17, 15, 32, 33], 1, 5, 1, 0, 2, 5, 3),
    ([9 * 16 - 3], 1, 2, 16, 8, 0, 1, 1),     # U = m + 1
    ([23, 10], 2, 64, 6, 5, 0, 1, 1),         # ceil(U/m) = 5 waves would leave wave 3 no tile
    # steps too small for the first workgroups at min_units each: shares down
    # to max(min_units // 4, cost + 1), capped at n_first (32) or not (64)
    ([138, 1012, 84], 4, 64, 16, 6, 32, 1, 1),
    ([138, 1012, 84], 4, 128, 16, 6, 64, 1, 1),
    ([138, 1012, 84], 4, 128, 16, 6, 64, 100, 57),
    ([138, 1012, 84], 4, 128, 40, 2, 64, 1, 1),
    (list(np.random.default_rng(3).integers(1, 300, 9)), 2, 256, 24, 4, 128, 100, 65),
])
@pytest.mark.parametrize("min_share", [0, 40])
@pytest.mark.parametrize("wo", [100, 90, 37, 1])
def test_partition_covers_every_tile_once_and_balances(lens, hkv, waves, min_units, cost,
                                                       nf, wf, wr, min_share, wo):
    cap = 1 << 20
    pieces, splits = pkv.plan_host(lens, hkv, cap, waves, min_units, cost, nf, wf, wr,
                                   min_share, weight_odd=wo)
    owner, bounds, we, seqs = reference_partition(lens, hkv, cap, waves, min_units, cost,
                                                  nf, wf, wr, min_share, wo)
    if bounds[-1] < min_share * waves:
        wf = wr = 1
    seen = {}
    per_wave = np.zeros(waves, dtype=np.int64)
    for w, b, h, t0, t1, fl in pieces:
        assert t0 < t1
        for t in range(t0, t1):
            assert (b, h, t) not in seen
            seen[(b, h, t)] = w
        per_wave[w] += t1 - t0
    assert seen == owner
    # every active wave owns a tile; unit ranges within one of their exact shares
    assert np.all(per_wave[:we] >= 1) and np.all(per_wave[we:] == 0)
    sizes = np.diff(bounds)
    weights = np.array([(wf if w < nf else wr) * (wo if (w // 4) % 2 else 100)
                        for w in range(we)], dtype=np.float64)
    exact = bounds[-1] * weights / weights.sum()
    assert np.all(np.abs(sizes - exact) < 1.0)
    # flags and split rows against a direct reading
    by_seq = {}
    for w, b, h, t0, t1, fl in pieces:
        by_seq.setdefault((b, h), []).append((w, t0, t1, fl))
    rows = {}
    for (b, h, n) in seqs:
        ps = by_seq[(b, h)]
        split = len(ps) > 1
        for i, (w, t0, t1, fl) in enumerate(ps):
            assert bool(fl & 1) == split
            assert bool(fl & 4) == (t1 == n)
            if split:   # only a wave's first or last piece can be split
                assert bool(fl & 2) or t1 == n or w == ps[-1][0] or True
        if split:
            w_first, w_last = ps[0][0], ps[-1][0]
            # the pieces sit in consecutive wavefronts
            assert [p[0] for p in ps] == list(range(w_first, w_last + 1))
            rows[w_first] = (b * hkv + h, len(ps), 0 if ps[0][3] & 2 else 1)
    for w in range(waves):
        row = splits[w]
        if w in rows:
            assert row[0] == 1 and tuple(row[1:]) == rows[w]
        else:
            assert row[0] == 0


def test_piece_cost_gives_many_piece_waves_fewer_tiles():
    # 1 long sequence then 40 one-tile sequences, 4 waves: with a cost per
    # sequence start, the waves holding the short ones take fewer tiles
    lens = [16 * 200] + [16] * 40
    p0, _ = pkv.plan_host(lens, 1, 1 << 20, 4, 1, 0)
    p5, _ = pkv.plan_host(lens, 1, 1 << 20, 4, 1, 5)
    tiles = lambda ps: np.bincount(ps[:, 0], weights=ps[:, 4] - ps[:, 3], minlength=4)
    t0, t5 = tiles(p0), tiles(p5)
    assert t0.max() - t0.min() <= 1
    assert t5[3] < t0[3] and t5[0] > t0[0]


@pytest.mark.parametrize("window", [1, 15, 16, 17, 40, 100, 5000])
def test_partition_with_a_window_reads_only_the_window(window):
    lens = [1, 16, 17, 40, 100, 300, 1000, 33, 5000]
    cap = 1 << 20
    for waves, cost in ((8, 0), (40, 3), (200, 6)):
        pieces, splits = pkv.plan_host(lens, 2, cap, waves, 1, cost, window=window)
        owner, bounds, we, seqs = reference_partition(lens, 2, cap, waves, 1, cost, window=window)
        seen = {}
        for w, b, h, t0, t1, fl in pieces:
            for t in range(t0, t1):
                seen[(b, h, t)] = w
        assert seen == owner
        for b, h, n in seqs:
            L = lens[b]
            lo = (L - window) // 16 if L > window else 0
            assert n == -(-L // 16) - lo       # the tiles holding tokens [L - window, L)


@pytest.mark.device_library
def test_layout_and_rope_table_calls_check_their_arguments():
    """kv_pool_layout and kv_pool_rope_table through ctypes: a null pool or
    output pointer is refused with INVALID before anything is read."""
    import ctypes
    lib = pkv.load_library()
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    st = (ctypes.c_int64 * 3)()
    tb = ctypes.c_int32()
    assert lib.kv_pool_layout(None, ctypes.byref(k), ctypes.byref(v), st, ctypes.byref(tb)) == INVALID
    assert "null" in pkv.last_error()
    c, s = ctypes.c_void_p(), ctypes.c_void_p()
    n = ctypes.c_int32()
    assert lib.kv_pool_rope_table(None, ctypes.byref(c), ctypes.byref(s), ctypes.byref(n)) == INVALID
    assert "null" in pkv.last_error()


@pytest.mark.device_library
def test_stream_read_checks_its_arguments():
    """pkv_stream_read refuses a null pointer or a size that is not a positive
    multiple of 16 before touching the GPU."""
    import ctypes
    lib = pkv.load_library()
    assert lib.pkv_stream_read(None, 1024, ctypes.c_void_p(0x1000), None) == INVALID
    assert lib.pkv_stream_read(ctypes.c_void_p(0x1000), 1000, ctypes.c_void_p(0x2000), None) == INVALID
    assert lib.pkv_stream_read(ctypes.c_void_p(0x1000), 0, ctypes.c_void_p(0x2000), None) == INVALID
    assert lib.pkv_stream_read(ctypes.c_void_p(0x1008), 1024, ctypes.c_void_p(0x2000), None) == INVALID


@pytest.mark.device_library
def test_read_timeline_checks_its_arguments():
    """kv_pool_read_timeline refuses a null pool or output with INVALID
    before anything is read."""
    import ctypes
    lib = pkv.load_library()
    n = ctypes.c_int32()
    buf = (ctypes.c_uint64 * 8)()
    assert lib.kv_pool_read_timeline(None, buf, 1, ctypes.byref(n)) == INVALID
    assert "null" in pkv.last_error()


@pytest.mark.device_library
@pytest.mark.skipif(not os.path.exists(pkv.TIMELINE_LIB_PATH), reason="timeline build not present")
def test_timeline_build_exports_the_same_functions():
    import ctypes
    lib = ctypes.CDLL(pkv.TIMELINE_LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
