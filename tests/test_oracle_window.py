"""Pins of the oracle's sliding-window attention (a request attends to its
last `window` tokens, the new one included): a window at least as long as
the context changes nothing, a window of one returns the new token's value,
the window equals full attention over a request that holds only the window's
tokens (same position), and a 50-digit brute force over the window's tokens
agrees; a window one token off fails the brute force."""
import numpy as np
import pytest

import oracle
from oracle.variants import brute_force_attention


def problem(lens, kv="bf16", hkv=2, hq=4, d=8, bs=4, seed=3):
    rng = np.random.default_rng(seed)
    nblk = sum(-(-L // bs) for L in lens) + 2
    x = rng.standard_normal((2, nblk, hkv, bs, d)).astype(np.float32)
    k_scale = v_scale = None
    if kv == "bf16":
        kp, vp = oracle.bf16_bits_from_f32(x[0]), oracle.bf16_bits_from_f32(x[1])
    elif kv == "fp8":
        k_scale = np.full(hkv, 0.01, np.float32)
        v_scale = np.full(hkv, 0.02, np.float32)
        kp, vp = oracle.fp8_encode(x[0] * 100.0), oracle.fp8_encode(x[1] * 50.0)
    else:
        kp, vp = x[0], x[1]
    perm = rng.permutation(nblk)
    maxb = max(-(-L // bs) for L in lens)
    tables = np.full((len(lens), maxb), -1, np.int32)
    at = 0
    for b, L in enumerate(lens):
        for j in range(-(-L // bs)):
            tables[b, j] = perm[at]
            at += 1
    io = "f32" if kv == "f32" else "bf16"
    enc = (lambda a: a) if io == "f32" else oracle.bf16_bits_from_f32
    q = enc(rng.standard_normal((len(lens), hq, d)).astype(np.float32))
    kn = enc(rng.standard_normal((len(lens), hkv, d)).astype(np.float32))
    vn = enc(rng.standard_normal((len(lens), hkv, d)).astype(np.float32))
    return dict(k_pool=kp, v_pool=vp, kv_dtype=kv, io_dtype=io, q=q, k_new=kn, v_new=vn,
                positions=np.array(lens, np.int32) - 1 + 7, block_tables=tables,
                context_lens=np.array(lens, np.int32), block_size=bs, rope_theta=1.0e4,
                k_scale=k_scale, v_scale=v_scale)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_window_at_least_the_context_changes_nothing(kv):
    p = problem([1, 6, 13, 9], kv)
    full = oracle.decode_step(**p)["out"]
    for w in (13, 14, 1000):
        np.testing.assert_array_equal(oracle.decode_step(**p, window=w)["out"], full)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_window_of_one_returns_the_new_value(kv):
    p = problem([1, 6, 13, 9], kv)
    r = oracle.decode_step(**p, window=1)
    hkv, hq = p["k_new"].shape[1], p["q"].shape[1]
    g = hq // hkv
    for b in range(4):
        v = oracle.kv_to_f64(r["v_app"][b][:, None, :], kv, p["v_scale"])[:, 0]
        for h in range(hq):
            np.testing.assert_array_equal(r["out"][b, h], v[h // g])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("w", [2, 4, 5, 7])
def test_window_equals_a_request_holding_only_the_window(kv, w):
    lens = [13, 9, 3]
    p = problem(lens, kv)
    win = oracle.decode_step(**p, window=w)
    bs = p["block_size"]
    for b, L in enumerate(lens):
        n = min(L, w)
        # a fresh one-request layout whose context is the last n tokens
        tab = p["block_tables"][b]
        kp = np.zeros((-(-n // bs) + 1,) + p["k_pool"].shape[1:], p["k_pool"].dtype)
        vp = np.zeros_like(kp)
        for t in range(n - 1):
            src = L - n + t
            kp[t // bs, :, t % bs] = p["k_pool"][tab[src // bs], :, src % bs]
            vp[t // bs, :, t % bs] = p["v_pool"][tab[src // bs], :, src % bs]
        one = dict(p, k_pool=kp, v_pool=vp, q=p["q"][b:b + 1], k_new=p["k_new"][b:b + 1],
                   v_new=p["v_new"][b:b + 1], positions=p["positions"][b:b + 1],
                   block_tables=np.arange(-(-n // bs), dtype=np.int32)[None, :],
                   context_lens=np.array([n], np.int32))
        r = oracle.decode_step(**one)
        np.testing.assert_array_equal(win["out"][b], r["out"][0])


def test_window_agrees_with_brute_force_and_an_off_by_one_does_not():
    lens = [9]
    p = problem(lens, "f32", hkv=1, hq=2, d=4, bs=4)
    w = 3
    r = oracle.decode_step(**p, window=w)
    kc = oracle.gather_request(r["k_pool"], p["block_tables"][0], 9, 4).astype(np.float64)
    vc = oracle.gather_request(r["v_pool"], p["block_tables"][0], 9, 4).astype(np.float64)
    q = p["q"][0].astype(np.float64)
    pos = int(p["positions"][0])
    bf = np.array(brute_force_attention(q, kc[:, 9 - w:], vc[:, 9 - w:], pos, 1.0e4), dtype=np.float64)
    np.testing.assert_allclose(r["out"][0], bf, rtol=0, atol=1e-13)
    for wrong in (w - 1, w + 1):
        other = oracle.decode_step(**p, window=wrong)["out"][0]
        assert np.abs(other - bf).max() > 1e-6
