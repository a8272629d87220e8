"""Pins of the oracle's multi-token step (T new tokens per request, causal
inside the chunk): T = 1 is the single-token step; T tokens equal T single
steps one after the other; a query never sees a later new token; and a
50-digit brute force over the tokens each query may see agrees."""
import numpy as np
import pytest

import oracle
from oracle.variants import brute_force_attention


def problem(lens, tq, kv="bf16", hkv=2, hq=4, d=8, bs=4, seed=5):
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
    B = len(lens)
    return dict(k_pool=kp, v_pool=vp, kv_dtype=kv, io_dtype=io,
                q=enc(rng.standard_normal((B, tq, hq, d)).astype(np.float32)),
                k_new=enc(rng.standard_normal((B, tq, hkv, d)).astype(np.float32)),
                v_new=enc(rng.standard_normal((B, tq, hkv, d)).astype(np.float32)),
                positions=np.array(lens, np.int32) - tq + 3, block_tables=tables,
                context_lens=np.array(lens, np.int32), block_size=bs, rope_theta=1.0e4,
                k_scale=k_scale, v_scale=v_scale)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_one_token_is_the_single_step(kv):
    p = problem([1, 6, 13], 1, kv)
    m = oracle.decode_step_multi(**p)
    s = oracle.decode_step(**dict(p, q=p["q"][:, 0], k_new=p["k_new"][:, 0], v_new=p["v_new"][:, 0]))
    np.testing.assert_array_equal(m["out"][:, 0], s["out"])
    np.testing.assert_array_equal(m["k_pool"], s["k_pool"])
    np.testing.assert_array_equal(m["v_pool"], s["v_pool"])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("tq", [2, 3, 5])
def test_t_tokens_equal_t_single_steps(kv, tq):
    lens = [5, 9, 13, 21]
    p = problem(lens, tq, kv)
    m = oracle.decode_step_multi(**p)
    kp, vp = p["k_pool"], p["v_pool"]
    for i in range(tq):
        s = oracle.decode_step(**dict(p, k_pool=kp, v_pool=vp, q=p["q"][:, i],
                                      k_new=p["k_new"][:, i], v_new=p["v_new"][:, i],
                                      positions=p["positions"] + i,
                                      context_lens=p["context_lens"] - tq + i + 1))
        np.testing.assert_array_equal(m["out"][:, i], s["out"])
        kp, vp = s["k_pool"], s["v_pool"]
    np.testing.assert_array_equal(m["k_pool"], kp)
    np.testing.assert_array_equal(m["v_pool"], vp)


def test_a_query_never_sees_a_later_new_token():
    p = problem([7, 12], 4)
    base = oracle.decode_step_multi(**p)["out"]
    for j in range(1, 4):
        k2, v2 = p["k_new"].copy(), p["v_new"].copy()
        k2[:, j] ^= np.uint16(0x1234)
        v2[:, j] ^= np.uint16(0x0f0f)
        out = oracle.decode_step_multi(**dict(p, k_new=k2, v_new=v2))["out"]
        np.testing.assert_array_equal(out[:, :j], base[:, :j])
        assert np.abs(out[:, j:] - base[:, j:]).max() > 0


def test_multi_agrees_with_brute_force():
    lens, tq = [6], 3
    p = problem(lens, tq, "f32", hkv=1, hq=2, d=4, bs=4)
    m = oracle.decode_step_multi(**p)
    kc = oracle.gather_request(m["k_pool"], p["block_tables"][0], 6, 4).astype(np.float64)
    vc = oracle.gather_request(m["v_pool"], p["block_tables"][0], 6, 4).astype(np.float64)
    for i in range(tq):
        seen = 6 - tq + i + 1
        bf = np.array(brute_force_attention(p["q"][0, i].astype(np.float64), kc[:, :seen],
                                            vc[:, :seen], int(p["positions"][0]) + i, 1.0e4),
                      dtype=np.float64)
        np.testing.assert_allclose(m["out"][0, i], bf, rtol=0, atol=1e-13)
