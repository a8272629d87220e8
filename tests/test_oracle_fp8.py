"""Pins of the oracle's FP8 cache path that do not go through the oracle's own
dequantisation (``kv_to_f64``): the E4M3 cache, read back, must lie within
the format's rounding bound of the raw values it was encoded from; the fp8
step must equal torch's ``scaled_dot_product_attention`` in float64 on K/V
that the test dequantises itself (torch's own E4M3 conversion times the
scale); a tiny case must equal a 50-digit brute force; and a hand-worked
step with chosen codes and scales must give its closed-form output.

The format and the scale semantics are those of "TensorRT-LLM Guide:
High-Throughput GPU Inference Engine", section "4. Native FP8 Quantization on
NVIDIA Hopper & Blackwell" (E4M3, 4 exponent and 3 mantissa bits, with
precomputed scale factors); the reading taken is ``real = code * scale``,
one scale per KV head for K and one for V.  CPU only."""
import numpy as np
import pytest
import torch

import oracle
import oracle.decode as odec
import workloads
from oracle.variants import brute_force_attention

import problem


def small(lengths, hq=8, hkv=2, d=16, bs=4, seed=11):
    return workloads.custom_workload(lengths, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                     block_size=bs, kv_dtype="fp8", io_dtype="bf16", seed=seed)


def torch_dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """``[Hkv, L, D]`` E4M3FN codes -> float64 through torch's own conversion,
    times the per-head scale (the scale's float32 value, widened exactly)."""
    v = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    s = torch.from_numpy(np.asarray(scale, np.float32)).to(torch.float64)
    return (v.to(torch.float64) * s.view(-1, 1, 1)).numpy()


def e4m3_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the E4M3FN spacing at |x| (|x| <= 448): 2^(e-4) in the normal
    binade [2^e, 2^(e+1)), e >= -6, and 2^-10 on the subnormal grid."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.where(a < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))


_KV_TO_F64 = odec.kv_to_f64


def planted_kv_to_f64(codes, kv_dtype, scale=None):
    """A plausible mistake: the fp8 code divided by the scale."""
    if kv_dtype != "fp8":
        return _KV_TO_F64(codes, kv_dtype, scale)
    v = oracle.fp8_decode(codes)
    return v / np.asarray(scale, np.float32).astype(np.float64).reshape(-1, 1, 1)


# ---------------------------------------------------------------- rounding bound
def test_cache_dequantises_within_e4m3_rounding_of_the_raw_draws():
    """The fp8 cache, read back by the oracle, against the raw float32 N(0,1)
    values it was encoded from: the code is the nearest E4M3 value to
    raw * f32(1 / scale), so |code_value - raw / scale| is at most half the
    E4M3 spacing there (up to the rounding of the reciprocal, 2^-24
    relative), and the dequantised value is code_value * scale."""
    wl = small([37, 64, 5], d=32, bs=8)
    arrs = problem.build(wl)
    for which, scale in (("k_cache", arrs["k_scale"]), ("v_cache", arrs["v_scale"])):
        raw = workloads.host_normals(wl, which).astype(np.float64)       # [nb, Hkv, bs, D]
        codes = arrs["k_pool"] if which == "k_cache" else arrs["v_pool"]
        deq = np.stack([oracle.kv_to_f64(codes[n], "fp8", scale) for n in range(codes.shape[0])])
        s = np.asarray(scale, np.float32).astype(np.float64).reshape(1, -1, 1, 1)
        bound = e4m3_half_ulp(raw / s) * s * (1 + 2.0 ** -20) + np.abs(raw) * 2.0 ** -22
        assert np.all(np.abs(deq - raw) <= bound), which
        # and the bound is not vacuous: the worst error is a sizeable part of it
        assert np.max(np.abs(deq - raw) / bound) > 0.5


def test_rounding_bound_catches_a_planted_division_by_the_scale():
    wl = small([37, 64, 5], d=32, bs=8)
    arrs = problem.build(wl)
    raw = workloads.host_normals(wl, "v_cache").astype(np.float64)
    deq = np.stack([planted_kv_to_f64(arrs["v_pool"][n], "fp8", arrs["v_scale"])
                    for n in range(arrs["v_pool"].shape[0])])
    s = np.asarray(arrs["v_scale"], np.float32).astype(np.float64).reshape(1, -1, 1, 1)
    bound = e4m3_half_ulp(raw / s) * s * (1 + 2.0 ** -20) + np.abs(raw) * 2.0 ** -22
    assert not np.all(np.abs(deq - raw) <= bound)


# ---------------------------------------------------------------- library routine
def sdpa_on_torch_dequant(wl, arrs, res, b):
    c = wl.cfg
    L = int(wl.context_lens[b])
    g = c.n_q_heads // c.n_kv_heads
    kc = oracle.gather_request(res["k_pool"], wl.block_tables[b], L, c.block_size)
    vc = oracle.gather_request(res["v_pool"], wl.block_tables[b], L, c.block_size)
    kt = torch.from_numpy(np.repeat(torch_dequant(kc, arrs["k_scale"]), g, axis=0))
    vt = torch.from_numpy(np.repeat(torch_dequant(vc, arrs["v_scale"]), g, axis=0))
    qr = oracle.rope_f64(oracle.io_to_f64(arrs["q"][b], "bf16"), int(wl.positions[b]),
                         c.rope_theta)
    qt = torch.from_numpy(qr)[:, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()


def test_fp8_step_matches_torch_sdpa_on_torch_dequantised_kv():
    wl = small([40, 1, 77, 16], hq=8, hkv=2, d=32, bs=8)
    arrs = problem.build(wl)
    res = problem.oracle_step(wl, arrs)
    for b in range(wl.batch):
        ref = sdpa_on_torch_dequant(wl, arrs, res, b)
        assert np.max(np.abs(ref - res["out"][b])) < 1e-12


def test_sdpa_pin_catches_a_planted_division_by_the_scale(monkeypatch):
    wl = small([40, 77], hq=8, hkv=2, d=32, bs=8)
    arrs = problem.build(wl)
    monkeypatch.setattr(odec, "kv_to_f64", planted_kv_to_f64)
    res = problem.oracle_step(wl, arrs)
    worst = max(np.max(np.abs(sdpa_on_torch_dequant(wl, arrs, res, b) - res["out"][b]))
                for b in range(wl.batch))
    assert worst > 1e-3


# ---------------------------------------------------------------- brute force
def test_fp8_step_matches_mpmath_brute_force_tiny():
    """Dequantised in the test, code by code, from the E4M3 fields
    (``fp8_code_value``, itself pinned to torch's conversion of all 256
    codes) times the scale; attention in 50-digit arithmetic."""
    wl = small([3, 6], hq=2, hkv=1, d=4, bs=2)
    arrs = problem.build(wl)
    res = problem.oracle_step(wl, arrs)
    ks, vs = float(arrs["k_scale"][0]), float(arrs["v_scale"][0])
    deq = np.vectorize(oracle.fp8_code_value)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        kc = oracle.gather_request(res["k_pool"], wl.block_tables[b], L, 2)
        vc = oracle.gather_request(res["v_pool"], wl.block_tables[b], L, 2)
        kf, vf = deq(kc) * ks, deq(vc) * vs
        q = oracle.io_to_f64(arrs["q"][b], "bf16")
        bf = brute_force_attention(q, kf, vf, int(wl.positions[b]), wl.cfg.rope_theta)
        for hq in range(2):
            for j in range(4):
                assert abs(float(bf[hq][j]) - res["out"][b][hq, j]) < 1e-13


# ---------------------------------------------------------------- hand-worked case
def hand_worked_step():
    """Two tokens of one request, one KV head, D = 16, block size 16; zero
    query, so both tokens weigh 1/2 and out = mean of the two values.
    Cached token 0: every V code 0x40 (2.0) with V scale 0.5, i.e. 1.0.
    New token: v_new = 0.25 in bf16 -> 0.25 * f32(1/0.5) = 0.5 -> code 0x30
    (0.5), stored; read back 0.5 * 0.5 = 0.25.  out = (1.0 + 0.25) / 2."""
    d, bs = 16, 16
    kp = np.zeros((2, 1, bs, d), np.uint8)
    vp = np.zeros((2, 1, bs, d), np.uint8)
    kp[1, 0, 0, :] = 0x38          # 1.0
    vp[1, 0, 0, :] = 0x40          # 2.0
    bf = oracle.bf16_bits_from_f32
    q = bf(np.zeros((1, 1, d), np.float32))
    kn = bf(np.full((1, 1, d), 0.75, np.float32))
    vn = bf(np.full((1, 1, d), 0.25, np.float32))
    return oracle.decode_step(
        k_pool=kp, v_pool=vp, kv_dtype="fp8", io_dtype="bf16", q=q, k_new=kn, v_new=vn,
        positions=np.array([0], np.int32), block_tables=np.array([[1]], np.int32),
        context_lens=np.array([2], np.int32), block_size=bs, rope_theta=1.0e4,
        k_scale=np.array([0.25], np.float32), v_scale=np.array([0.5], np.float32))


def test_hand_worked_fp8_step():
    res = hand_worked_step()
    assert np.all(res["out"] == 0.625)
    # the new key at position 0 is not rotated: 0.75 * f32(1/0.25) = 3.0 = 1.5 * 2^1 -> 0x44
    assert np.all(res["k_app"] == 0x44)
    assert np.all(res["v_app"] == 0x30)
    # one-token context: the stored value comes back exactly, code * scale
    kp = np.zeros((1, 1, 16, 16), np.uint8)
    r1 = oracle.decode_step(
        k_pool=kp, v_pool=kp.copy(), kv_dtype="fp8", io_dtype="bf16",
        q=oracle.bf16_bits_from_f32(np.ones((1, 2, 16), np.float32)),
        k_new=oracle.bf16_bits_from_f32(np.ones((1, 1, 16), np.float32)),
        v_new=oracle.bf16_bits_from_f32(np.full((1, 1, 16), -1.5, np.float32)),
        positions=np.array([3], np.int32), block_tables=np.array([[0]], np.int32),
        context_lens=np.array([1], np.int32), block_size=16, rope_theta=1.0e4,
        k_scale=np.array([1.0], np.float32), v_scale=np.array([0.5], np.float32))
    # -1.5 * 2 = -3.0 -> code 0xC4, read back -3.0 * 0.5
    assert np.all(r1["v_app"] == 0xC4)
    assert np.all(r1["out"] == -1.5)


def test_hand_worked_case_catches_a_planted_division_by_the_scale(monkeypatch):
    monkeypatch.setattr(odec, "kv_to_f64", planted_kv_to_f64)
    res = hand_worked_step()
    assert not np.all(res["out"] == 0.625)
