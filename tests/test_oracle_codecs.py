"""Pins of the oracle's storage codecs (bfloat16, FP8 E4M3FN).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_fp8_to_f32(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def torch_f32_to_fp8(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy())
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_decode(codes)
    ref = torch_fp8_to_f32(codes).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                       # S.1111.111 for both signs
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs too (0x80 is -0)
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_fp8_landmarks_golden():
    g = json.load(open(os.path.join(GOLDEN, "fp8_e4m3fn_landmarks.json")))
    for hexcode, val in g["codes"].items():
        v = oracle.fp8_code_value(int(hexcode, 16))
        assert v == val and math.copysign(1, v) == math.copysign(1, val)
    for hexcode in g["nan_codes"]:
        assert math.isnan(oracle.fp8_code_value(int(hexcode, 16)))


def test_fp8_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.fp8_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(vals), codes)


def test_fp8_encode_ties_and_saturation():
    cases = {
        1.5 * 2.0 ** -9: 0x02,     # tie between 1 and 2 ulps -> even (2)
        2.0 ** -10: 0x00,          # tie between 0 and 2**-9 -> even (0)
        2.5 * 2.0 ** -9: 0x02,     # tie between 2 and 3 -> even (2)
        3.5 * 2.0 ** -9: 0x04,     # tie between 3 and 4 -> even (4)
        1.0625: 0x38,              # tie 1.0 / 1.125 -> even (1.0)
        1.1875: 0x3A,              # tie 1.125 / 1.25 -> even (1.25)
        464.0: 0x7E,               # beyond 448 saturates
        465.0: 0x7E,
        1.0e4: 0x7E,
        float("inf"): 0x7E,
        -1.0e4: 0xFE,
        -0.0: 0x80,
        -1e-30: 0x80,
    }
    x = np.array(list(cases.keys()), dtype=np.float32)
    want = np.array(list(cases.values()), dtype=np.uint8)
    assert np.array_equal(oracle.fp8_encode(x), want)


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-2 ** -6, 2 ** -6, 50000).astype(np.float32),
        rng.uniform(-448, 448, 50000).astype(np.float32),
    ])
    # exact midpoints between neighbouring codes (ties)
    vals = oracle.fp8_decode(np.arange(127, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    assert np.array_equal(oracle.fp8_encode(x), torch_f32_to_fp8(x))


def test_fp8_encode_saturates_where_torch_gives_nan():
    x = np.array([465.0, 480.0, 1e6], dtype=np.float32)
    assert np.all(np.isnan(torch_fp8_to_f32(torch_f32_to_fp8(x))))   # torch does not saturate
    assert np.all(oracle.fp8_decode(oracle.fp8_encode(x)) == 448.0)


def test_bf16_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(300000).astype(np.float32),
        (rng.standard_normal(10000) * 1e-39).astype(np.float32),  # subnormals
        np.array([3.3895314e38, -3.3895314e38, 1.0, -0.0, 0.0, np.inf, -np.inf], np.float32),
        # around the overflow threshold: largest finite float32, the bf16
        # midpoint 0x7F7F8000 (ties up to inf) and its neighbours
        np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000, 0x7F7F0001],
                 np.uint32).view(np.float32),
    ])
    # exact ties: bf16 value + half an ulp
    base = rng.integers(0, 0x7F00, 20000, dtype=np.uint32) << np.uint32(16)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_from_f32(x), ref)


def test_bf16_widening_is_exact():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    same = (f.view(np.uint32) == t.view(np.uint32)) | (np.isnan(f) & np.isnan(t))
    assert same.all()


def test_bf16_encode_of_bf16_values_is_identity():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(oracle.bf16_bits_from_f32(f[finite]), bits[finite])
