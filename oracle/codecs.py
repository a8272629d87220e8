"""Storage codecs of the KV cache: bfloat16 and FP8 E4M3.  Test infrastructure.

Both encoders are the definitions written out: the result is the nearest
representable value, ties broken towards the even significand.  They are
deliberately slow and plain.

FP8 reading.  "TensorRT-LLM Guide: High-Throughput GPU Inference Engine",
section "4. Native FP8 Quantization on NVIDIA Hopper & Blackwell", names E4M3
(4 exponent bits, 3 mantissa bits) as the format.  The variant taken here is
the OCP E4M3FN encoding: exponent bias 7, no infinities, the single NaN
pattern S.1111.111 per sign, largest finite magnitude 448, subnormals
``m * 2**-9``.  The pages say nothing about rounding or overflow; the reading
taken is round-to-nearest-even with saturation to +-448 (values at or beyond
448 in magnitude encode as 448).
"""
from __future__ import annotations

import math

import numpy as np

FP8_MAX = 448.0


# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (IEEE 754).

    For each finite value the two bfloat16 neighbours are the value with its
    low 16 bits cleared (towards zero) and the next one away from zero; the
    nearer wins, measured exactly in float64, and a tie picks the neighbour
    whose last kept bit is 0.  Above the largest finite bfloat16 the next
    neighbour is infinity, weighed as 2**128.  NaN maps to a quiet NaN with
    the same sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000))
    hi = lo + np.uint32(0x10000)
    xv = x.astype(np.float64)
    lo_v = lo.view(np.float32).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        hi_v = hi.view(np.float32).astype(np.float64)
        # Past the largest finite bfloat16 the upper neighbour is infinity;
        # IEEE rounding measures against 2**128 (the next power of the
        # exponent range), so values beyond the midpoint overflow to inf.
        over = np.isinf(hi_v) & np.isfinite(xv)
        hi_v = np.where(over, np.copysign(2.0 ** 128, xv), hi_v)
        d_lo = np.abs(xv - lo_v)
        d_hi = np.abs(hi_v - xv)
    lo_even = ((lo >> np.uint32(16)) & np.uint32(1)) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(pick_hi, hi, lo) >> np.uint32(16)
    nan = np.isnan(x)
    out = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), out)
    inf = np.isinf(x)
    out = np.where(inf, u >> np.uint32(16), out)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------
# FP8 E4M3FN
# --------------------------------------------------------------------------
def fp8_code_value(code: int) -> float:
    """Value of one E4M3FN code from its fields (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_FP8_TABLE = np.array([fp8_code_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0..126 are increasing in value
_FP8_POS = _FP8_TABLE[:127].copy()


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> float64 values (exact)."""
    return _FP8_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp8_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3FN codes, saturating round-to-nearest-even.

    Magnitudes are clamped to 448 first; then the nearest of the 127
    non-negative finite values is chosen (exact comparison in float64), a tie
    going to the even code.  The sign bit is copied from the input, so a
    negative value that rounds to zero gives -0 (0x80).  NaN gives 0x7F with
    the input's sign.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), FP8_MAX)
    idx = np.searchsorted(_FP8_POS, a, side="left")      # first value >= a
    idx = np.clip(idx, 0, 126)
    below = np.clip(idx - 1, 0, 126)
    v_hi = _FP8_POS[idx]
    v_lo = _FP8_POS[below]
    d_hi = v_hi - a
    d_lo = a - v_lo
    exact = v_hi == a
    pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & (idx % 2 == 0))
    mag = np.where(pick_hi, idx, below).astype(np.uint8)
    sign = (np.signbit(x)).astype(np.uint8) << np.uint8(7)
    code = mag | sign
    nan = np.isnan(x)
    code = np.where(nan, np.uint8(0x7F) | sign, code)
    return code.astype(np.uint8)


def _selfcheck() -> None:  # pragma: no cover - quick sanity when run directly
    assert fp8_code_value(0x7E) == 448.0
    assert math.isnan(fp8_code_value(0x7F))
    assert fp8_code_value(0x01) == 2.0 ** -9


if __name__ == "__main__":  # pragma: no cover
    _selfcheck()
