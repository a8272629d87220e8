"""Second and third computations of the same step.  Test infrastructure.

These exist to pin ``decode.decode_step`` to something other than itself:

* ``padded_static_batch`` - the static batch of "TensorRT-LLM Guide:
  High-Throughput GPU Inference Engine" (section "2. The Failure of Static
  Batching"): every request padded to the longest context, the padding masked
  out with ``-inf`` before the softmax.  Dense arrays, one vectorised gather
  by token index, no per-request loop;
* ``split_merge`` - attention over token chunks, each reduced to a running
  max, a sum of exponentials and an unnormalised output, merged afterwards;
  this checks the decomposition the GPU path uses for long contexts;
* ``brute_force_rotate_key`` / ``brute_force_attention`` - scalar Python
  loops for tiny shapes: the float32 key rotation re-derived with exact
  rationals, and the attention in 50-digit mpmath.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import Optional

import numpy as np

from .decode import io_to_f64, kv_to_f64
from .rope import rope_f64


def padded_static_batch(*, k_pool_after: np.ndarray, v_pool_after: np.ndarray,
                        kv_dtype: str, io_dtype: str, q: np.ndarray,
                        positions: np.ndarray, block_tables: np.ndarray,
                        context_lens: np.ndarray, block_size: int,
                        rope_theta: float,
                        k_scale: Optional[np.ndarray] = None,
                        v_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention of the whole batch as one padded, masked dense computation.

    ``k_pool_after``/``v_pool_after`` already hold the appended token.
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    bsz = lens.shape[0]
    lmax = int(lens.max())
    t = np.arange(lmax)
    valid = t[None, :] < lens[:, None]                         # [B, Lmax]
    blk_idx = np.where(valid, t[None, :] // block_size, 0)
    phys = np.take_along_axis(block_tables.astype(np.int64), blk_idx, axis=1)
    phys = np.where(valid, phys, 0)
    slot = t[None, :] % block_size
    # [B, Lmax, Hkv, D] -> [B, Hkv, Lmax, D]
    kd = k_pool_after[phys, :, np.broadcast_to(slot, phys.shape), :]
    vd = v_pool_after[phys, :, np.broadcast_to(slot, phys.shape), :]
    kd = np.moveaxis(kd, 2, 1)
    vd = np.moveaxis(vd, 2, 1)
    kf = np.stack([kv_to_f64(kd[b], kv_dtype, k_scale) for b in range(bsz)])
    vf = np.stack([kv_to_f64(vd[b], kv_dtype, v_scale) for b in range(bsz)])
    hkv = kf.shape[1]
    hq = q.shape[1]
    g = hq // hkv
    d = kf.shape[-1]
    qf = np.stack([rope_f64(io_to_f64(q[b], io_dtype), int(positions[b]),
                            rope_theta) for b in range(bsz)])   # [B, Hq, D]
    # repeat KV heads for their query heads: [B, Hq, Lmax, D]
    kr = np.repeat(kf, g, axis=1)
    vr = np.repeat(vf, g, axis=1)
    scores = np.einsum("bhd,bhtd->bht", qf, kr) / math.sqrt(d)
    scores = np.where(valid[:, None, :], scores, -np.inf)
    m = scores.max(axis=2, keepdims=True)
    w = np.exp(scores - m)
    w = w / w.sum(axis=2, keepdims=True)
    vr = np.where(valid[:, None, :, None], vr, 0.0)
    return np.einsum("bht,bhtd->bhd", w, vr)


def split_merge(q_rot: np.ndarray, k: np.ndarray, v: np.ndarray,
                chunk: int) -> np.ndarray:
    """Attention of one request computed chunk by chunk, then merged.

    Each chunk ``c`` gives ``m_c = max s``, ``l_c = sum exp(s - m_c)`` and
    ``a_c = sum exp(s - m_c) v``; with ``M = max_c m_c`` the result is
    ``sum_c exp(m_c - M) a_c / sum_c exp(m_c - M) l_c``.
    """
    hq, d = q_rot.shape
    hkv, length, _ = k.shape
    g = hq // hkv
    out = np.empty((hq, d))
    for h in range(hq):
        kv = h // g
        ms, ls, accs = [], [], []
        for c0 in range(0, length, chunk):
            s = (k[kv, c0:c0 + chunk] @ q_rot[h]) / math.sqrt(d)
            m = s.max()
            w = np.exp(s - m)
            ms.append(m)
            ls.append(w.sum())
            accs.append(w @ v[kv, c0:c0 + chunk])
        mm = max(ms)
        f = np.array([math.exp(m - mm) for m in ms])
        out[h] = (f[:, None] * np.array(accs)).sum(0) / (f * np.array(ls)).sum()
    return out


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------
def _round_f32(fr: Fraction) -> float:
    """Correctly rounded (nearest-even) float32 of an exact rational."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix e so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormal spacing below 2**-126
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    val = float(q * ulp)
    assert struct.unpack("f", struct.pack("f", val))[0] == val
    return sign * val


def _f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def brute_force_rotate_key(k_new32: np.ndarray, cos32, sin32) -> np.ndarray:
    """Rotated key by scalar loops with exact rationals.

    Each float32 operation of the pinned key rotation is evaluated exactly
    as a rational and then rounded once to float32 (nearest-even), which is
    what a single IEEE float32 operation does.  ``k_new32 [Hkv, D]``;
    ``cos32``/``sin32`` the float32 table row of the position.  Returns the
    rotated float32 values as float64 ``[Hkv, D]``.
    """
    hkv, d = k_new32.shape
    h2 = d // 2
    key = np.empty((hkv, d))
    for h in range(hkv):
        for i in range(h2):
            x0 = Fraction(float(k_new32[h, i]))
            x1 = Fraction(float(k_new32[h, i + h2]))
            c = Fraction(float(cos32[i]))
            s = Fraction(float(sin32[i]))
            a = Fraction(_round_f32(x0 * c))
            b = Fraction(_round_f32(x1 * s))
            key[h, i] = _round_f32(a - b)
            a2 = Fraction(_round_f32(x1 * c))
            b2 = Fraction(_round_f32(x0 * s))
            key[h, i + h2] = _round_f32(a2 + b2)
    return key


def brute_force_attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                          position: int, theta: float, dps: int = 50):
    """mpmath attention of one request over stored float64 K/V values.

    ``q [Hq, D]`` un-rotated; ``k_all``/``v_all [Hkv, L, D]``.  The query is
    rotated with mpmath cos/sin; exp and sums are 50-digit.
    """
    import mpmath

    mpmath.mp.dps = dps
    hq, d = q.shape
    hkv, length, _ = k_all.shape
    g = hq // hkv
    h2 = d // 2
    out = [[None] * d for _ in range(hq)]
    for hh in range(hq):
        kv = hh // g
        qr = [None] * d
        for i in range(h2):
            ang = mpmath.mpf(position) * mpmath.power(mpmath.mpf(theta),
                                                      mpmath.mpf(-2 * i) / d)
            c, s = mpmath.cos(ang), mpmath.sin(ang)
            x0, x1 = mpmath.mpf(float(q[hh, i])), mpmath.mpf(float(q[hh, i + h2]))
            qr[i] = x0 * c - x1 * s
            qr[i + h2] = x1 * c + x0 * s
        scores = []
        for t in range(length):
            acc = mpmath.mpf(0)
            for j in range(d):
                acc += qr[j] * mpmath.mpf(float(k_all[kv, t, j]))
            scores.append(acc / mpmath.sqrt(d))
        m = max(scores)
        w = [mpmath.exp(sc - m) for sc in scores]
        tot = mpmath.fsum(w)
        for j in range(d):
            out[hh][j] = mpmath.fsum(w[t] * mpmath.mpf(float(v_all[kv, t, j]))
                                     for t in range(length)) / tot
    return out
