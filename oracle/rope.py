"""Rotary position embedding (RoPE).  Test infrastructure.

"Scaling TensorRT-LLM: Kernel Fusion and Inflight Batching in Production",
section "What Gets Fused", applies the rotary embedding inside the attention
kernel; "TensorRT-LLM Guide: High-Throughput GPU Inference Engine", section
"The Core Architectural Pillars of TensorRT-LLM", fuses the attention kernels
with positional encodings.  Neither page fixes the variant, so the reading
taken is the rotate-half form used by Llama-family models: for head dimension
``D`` and ``i < D/2`` the pair ``(x[i], x[i + D/2])`` is rotated by the angle
``p * theta**(-2i/D)`` where ``p`` is the token position; all ``D``
dimensions rotate, and there is no frequency scaling.

Tables.  ``cos`` and ``sin`` of each angle are evaluated in double precision
with the C library (Python's ``math.cos`` / ``math.sin`` / ``**``) and
rounded once to float32.

Append arithmetic.  The rotated key is stored in the cache, so its bits must
be reproducible.  The reading taken: every operation is one IEEE float32
operation rounded to nearest-even, in this order and with no fused
multiply-add::

    y[i]       = (x[i] * C[i])       - (x[i + D/2] * S[i])
    y[i + D/2] = (x[i + D/2] * C[i]) + (x[i] * S[i])
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np


def inv_freq(theta: float, head_dim: int) -> list:
    """``theta ** (-(2 i) / D)`` for ``i < D/2`` in double precision."""
    return [float(theta) ** (-(2 * i) / head_dim) for i in range(head_dim // 2)]


def rope_rows_f32(theta: float, head_dim: int, positions: Sequence[int]):
    """float32 cos/sin rows ``[len(positions), D/2]`` of the RoPE table."""
    f = inv_freq(theta, head_dim)
    n = len(positions)
    c = np.empty((n, head_dim // 2), dtype=np.float32)
    s = np.empty((n, head_dim // 2), dtype=np.float32)
    for r, p in enumerate(positions):
        for i, fi in enumerate(f):
            ang = float(p) * fi
            c[r, i] = np.float32(math.cos(ang))
            s[r, i] = np.float32(math.sin(ang))
    return c, s


def rope_f64(x: np.ndarray, position: int, theta: float) -> np.ndarray:
    """Rotate ``x[..., D]`` by ``position`` entirely in float64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    f = inv_freq(theta, d)
    ang = np.array([float(position) * fi for fi in f], dtype=np.float64)
    c = np.array([math.cos(a) for a in ang])
    s = np.array([math.sin(a) for a in ang])
    x0 = x[..., :h]
    x1 = x[..., h:]
    return np.concatenate([x0 * c - x1 * s, x1 * c + x0 * s], axis=-1)


def rope_k_f32(x: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray) -> np.ndarray:
    """Rotate float32 ``x[..., D]`` with the pinned float32 arithmetic.

    numpy float32 array operations are single IEEE operations (one rounding
    each, never fused), which is the arithmetic the stored key must follow.
    """
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    h = x.shape[-1] // 2
    x0 = x[..., :h]
    x1 = x[..., h:]
    y0 = np.subtract(np.multiply(x0, c, dtype=np.float32),
                     np.multiply(x1, s, dtype=np.float32), dtype=np.float32)
    y1 = np.add(np.multiply(x1, c, dtype=np.float32),
                np.multiply(x0, s, dtype=np.float32), dtype=np.float32)
    return np.concatenate([y0, y1], axis=-1).astype(np.float32)
