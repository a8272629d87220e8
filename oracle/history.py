"""Decode steps over dense per-sequence histories.  TEST INFRASTRUCTURE ONLY.

The observable contract of a paged cache under a block allocator: every
sequence attends over exactly its own tokens (a forked sequence over the
shared prefix and then its own), whatever blocks hold them.  Here each
sequence's cache is a plain contiguous array of its stored K/V codes; a step
appends the new token (RoPE of the key in the pinned fp32 arithmetic, cast
to the cache type) and attends over the whole history in float64, exactly as
``decode.decode_step`` does for one request after its gather.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .decode import (attention_request, cast_to_kv, fp8_inverse_scale, io_to_f32, io_to_f64,
                     kv_to_f64)
from .rope import rope_f64, rope_k_f32, rope_rows_f32


class DenseHistories:
    """Per-sequence contiguous K/V codes ``[Hkv, L, D]``."""

    def __init__(self, kv_dtype: str, io_dtype: str, rope_theta: float,
                 k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
        self.kv_dtype, self.io_dtype, self.theta = kv_dtype, io_dtype, rope_theta
        self.k_scale, self.v_scale = k_scale, v_scale
        self.k: Dict[int, np.ndarray] = {}
        self.v: Dict[int, np.ndarray] = {}

    def add(self, sid: int, k_codes: np.ndarray, v_codes: np.ndarray) -> None:
        self.k[sid] = np.array(k_codes, copy=True)
        self.v[sid] = np.array(v_codes, copy=True)

    def fork(self, parent: int, child: int) -> None:
        self.add(child, self.k[parent], self.v[parent])

    def release(self, sid: int) -> None:
        del self.k[sid], self.v[sid]

    def step(self, seq_ids, q, k_new, v_new, positions) -> np.ndarray:
        """Append row b of k_new/v_new to sequence seq_ids[b] and return the
        float64 attention output ``[B, Hq, D]``."""
        hkv = next(iter(self.k.values())).shape[0] if self.k else k_new.shape[1]
        if self.kv_dtype == "fp8":
            inv_k, inv_v = fp8_inverse_scale(self.k_scale), fp8_inverse_scale(self.v_scale)
        else:
            inv_k = inv_v = [None] * hkv
        out = np.empty(q.shape, dtype=np.float64)
        for b, sid in enumerate(seq_ids):
            d = q.shape[2]
            c_row, s_row = rope_rows_f32(self.theta, d, [int(positions[b])])
            k32 = io_to_f32(k_new[b], self.io_dtype)
            v32 = io_to_f32(v_new[b], self.io_dtype)
            kr = np.stack([cast_to_kv(rope_k_f32(k32[h], c_row[0], s_row[0]), self.kv_dtype,
                                      inv_k[h]) for h in range(hkv)])
            vr = np.stack([cast_to_kv(v32[h], self.kv_dtype, inv_v[h]) for h in range(hkv)])
            self.k[sid] = np.concatenate([self.k[sid], kr[:, None, :]], axis=1)
            self.v[sid] = np.concatenate([self.v[sid], vr[:, None, :]], axis=1)
            kf = kv_to_f64(self.k[sid], self.kv_dtype, self.k_scale)
            vf = kv_to_f64(self.v[sid], self.kv_dtype, self.v_scale)
            q_rot = rope_f64(io_to_f64(q[b], self.io_dtype), int(positions[b]), self.theta)
            out[b] = attention_request(q_rot, kf, vf)
        return out
