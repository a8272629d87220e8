"""Reference decode step: append, gather, RoPE, attention.  Test infrastructure.

Cache representation used here: the *logical* layout ``[num_blocks, Hkv,
block_size, D]`` of storage codes -- float32 values for an fp32 cache,
``uint16`` bfloat16 bit patterns for a bf16 cache, ``uint8`` E4M3FN codes for
an fp8 cache.  Inputs ``q [B, Hq, D]``, ``k_new``/``v_new [B, Hkv, D]`` are
float32 arrays for fp32 I/O or ``uint16`` bfloat16 bits for bf16 I/O.

Readings of the pages taken here (the pages never spell the step out):

* ``context_lens[b]`` counts the new token; the new token's K/V go to slot
  ``L_b - 1`` and attention runs over all ``L_b`` tokens, the new one
  included, with no causal mask (the single query is the newest token);
* the scale is ``1 / sqrt(D)``; there is no output projection (the step ends
  at the attention output);
* query head ``hq`` reads KV head ``hq // G`` with ``G = Hq / Hkv`` (KV heads
  shared by groups of query heads, "TensorRT-LLM Guide: High-Throughput GPU
  Inference Engine", section "3. Custom Fused Attention Kernels: FMHA and
  XQA");
* cached keys are stored already rotated; only the new key is rotated, and
  values are never rotated;
* FP8 scales are per KV head with ``real = code * scale`` (precomputed,
  "delayed" scale factors, same page, section "4. Native FP8 Quantization on
  NVIDIA Hopper & Blackwell"); the new token is encoded as
  ``E4M3(y * f32(1 / scale))`` with the reciprocal taken in float32;
* the block holding slot ``L - 1`` is found through the request's block
  table like every other slot ("Scaling TensorRT-LLM: Kernel Fusion and
  Inflight Batching in Production", section "The Paged KV-Cache: vLLM
  Borrowed by TensorRT-LLM").
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .codecs import (bf16_bits_from_f32, bf16_bits_to_f32, fp8_decode,
                     fp8_encode)
from .rope import rope_f64, rope_k_f32, rope_rows_f32


def io_to_f32(x: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if io_dtype == "bf16":
        return bf16_bits_to_f32(x)
    raise ValueError(io_dtype)


def io_to_f64(x: np.ndarray, io_dtype: str) -> np.ndarray:
    return io_to_f32(x, io_dtype).astype(np.float64)


def kv_to_f64(codes: np.ndarray, kv_dtype: str,
              scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Dequantise cache codes ``[..., Hkv, T, D]`` to float64 (exact).

    For fp8 the per-head scale multiplies along the KV-head axis (third from
    last); ``code_value * scale`` is exact in float64.
    """
    if kv_dtype == "f32":
        return np.asarray(codes, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return bf16_bits_to_f32(codes).astype(np.float64)
    if kv_dtype == "fp8":
        v = fp8_decode(codes)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        return v * s.reshape(-1, 1, 1)
    raise ValueError(kv_dtype)


def fp8_inverse_scale(scale: np.ndarray) -> np.ndarray:
    """``f32(1 / scale)`` computed as a float32 division."""
    s = np.asarray(scale, dtype=np.float32)
    return np.divide(np.float32(1.0), s, dtype=np.float32)


def cast_to_kv(y32: np.ndarray, kv_dtype: str,
               inv_scale: Optional[np.float32] = None) -> np.ndarray:
    """Encode float32 values into cache storage codes."""
    y32 = np.asarray(y32, dtype=np.float32)
    if kv_dtype == "f32":
        return y32.copy()
    if kv_dtype == "bf16":
        return bf16_bits_from_f32(y32)
    if kv_dtype == "fp8":
        return fp8_encode(np.multiply(y32, np.float32(inv_scale),
                                      dtype=np.float32))
    raise ValueError(kv_dtype)


def gather_request(pool: np.ndarray, table_row: np.ndarray, length: int,
                   block_size: int) -> np.ndarray:
    """Contiguous ``[Hkv, L, D]`` codes of one request, block by block."""
    n_blocks = (length + block_size - 1) // block_size
    parts = []
    for j in range(n_blocks):
        phys = int(table_row[j])
        take = min(block_size, length - j * block_size)
        parts.append(pool[phys, :, :take, :])
    return np.concatenate(parts, axis=1)


def attention_request(q_rot: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """``softmax(q K^T / sqrt(D)) V`` in float64 for one request.

    ``q_rot [Hq, D]``, ``k``/``v [Hkv, L, D]``; query head ``hq`` reads KV
    head ``hq // G``.  The max is subtracted before ``exp`` (exact shift of
    the softmax), which keeps every term finite.
    """
    hq, d = q_rot.shape
    hkv = k.shape[0]
    g = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hkv):
        qg = q_rot[h * g:(h + 1) * g]                     # [G, D]
        s = (qg @ k[h].T) / math.sqrt(d)                  # [G, L]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        out[h * g:(h + 1) * g] = (w @ v[h]) / w.sum(axis=1, keepdims=True)
    return out


def decode_step(*, k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: str,
                io_dtype: str, q: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, positions: np.ndarray,
                block_tables: np.ndarray, context_lens: np.ndarray,
                block_size: int, rope_theta: float,
                k_scale: Optional[np.ndarray] = None,
                v_scale: Optional[np.ndarray] = None, window: int = 0) -> dict:
    """One decode step for a ragged batch, entirely on the CPU.

    ``window`` >= 1 is sliding-window attention, which the "TensorRT-LLM"
    glossary entry (inferensys.com) names among the patterns its kernels
    exploit without defining it; the reading taken is the plainest one: the
    new token attends to the last ``window`` tokens of the request, itself
    included, i.e. tokens ``[max(0, L - window), L)``.  0 attends to all.

    Returns a dict with ``out`` (float64 ``[B, Hq, D]``), the updated pools
    ``k_pool``/``v_pool`` (copies; only slot ``L_b - 1`` of each request
    changes) and the appended codes ``k_app``/``v_app`` (``[B, Hkv, D]``).
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    bsz = int(np.asarray(context_lens).shape[0])
    hkv, d = kp.shape[1], kp.shape[3]
    hq = q.shape[1] if bsz else 0
    if kv_dtype == "fp8":
        inv_k = fp8_inverse_scale(k_scale)
        inv_v = fp8_inverse_scale(v_scale)
    else:
        inv_k = inv_v = [None] * hkv
    out = np.empty((bsz, hq, d), dtype=np.float64)
    k_app = np.empty((bsz, hkv, d), dtype=kp.dtype)
    v_app = np.empty((bsz, hkv, d), dtype=vp.dtype)

    # Append first: the attention reads the new token as stored.
    for b in range(bsz):
        length = int(context_lens[b])
        pos = int(positions[b])
        slot = length - 1
        phys = int(block_tables[b, slot // block_size])
        off = slot % block_size
        c_row, s_row = rope_rows_f32(rope_theta, d, [pos])
        k32 = io_to_f32(k_new[b], io_dtype)
        v32 = io_to_f32(v_new[b], io_dtype)
        for h in range(hkv):
            y = rope_k_f32(k32[h], c_row[0], s_row[0])
            k_app[b, h] = cast_to_kv(y, kv_dtype, inv_k[h])
            v_app[b, h] = cast_to_kv(v32[h], kv_dtype, inv_v[h])
            kp[phys, h, off, :] = k_app[b, h]
            vp[phys, h, off, :] = v_app[b, h]

    for b in range(bsz):
        length = int(context_lens[b])
        lo = max(0, length - window) if window > 0 else 0
        kc = gather_request(kp, block_tables[b], length, block_size)[:, lo:]
        vc = gather_request(vp, block_tables[b], length, block_size)[:, lo:]
        kf = kv_to_f64(kc, kv_dtype, k_scale)
        vf = kv_to_f64(vc, kv_dtype, v_scale)
        q_rot = rope_f64(io_to_f64(q[b], io_dtype), int(positions[b]),
                         rope_theta)
        out[b] = attention_request(q_rot, kf, vf)
    return {"out": out, "k_pool": kp, "v_pool": vp, "k_app": k_app,
            "v_app": v_app}


def decode_step_multi(*, k_pool: np.ndarray, v_pool: np.ndarray, kv_dtype: str,
                      io_dtype: str, q: np.ndarray, k_new: np.ndarray,
                      v_new: np.ndarray, positions: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray,
                      block_size: int, rope_theta: float,
                      k_scale: Optional[np.ndarray] = None,
                      v_scale: Optional[np.ndarray] = None) -> dict:
    """A step that brings T new tokens per request (speculative verification of
    draft tokens, or the tail of a chunked prefill; the pages name both
    without writing the attention out).  Reading taken: ``q [B, T, Hq, D]``,
    ``k_new``/``v_new [B, T, Hkv, D]``; ``context_lens`` counts all T new
    tokens, new token i goes to slot ``L - T + i`` at RoPE position
    ``positions[b] + i``, and its query attends causally to the tokens
    ``[0, L - T + i]``, i.e. to the cache and to the new tokens up to itself.
    All T appends happen before any attention.  Returns ``out [B, T, Hq, D]``
    (float64) and the updated pools.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    bsz, tq = q.shape[0], q.shape[1]
    hkv, d = kp.shape[1], kp.shape[3]
    hq = q.shape[2]
    if kv_dtype == "fp8":
        inv_k = fp8_inverse_scale(k_scale)
        inv_v = fp8_inverse_scale(v_scale)
    else:
        inv_k = inv_v = [None] * hkv
    out = np.empty((bsz, tq, hq, d), dtype=np.float64)
    for b in range(bsz):
        length = int(context_lens[b])
        for i in range(tq):
            slot = length - tq + i
            pos = int(positions[b]) + i
            phys = int(block_tables[b, slot // block_size])
            off = slot % block_size
            c_row, s_row = rope_rows_f32(rope_theta, d, [pos])
            k32 = io_to_f32(k_new[b, i], io_dtype)
            v32 = io_to_f32(v_new[b, i], io_dtype)
            for h in range(hkv):
                kp[phys, h, off, :] = cast_to_kv(rope_k_f32(k32[h], c_row[0], s_row[0]),
                                                 kv_dtype, inv_k[h])
                vp[phys, h, off, :] = cast_to_kv(v32[h], kv_dtype, inv_v[h])
    for b in range(bsz):
        length = int(context_lens[b])
        kf = kv_to_f64(gather_request(kp, block_tables[b], length, block_size), kv_dtype, k_scale)
        vf = kv_to_f64(gather_request(vp, block_tables[b], length, block_size), kv_dtype, v_scale)
        for i in range(tq):
            seen = length - tq + i + 1
            q_rot = rope_f64(io_to_f64(q[b, i], io_dtype), int(positions[b]) + i, rope_theta)
            out[b, i] = attention_request(q_rot, kf[:, :seen], vf[:, :seen])
    return {"out": out, "k_pool": kp, "v_pool": vp}
